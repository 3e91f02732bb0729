// ge_skinny.hip -- small-M (decode) kernels: the weights are streamed from
// memory once, straight into MFMA fragments, and the epilogue runs after an
// in-LDS reduction over the workgroup's K split.
//
// Shape of the work: M <= 32 rows of activations X (tiny, re-read from L2),
// weights W with K x N entries (the whole cost: the kernel is bound by HBM).
// One workgroup (8 waves) owns a block of output columns and the full K; its
// waves split K, so every weight byte is read once and there is no
// cross-workgroup reduction.
//
// bf16 weights, KN layout ([K, N], N contiguous):
//   a lane loads 8 rows x 16 bytes (8 columns) of one 32-deep K block and
//   transposes them in registers into 8 B fragments (8 k values of one
//   column each); MFMA tile t then covers the columns 8 c + t of the lanes'
//   16 column chunks c, i.e. a wave covers 128 consecutive columns.
//
// int4 weights, prepacked (see gemm_w4_prepack): for each 16-column tile and
// each 128-row K group, lane l's 16 bytes are its four B fragments (one per
// 32-deep block), 8 codes per dword.  A code c becomes the bf16 value 128 + c
// by OR-ing it into the mantissa of 0x4300; a second MFMA against a constant
// -(128 + z) fragment folds in -(128 + z) * sum(x), so the product is
// sum x * (c - z) for zero point z (8 on the pages),
// exact in fp32 before the per-group scale (page "Fusion Thinking",
// Pattern 3: zero point 8, per-group scales, dequantisation in registers).

#include "ge_launch.hpp"

namespace ge {
namespace {

constexpr int S_WAVES = 8;
constexpr int SK_RING = 4;  // bf16 streaming: blocks in flight per wave
constexpr int S_THREADS = 64 * S_WAVES;
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint32_t n = bytes > 0 ? (bytes >= (1ll << 31) ? 0x7fffffffu : (uint32_t)bytes) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// Cache policy operand of a buffer access: non-temporal.  Weights that a call streams once are read
// with it, so that they do not displace from the caches the activations that every workgroup
// re-reads (16x28672x8192 bf16 decode: 79.9 -> 70.1 us per call; 16x8192x8192 8-bit: 18.4-18.9 ->
// 17.5-18.2 us).  The int4 codes of the K-split kernel measured 1.5% slower with it and keep the
// default policy.
constexpr int NT = 2;
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, NT));
}

// even / odd bf16 halves of two dwords (x supplies the low half)
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return (x & 0xffffu) | (y << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return (x >> 16) | (y & 0xffff0000u); }

// ---------------------------------------------------------------------------
// shared tail: reduce the waves' partial tiles in LDS, then the epilogue on
// 8-column row chunks (16-byte accesses where aligned)
// ---------------------------------------------------------------------------

// 16-byte epilogue accesses are possible (bf16 tensors, 16-byte aligned rows)
__device__ __forceinline__ bool epi_vec_ok(const Problem &p) {
    const EpiArgs &e = p.epi;
    return ((p.N & 7) == 0) && (((uintptr_t)e.D & 15) == 0) && ((e.ldd & 7) == 0) &&
           (!(e.flags & GE_FLAG_RESIDUAL) || ((((uintptr_t)e.R & 15) == 0) && ((e.ldr & 7) == 0))) &&
           (!(e.flags & GE_FLAG_C) || ((((uintptr_t)e.C & 15) == 0) && ((e.ldc & 7) == 0))) &&
           (!(e.flags & GE_FLAG_BIAS) || (((uintptr_t)e.bias & 15) == 0)) && e.d_type == GE_BF16 &&
           (!(e.flags & GE_FLAG_RESIDUAL) || e.r_type == GE_BF16) && (!(e.flags & GE_FLAG_C) || e.c_type == GE_BF16) &&
           (!(e.flags & GE_FLAG_BIAS) || e.bias_type == GE_BF16);
}

// epilogue of the 8 accumulators of row m, columns n .. n + 7 (clipped at N)
template <int ACT>
__device__ __forceinline__ void finish_chunk(const Problem &p, bool vec_ok, int m, int n, const float v[8]) {
    const EpiArgs &e = p.epi;
    if (vec_ok && n + 8 <= p.N) {
        epi_row8<ACT>(e, v, m, n);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (n + q < p.N) store_elem(e.D, e.d_type, (int64_t)m * e.ldd + n + q, epi_scalar<ACT>(e, v[q], m, n + q));
    }
}

// red: [NWV][MR][NC] fp32 partials in LDS (MR rows, NC columns), NWV waves
template <int MR, int NC, int NWV = S_WAVES>
__device__ __forceinline__ void reduce_epilogue(const Problem &p, const float *red, int n0) {
    constexpr int CH = NC / 8;  // 8-column chunks per row
    const bool vec_ok = epi_vec_ok(p);
    with_act(p.epi.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
        for (int item = threadIdx.x; item < MR * CH; item += 64 * NWV) {
            const int r = item / CH, c = item % CH;
            const int m = r, n = n0 + c * 8;
            if (m >= p.M || n >= p.N) continue;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = 0.0f;
#pragma unroll
            for (int w = 0; w < NWV; ++w) {
                const f32x4 a = *(const f32x4 *)&red[(w * MR + r) * NC + c * 8];
                const f32x4 b = *(const f32x4 *)&red[(w * MR + r) * NC + c * 8 + 4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] += a[q];
                    v[4 + q] += b[q];
                }
            }
            finish_chunk<ACT>(p, vec_ok, m, n, v);
        }
    });
}

// ---------------------------------------------------------------------------
// bf16 weights
// ---------------------------------------------------------------------------

// MT: 16-row tiles of X (M <= 16 MT).  WG: NCH 8-column chunks (NCH <= 16,
// one per lane of a 16-lane row; the remaining lanes idle), 8 waves splitting
// K.  NCH is chosen per shape so that the workgroups fill the CUs evenly.
// One wave's share of a column block: 32-deep blocks [kb0, kb1) of the NC = 8 NCH columns
// from n0, accumulated into acc (lane (g, i) holds rows mt*16 + 4 g + e, columns 8 i + t).
template <int MT, int NCH>
__device__ __forceinline__ void stream_bf16(const Problem &p, int n0, int kb0, int kb1, f32x4 (&acc)[MT][8]) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i = lane & 15;
    const int nkb = (p.K + 31) / 32;

    // W: lane -> rows 8 g + r of the block, 16-byte column chunk i (columns n0 + 8 i ..).  The
    // range starts at the wave's first row and column n0, so only the wave's share of W has to
    // span less than 2^31 bytes (an empty share gets an empty range).
    const bool nin = i < NCH && n0 + 8 * i < p.N;
    const int r0 = kb0 * 32, r1 = min(p.K, kb1 * 32);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc((const uint16_t *)p.B + ((int64_t)r0 * p.ldb + n0),
                                                ((int64_t)(r1 - r0 - 1) * p.ldb + (p.N - n0)) * 2);
    // X: lane -> row mt*16 + i, k = 8 g .. 8 g + 7 of the block
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);

    auto load_w = [&](int kb, u32x4 (&w)[8]) {
        const int k = kb * 32 + 8 * g;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t off = (uint32_t)(((int64_t)(k + r - r0) * p.ldb + 8 * i) * 2);
            w[r] = bload16_nt(rw, (nin && k + r < r1) ? off : OOB);  // a wave reads rows >= r0 only
        }
    };
    auto load_x = [&](int kb, bf16x8 (&x)[MT]) {
        const int k = kb * 32 + 8 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + i;
            const uint32_t off = (uint32_t)(((int64_t)m * p.lda + k) * 2);
            x[mt] = __builtin_bit_cast(bf16x8, bload16(rx, (m < p.M && k < p.K) ? off : OOB));
        }
    };

    // ring of SK_RING blocks: weights and activations of block kb + SK_RING - 1 are requested
    // together while block kb is multiplied (loaded as a pair, so waiting for one block's
    // activations never waits for a later block's weights); blocks past the wave's share read
    // zeros and add nothing
    u32x4 w[SK_RING][8];
    bf16x8 xr[SK_RING][MT];
    auto load_blk = [&](int kb, int slot) {
        const bool in = kb < kb1;
        load_w(in ? kb : nkb + 1, w[slot]);
        load_x(in ? kb : nkb + 1, xr[slot]);
    };
#pragma unroll
    for (int j = 0; j < SK_RING - 1; ++j) load_blk(kb0 + j, j);
    for (int kb = kb0; kb < kb1; kb += SK_RING) {
#pragma unroll
        for (int u = 0; u < SK_RING; ++u) {
            load_blk(kb + u + SK_RING - 1, (u + SK_RING - 1) % SK_RING);
            const u32x4 (&wc)[8] = w[u];
            // 8 rows x 8 columns -> 8 fragments (k-vectors of one column each)
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
                u32x4 lo, hi;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    lo[q] = pack_lo(wc[2 * q][dw], wc[2 * q + 1][dw]);
                    hi[q] = pack_hi(wc[2 * q][dw], wc[2 * q + 1][dw]);
                }
                const bf16x8 f0 = __builtin_bit_cast(bf16x8, lo), f1 = __builtin_bit_cast(bf16x8, hi);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][2 * dw] = mfma_bf16(xr[u][mt], f0, acc[mt][2 * dw]);
                    acc[mt][2 * dw + 1] = mfma_bf16(xr[u][mt], f1, acc[mt][2 * dw + 1]);
                }
            }
        }
    }
}

// partial tile of one wave -> LDS red[wave][MR][NC]
template <int MT, int NCH>
__device__ __forceinline__ void acc_to_lds(float *red, const f32x4 (&acc)[MT][8]) {
    constexpr int NC = 8 * NCH, MR = 16 * MT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    if (i < NCH) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                float *dst = &red[(wave * MR + mt * 16 + 4 * g + e4) * NC + 8 * i];
                *(f32x4 *)dst = f32x4{acc[mt][0][e4], acc[mt][1][e4], acc[mt][2][e4], acc[mt][3][e4]};
                *(f32x4 *)(dst + 4) = f32x4{acc[mt][4][e4], acc[mt][5][e4], acc[mt][6][e4], acc[mt][7][e4]};
            }
    }
}

template <int MT, int NCH>
__global__ __launch_bounds__(S_THREADS) void skinny_bf16_kernel(Problem p) {
    constexpr int NC = 8 * NCH;
    constexpr int MR = 16 * MT;
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * NC;
    const int nkb = (p.K + 31) / 32;
    const int per = (nkb + S_WAVES - 1) / S_WAVES;
    const int kb0 = wave * per, kb1 = min(nkb, kb0 + per);

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_bf16<MT, NCH>(p, n0, kb0, kb1, acc);
    acc_to_lds<MT, NCH>(red, acc);
    __syncthreads();
    reduce_epilogue<MR, NC>(p, red, n0);
}

// ---------------------------------------------------------------------------
// bf16 weights, prepacked (gemm_b_prepack), M <= 16
// ---------------------------------------------------------------------------
// Layout: per 128-column block and 32-deep K block, 8 KB: the B fragments of
// the block's eight 16-column MFMA tiles, 1 KB each, lane l's 16 bytes
// (column 16 t + l % 16, k = 8 (l / 16) .. + 7) at byte 16 l.  K blocks follow
// each other, so a wave's share of a column block is one contiguous run, read
// with 16-byte loads that are already MFMA fragments.  (The raw [K, N] layout
// gives each wave 256-byte row pieces 2 N bytes apart, and a transpose.)
// One workgroup per column block, 8 waves splitting K, a ring of SK_RING
// blocks in flight per wave; the K partials are reduced in LDS and the shared
// epilogue runs on 8-column row chunks.
// Blocks kbA .. kbB - 1 of column block cb: wave w takes kbA + w, kbA + w + 8, ..., so at any time
// the workgroup reads 8 consecutive 8 KB pieces (64 KB of contiguous memory); a ring of SK_RING
// blocks in flight per wave, blocks past kbB read zeros and add nothing.  acc[mt][t]: lane (g, i)
// holds rows 16 mt + 4 g + e of column 16 t + i (MT 16-row tiles of X share each weight fragment).
template <int MT, int TB = 8>
__device__ __forceinline__ void stream_bf16p(const Problem &p, int cb, int kbA, int kbB, f32x4 (&acc)[MT][TB]) {
    constexpr int PIECE = TB * 1024;  // bytes of one 32-row piece of a block
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int nkb = p.K / 32;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc((const char *)p.B + (int64_t)cb * nkb * PIECE, (int64_t)nkb * PIECE);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);
    u32x4 w[SK_RING][TB];
    bf16x8 xr[SK_RING][MT];
    auto load_blk = [&](int kb, int slot) {
        const bool in = kb < kbB;
#pragma unroll
        for (int t = 0; t < TB; ++t) w[slot][t] = bload16_nt(rw, in ? (uint32_t)(kb * PIECE + t * 1024 + lane * 16) : OOB);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + i;
            const uint32_t xoff = (uint32_t)(((int64_t)m * p.lda + 8 * g) * 2);
            xr[slot][mt] = __builtin_bit_cast(bf16x8, bload16(rx, in && m < p.M ? xoff + (uint32_t)kb * 64 : OOB));
        }
    };
#pragma unroll
    for (int j = 0; j < SK_RING - 1; ++j) load_blk(kbA + wave + S_WAVES * j, j);
    for (int kb = kbA + wave; kb < kbB; kb += S_WAVES * SK_RING) {
#pragma unroll
        for (int u = 0; u < SK_RING; ++u) {
            load_blk(kb + S_WAVES * (u + SK_RING - 1), (u + SK_RING - 1) % SK_RING);
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][t] = mfma_bf16(xr[u][mt], __builtin_bit_cast(bf16x8, w[u][t]), acc[mt][t]);
        }
    }
}

// partial tile of one wave (prepacked lane mapping) -> LDS red[wave][16 MT][16 TB]
template <int MT, int TB = 8>
__device__ __forceinline__ void accp_to_lds(float *red, const f32x4 (&acc)[MT][TB]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                red[(wave * 16 * MT + 16 * mt + 4 * g + e4) * (16 * TB) + 16 * t + i] = acc[mt][t][e4];
}

// one workgroup per column block of TB 16-column tiles (128 or 112 columns)
template <int MT, int TB>
__global__ __launch_bounds__(S_THREADS) void skinny_bf16p_kernel(Problem p) {
    constexpr int NC = 16 * TB, MR = 16 * MT;
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];
    f32x4 acc[MT][TB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_bf16p<MT, TB>(p, blockIdx.x, 0, p.K / 32, acc);
    accp_to_lds<MT, TB>(red, acc);
    __syncthreads();
    reduce_epilogue<MR, NC>(p, red, blockIdx.x * NC);
}

// raw [K, N] bf16 (row stride ldb) -> the prepacked layout of TB-tile blocks; item u writes the 16
// bytes of lane u % 64 of tile (u / 64) % TB of piece u / (64 TB) = cb * (K / 32) + kb, i.e. bytes
// 16 u .. 16 u + 15
template <int TB>
__global__ __launch_bounds__(256) void b_prepack_kernel(int32_t K, int32_t N, const uint16_t *B, int64_t ldb,
                                                        uint16_t *Bp) {
    const int64_t nkb = K / 32, total = (int64_t)(N / (16 * TB)) * nkb * 64 * TB;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(u & 63), t = (int)((u >> 6) % TB);
        const int64_t piece = (u >> 6) / TB, kb = piece % nkb, cb = piece / nkb;
        const int64_t n = cb * 16 * TB + t * 16 + (l & 15), k = kb * 32 + 8 * (l >> 4);
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            out[q] = (uint32_t)B[(k + 2 * q) * ldb + n] | ((uint32_t)B[(k + 2 * q + 1) * ldb + n] << 16);
        *(u32x4 *)(Bp + u * 8) = out;
    }
}

// Stream-K decode (bf16 weights, M <= 16, 128-column blocks): the (column block, 32-row
// block) units are dealt to the G workgroups in equal contiguous ranges, so every CU streams
// the same number of weight bytes even when the column blocks do not divide among the CUs
// (16 x 28672: 224 blocks on 256 CUs).  A range covers whole column blocks or parts of at
// most a few; a workgroup that holds only part of a block writes its partial tile to slot
// (its index - the index of the block's first workgroup) of the block, counts its 32-row
// blocks in, and the one that completes the count sums the slots in order and runs the
// epilogue.  The handoff is the one of the 8-bit split (device-scope accesses, no fences).
__device__ __forceinline__ int sk_owner(int64_t unit, int64_t U, int G) {
    int w = (int)(unit * G / U);
    while (w + 1 < G && U * (w + 1) / G <= unit) ++w;
    while (w > 0 && U * w / G > unit) --w;
    return w;
}

template <bool PACKED>
__global__ __launch_bounds__(S_THREADS) void skinny_bf16_sk_kernel(Problem p) {
    constexpr int MT = 1, NCH = 16, NC = 128, MR = 16, CH = NC / 8, MAXS = 8;
    constexpr int SC1 = 16;  // cache policy operand: device scope
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];
    __shared__ int s_last;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = (int)gridDim.x, wg = (int)blockIdx.x;
    const int ncb = (p.N + NC - 1) / NC, nkb = (p.K + 31) / 32;
    const int64_t U = (int64_t)ncb * nkb;
    const int64_t u1 = U * (wg + 1) / G;
    const int slots = p.split;  // tile slots per column block (plan scratch)
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(p.split_ws, (int64_t)ncb * slots * MR * NC * 4);

    for (int64_t u = U * wg / G; u < u1;) {
        const int cb = (int)(u / nkb), kbA = (int)(u % nkb);
        const int kbB = (int)((u1 - u) < (int64_t)(nkb - kbA) ? kbA + (u1 - u) : nkb);
        const int n0 = cb * NC;
        const int per = (kbB - kbA + S_WAVES - 1) / S_WAVES;
        const int k0 = min(kbB, kbA + wave * per), k1 = min(kbB, k0 + per);
        f32x4 acc[MT][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (PACKED) {
            stream_bf16p<MT>(p, cb, kbA, kbB, acc);
            accp_to_lds<MT>(red, acc);
        } else {
            stream_bf16<MT, NCH>(p, n0, k0, k1, acc);
            acc_to_lds<MT, NCH>(red, acc);
        }
        __syncthreads();
        if (kbA == 0 && kbB == nkb) {
            reduce_epilogue<MR, NC>(p, red, n0);
        } else {
            const int first = sk_owner((int64_t)cb * nkb, U, G);
            const int nsl = sk_owner((int64_t)cb * nkb + nkb - 1, U, G) - first + 1;
            const uint32_t mine = (uint32_t)(((int64_t)cb * slots + (wg - first)) * (MR * NC) * 4);
            // this workgroup's partial tile: sum of its waves, 16-byte device-scope stores
            for (int item = threadIdx.x; item < MR * CH; item += S_THREADS) {
                const int r = item / CH, c = item % CH;
                f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < S_WAVES; ++w) {
                    a += *(const f32x4 *)&red[(w * MR + r) * NC + c * 8];
                    b += *(const f32x4 *)&red[(w * MR + r) * NC + c * 8 + 4];
                }
                const uint32_t off = mine + (uint32_t)(r * NC + c * 8) * 4;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), rt, off, 0, SC1);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), rt, off + 16, 0, SC1);
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's tile stores are complete
            GE_DEBUG_FENCE();
            __syncthreads();
            if (threadIdx.x == 0) {
                const uint32_t add = (uint32_t)(kbB - kbA);
                const uint32_t prev = __hip_atomic_fetch_add(p.split_cnt + cb, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_last = prev + add == (uint32_t)nkb;
            }
            __syncthreads();
            if (s_last) {
                GE_DEBUG_FENCE();
                const bool vec_ok = epi_vec_ok(p);
                with_act(p.epi.act, [&](auto ACTC) {
                    constexpr int ACT = decltype(ACTC)::value;
                    for (int item = threadIdx.x; item < MR * CH; item += S_THREADS) {
                        const int r = item / CH, c = item % CH;
                        const int m = r, n = n0 + c * 8;
                        if (m >= p.M || n >= p.N) continue;
                        // every slot requested at once (slots past nsl read zeros), summed in slot order
                        f32x4 tl[MAXS][2];
#pragma unroll
                        for (int q = 0; q < MAXS; ++q) {
                            const uint32_t off =
                                q < nsl ? (uint32_t)((((int64_t)cb * slots + q) * (MR * NC) + r * NC + c * 8) * 4) : OOB;
                            tl[q][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, SC1));
                            tl[q][1] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, q < nsl ? off + 16 : OOB, 0, SC1));
                        }
                        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int q = 0; q < MAXS; ++q)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                v[e] += tl[q][0][e];
                                v[4 + e] += tl[q][1][e];
                            }
                        finish_chunk<ACT>(p, vec_ok, m, n, v);
                    }
                });
                if (threadIdx.x == 0)
                    __hip_atomic_store(p.split_cnt + cb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();  // red and s_last are reused by the next range segment
        u += kbB - kbA;
    }
}

// ---------------------------------------------------------------------------
// int4 weights, prepacked
// ---------------------------------------------------------------------------

// Four bf16 pairs (a B fragment, k in order) from one packed dword of 8 codes:
// pair q = (code at nibble q, code at nibble q + 4), each as bf16 128 + code.
// (w >> 4q) & 0x000f000f | 0x43004300 is one v_and_or_b32 per pair when the
// mask sits in a scalar register and the magic in a vector one (that encoding
// takes no literal operand; with both as literals the compiler spends an AND
// and an OR): 7 instructions per 8 codes.  The two constants are hidden from
// constant folding by empty asm statements; the arithmetic itself stays
// ordinary code, so the compiler's hazard handling around the MFMAs that read
// the result still applies.
struct W4Unpack {
    uint32_t mask, magic;
    __device__ __forceinline__ W4Unpack() {
        mask = 0x000f000fu;
        magic = 0x43004300u;
        asm volatile("" : "+s"(mask));
        asm volatile("" : "+v"(magic));
    }
    __device__ __forceinline__ uint32_t pair(uint32_t src) const { return (src & mask) | magic; }
    __device__ __forceinline__ bf16x8 operator()(uint32_t w) const {
        const u32x4 f = {pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12)};
        return __builtin_bit_cast(bf16x8, f);
    }
};

// NTW 16-column tiles per workgroup; W4_WAVES waves split the 128-row packing
// groups.  SPG: 32-deep blocks per scale group (group size / 32 = 1, 2 or 4).
// A wave takes its groups in rounds of RND: X, weights and scales of a whole
// round are requested at once, in group order, so the wave computes group j
// as soon as its bytes are in while the later groups are still arriving.  For
// K = 8192 a round is the wave's entire share and a workgroup has all of its
// weight bytes in flight at once.  Groups past the share read zeros.
// Per group the sum of x * (c - z) is x * (128 + c) (one MFMA per 32-deep
// block and tile) plus x * -(128 + z), which does not depend on the column and
// is computed once for all tiles.
#ifndef GE_W4_WAVES
#define GE_W4_WAVES 8
#endif
#ifndef GE_W4_RND
#define GE_W4_RND 4
#endif
constexpr int W4_WAVES = GE_W4_WAVES;
constexpr int W4_THREADS = 64 * W4_WAVES;

// MT 16-row tiles of X (M <= 16 MT) share each weight fragment; rounds shrink by MT so that the
// activations in flight take the same registers.
template <int NTW, int SPG, int MT>
__global__ __launch_bounds__(W4_THREADS) void skinny_w4_kernel(Problem p) {
    constexpr int NC = 16 * NTW;
    constexpr int MR = 16 * MT;
    constexpr int NSG = 4 / SPG;               // scale groups per 128-row packing group
    constexpr int RND0 = SPG == 1 ? (GE_W4_RND + 1) / 2 : GE_W4_RND;  // groups per round (32-row groups carry 4 scales each)
    constexpr int RND = RND0 / MT > 0 ? RND0 / MT : 1;
    __shared__ __attribute__((aligned(16))) float red[W4_WAVES * MR * NC];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int nt0 = blockIdx.x * NTW;  // first 16-column tile
    const int n0 = nt0 * 16;
    const int ntiles = p.N / 16;
    const int ngroups = p.K / 128;
    const int per = (ngroups + W4_WAVES - 1) / W4_WAVES;
    const int g0 = wave * per, g1 = min(ngroups, g0 + per);

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.B, (int64_t)p.K * p.N / 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scales, ((int64_t)(p.K / p.group - 1) * p.ld_s + p.N) * 2);

    // constant fragment -(128 + zero point) (exact in bf16) for the zero-point correction
    const uint32_t nz = f32_to_bf16(-(128.0f + (float)p.zero_point));
    const uint32_t nz2 = nz | (nz << 16);
    const bf16x8 negz = __builtin_bit_cast(bf16x8, u32x4{nz2, nz2, nz2, nz2});
    const W4Unpack unpack_w4;

    f32x4 tot[MT][NTW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) tot[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int base = g0; base < g1; base += RND) {
        bf16x8 x[RND][MT][4];
        u32x4 w[RND][NTW];
        uint16_t sraw[RND][NTW][NSG];
#pragma unroll
        for (int j = 0; j < RND; ++j) {
            const int gi = base + j;
            const bool gin = gi < g1;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int k = gi * 128 + kb * 32 + 8 * g, m = 16 * mt + i;
                    const uint32_t off = (uint32_t)(((int64_t)m * p.lda + k) * 2);
                    x[j][mt][kb] = __builtin_bit_cast(bf16x8, bload16(rx, (m < p.M && gin) ? off : OOB));
                }
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const bool tin = gin && nt0 + t < ntiles;
                w[j][t] = bload16(rw, tin ? (uint32_t)(w4p_frag_offset(nt0 + t, gi, ngroups, ntiles) + lane * 16) : OOB);
                const int n = n0 + 16 * t + i;
#pragma unroll
                for (int sg = 0; sg < NSG; ++sg)
                    sraw[j][t][sg] = __builtin_amdgcn_raw_buffer_load_b16(
                        rs, tin && n < p.N ? (int)(((int64_t)(gi * NSG + sg) * p.ld_s + n) * 2) : (int)OOB, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < RND; ++j) {
#pragma unroll
            for (int sg = 0; sg < NSG; ++sg) {
                f32x4 corr[MT], u[MT][NTW];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    corr[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < NTW; ++t) u[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int kb = sg * SPG; kb < (sg + 1) * SPG; ++kb) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) corr[mt] = mfma_bf16(x[j][mt][kb], negz, corr[mt]);
#pragma unroll
                    for (int t = 0; t < NTW; ++t) {
                        const bf16x8 wf = unpack_w4(w[j][t][kb]);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) u[mt][t] = mfma_bf16(x[j][mt][kb], wf, u[mt][t]);
                    }
                }
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    const float sv = bf16_to_f32(sraw[j][t][sg]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int q = 0; q < 4; ++q) tot[mt][t][q] = fmaf(sv, u[mt][t][q] + corr[mt][q], tot[mt][t][q]);
                }
            }
        }
    }

    // partial tile -> LDS: lane (g, i) holds rows 16 mt + 4 g + e, column 16 t + i
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) red[(wave * MR + 16 * mt + 4 * g + e4) * NC + 16 * t + i] = tot[mt][t][e4];
    __syncthreads();
    reduce_epilogue<MR, NC, W4_WAVES>(p, red, n0);
}

// ---------------------------------------------------------------------------
// 8-bit weights (u8 with a zero point, or OCP fp8 E4M3), raw [K, N] bytes
// ---------------------------------------------------------------------------

// Cross-workgroup K split.  The S workgroups of one column block each reduce
// their waves' partials, write the [MR, NC] fp32 tile to the plan's scratch
// ([S][column blocks][MR][NC]) and count themselves in; the last to arrive
// sums the S tiles in split order (so the result does not depend on arrival
// order), runs the epilogue and re-arms the counter for the next launch.
// Launches that share one scratch buffer must not overlap.
//
// Tiles are written and read with 16-byte buffer accesses carrying the
// device-scope cache policy (sc1: the access is coherent across the XCDs'
// L2 caches, as a device-scope atomic access is), and the counters with
// device-scope atomics, so no fence has to write back or invalidate whole L2
// caches (fences made the split slower than no split at all; 4-byte atomic
// stores of the tiles cost 8x their bytes in write traffic).  Ordering: every
// wave waits until its tile stores have completed before the barrier, the
// counter increment follows the barrier, and the last workgroup's tile loads
// are issued only after the increment has returned (barrier and LDS flag in
// between).
// SWI (NS = 2): the two tiles are the gate and the up product of one column block, combined as
// silu(gate) * up instead of summed
template <int MR, int NC, int NS, int NWV = S_WAVES, bool SWI = false>
__device__ __forceinline__ void split_reduce_epilogue(const Problem &p, const float *red, int n0, int cb, int ks,
                                                      int ncb, int *s_last) {
    static_assert(!SWI || NS == 2, "gate and up");
    constexpr int CH = NC / 8;
    constexpr int SC1 = 16;  // cache policy operand: device scope
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(p.split_ws, (int64_t)NS * ncb * MR * NC * 4);
    const uint32_t mine = (uint32_t)(((int64_t)ks * ncb + cb) * (MR * NC) * 4);
    for (int item = threadIdx.x; item < MR * CH; item += 64 * NWV) {
        const int r = item / CH, c = item % CH;
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            a += *(const f32x4 *)&red[(w * MR + r) * NC + c * 8];
            b += *(const f32x4 *)&red[(w * MR + r) * NC + c * 8 + 4];
        }
        const uint32_t off = mine + (uint32_t)(r * NC + c * 8) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), rt, off, 0, SC1);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), rt, off + 16, 0, SC1);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's tile stores are complete
    GE_DEBUG_FENCE();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(p.split_cnt + cb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = prev == (uint32_t)(NS - 1);
    }
    __syncthreads();
    if (!*s_last) return;
    GE_DEBUG_FENCE();
    const bool vec_ok = epi_vec_ok(p);
    with_act(p.epi.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
        for (int item = threadIdx.x; item < MR * CH; item += 64 * NWV) {
            const int r = item / CH, c = item % CH;
            const int m = r, n = n0 + c * 8;
            if (m >= p.M || n >= p.N) continue;
            // all NS tiles requested at once, then summed in split order
            f32x4 tl[NS][2];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const uint32_t off = (uint32_t)((((int64_t)q * ncb + cb) * (MR * NC) + r * NC + c * 8) * 4);
                tl[q][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, SC1));
                tl[q][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off + 16, 0, SC1));
            }
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr (SWI) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = activate<GE_ACT_SILU>(tl[0][0][e]) * tl[1][0][e];
                    v[4 + e] = activate<GE_ACT_SILU>(tl[0][1][e]) * tl[1][1][e];
                }
            } else {
#pragma unroll
                for (int q = 0; q < NS; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] += tl[q][0][e];
                        v[4 + e] += tl[q][1][e];
                    }
            }
            finish_chunk<ACT>(p, vec_ok, m, n, v);
        }
    });
    if (threadIdx.x == 0) __hip_atomic_store(p.split_cnt + cb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// SwiGLU on prepacked weights, M <= 32: workgroup 2 cb + h streams column block cb of W_gate
// (h = 0) or of W_up (h = 1, p.B2) through the prepacked decode loop; of the two, the one that
// arrives second combines silu(gate) * up into the block's output (page "Fusion Thinking",
// Pattern 2: the dual product's epilogue; here the two products of a block run on two CUs side by
// side, so that the 2 N / NC workgroups fill the GPU at decode sizes)
template <int MT, int TB>
__global__ __launch_bounds__(S_THREADS) void skinny_bf16p_swiglu_kernel(Problem p) {
    constexpr int NC = 16 * TB, MR = 16 * MT;
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];
    __shared__ int s_last;
    const int h = blockIdx.x & 1, cb = blockIdx.x >> 1, ncb = gridDim.x >> 1;
    Problem q = p;
    if (h) q.B = p.B2;
    f32x4 acc[MT][TB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_bf16p<MT, TB>(q, cb, 0, p.K / 32, acc);
    accp_to_lds<MT, TB>(red, acc);
    __syncthreads();
    split_reduce_epilogue<MR, NC, 2, S_WAVES, true>(p, red, cb * NC, cb, h, ncb, &s_last);
}

// The same pairs on raw [K, N] weights (row stride ldb): workgroup 2 cb + h streams the NC = 8 NCH
// columns from cb * NC of W_gate (h = 0) or W_up (h = 1) like the raw decode kernel
template <int MT, int NCH>
__global__ __launch_bounds__(S_THREADS) void skinny_bf16_swiglu_kernel(Problem p) {
    constexpr int NC = 8 * NCH, MR = 16 * MT;
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];
    __shared__ int s_last;
    const int h = blockIdx.x & 1, cb = blockIdx.x >> 1, ncb = gridDim.x >> 1;
    Problem q = p;
    if (h) q.B = p.B2;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkb = (p.K + 31) / 32;
    const int per = (nkb + S_WAVES - 1) / S_WAVES;
    const int kb0 = wave * per, kb1 = min(nkb, kb0 + per);
    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_bf16<MT, NCH>(q, cb * NC, kb0, kb1, acc);
    acc_to_lds<MT, NCH>(red, acc);
    __syncthreads();
    split_reduce_epilogue<MR, NC, 2, S_WAVES, true>(p, red, cb * NC, cb, h, ncb, &s_last);
}

#ifndef GE_W4S_RING
#define GE_W4S_RING 2
#endif
#ifndef GE_W4S_CODE_POLICY
#define GE_W4S_CODE_POLICY 0
#endif
constexpr int W4S_RING = GE_W4S_RING;
constexpr int W4S_CODE_POLICY = GE_W4S_CODE_POLICY;

// int4 weights (prepacked, 128-row groups), M <= 16, K split over workgroups.
// A workgroup owns one block of NTW prepacked 16-column tiles and 1/NS of K;
// its 8 waves split that range by whole groups, and a wave streams its groups
// through a ring of two: the codes (NTW x 16 bytes per lane), activations
// (4 x 16 bytes) and scales of the group after next are requested as soon as
// a group has been consumed.  With several groups per wave the requests of
// the whole GPU reach memory in group order, so the dequantisation of the
// first groups runs while later ones are still arriving instead of all of it
// after the last byte (at 16 x 8192 x 8192: 64-column blocks, NS = 2, four
// groups per wave).  Against 32-column workgroups over the whole of K, each
// activation byte read from L2 serves twice as many weight bytes.
// Per group and tile the sum of x * (c - z) is -(128 + z) * sum(x) (four MFMAs
// against a constant fragment, computed first) plus x * (128 + c) (four
// MFMAs accumulating onto it), times the tile's scales, into fp32 totals.
template <int NTW, int NS, int NWV>
__global__ __launch_bounds__(64 * NWV) void skinny_w4s_kernel(Problem p) {
    static_assert(W4P_BLOCK_TILES % NTW == 0, "a workgroup's tiles lie in one block of the prepacked layout");
    constexpr int NC = 16 * NTW, MR = 16;
    constexpr bool SPLIT = NS > 1;
    __shared__ __attribute__((aligned(16))) float red[NWV * MR * NC];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int ncb = (int)gridDim.x / NS;
    const int cb = (int)blockIdx.x % ncb;
    const int ks = (int)blockIdx.x / ncb;
    const int n0 = cb * NC, nt0 = cb * NTW;

    const int ngroups = p.K / 128;
    const int nvw = NS * NWV;
    const int per = (ngroups + nvw - 1) / nvw;
    const int g0 = (ks * NWV + wave) * per, g1 = min(ngroups, g0 + per);

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.B, (int64_t)p.K * p.N / 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scales, ((int64_t)(ngroups - 1) * p.ld_s + p.N) * 2);
    // lane parts of the offsets; a group's part is uniform (groups past the wave's share read
    // zeros: lane part OOB, uniform part 0)
    const uint32_t vx = i < p.M ? (uint32_t)((i * p.lda + 8 * g) * 2) : OOB;
    const uint32_t vw = (uint32_t)(lane * 16);
    const uint32_t vs = (uint32_t)((n0 + i) * 2);
    // the workgroup's first tile in its block of the prepacked layout (every block is whole)
    const uint32_t blk = (uint32_t)(((int64_t)(nt0 / W4P_BLOCK_TILES) * ngroups * W4P_BLOCK_TILES +
                                     nt0 % W4P_BLOCK_TILES) * 1024);

    const uint32_t nz = f32_to_bf16(-(128.0f + (float)p.zero_point));
    const uint32_t nz2 = nz | (nz << 16);
    const bf16x8 negz = __builtin_bit_cast(bf16x8, u32x4{nz2, nz2, nz2, nz2});
    const W4Unpack unpack_w4;

    f32x4 tot[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) tot[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 x[W4S_RING][4];
    u32x4 w[W4S_RING][NTW];
    uint32_t sr[W4S_RING][NTW / 2];  // scales of columns 16 t + i, two per register
    auto load = [&](int gi, int slot) {
        const bool in = gi < g1;
        const uint32_t lx = in ? vx : OOB, lw = in ? vw : OOB, ls = in ? vs : OOB;
        // codes first: they come from memory, the activations mostly from L2
#pragma unroll
        for (int t = 0; t < NTW; ++t)
            w[slot][t] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rw, lw, in ? (uint32_t)(blk + gi * (W4P_BLOCK_TILES * 1024) + t * 1024) : 0u,
                           W4S_CODE_POLICY));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            x[slot][kb] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, lx, in ? (uint32_t)(gi * 256 + kb * 64) : 0u, 0));
        const uint32_t so = in ? (uint32_t)(gi * p.ld_s * 2) : 0u;
#pragma unroll
        for (int t = 0; t < NTW; t += 2) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, ls, so + t * 32, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, ls, so + t * 32 + 32, 0);
            sr[slot][t / 2] = lo | (hi << 16);
        }
    };
    auto consume = [&](int slot) {
        f32x4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) corr = mfma_bf16(x[slot][kb], negz, corr);
        f32x4 u[NTW];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                u[t] = mfma_bf16(x[slot][kb], unpack_w4(w[slot][t][kb]), kb == 0 ? corr : u[t]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const float sv = (t & 1) ? bf16hi(sr[slot][t / 2]) : bf16lo(sr[slot][t / 2]);
#pragma unroll
            for (int q = 0; q < 4; ++q) tot[t][q] = fmaf(sv, u[t][q], tot[t][q]);
        }
    };

    // ring of W4S_RING groups: group j sits in slot j % W4S_RING
    load(g0, 0);
#pragma unroll
    for (int u = 1; u < W4S_RING; ++u)
        if (g0 + u < g1) load(g0 + u, u);
    for (int j0 = g0; j0 < g1; j0 += W4S_RING) {
#pragma unroll
        for (int u = 0; u < W4S_RING; ++u) {
            const int gi = j0 + u;
            if (gi < g1) {
                consume(u);
                if (gi + W4S_RING < g1) load(gi + W4S_RING, u);
            }
        }
    }

    // partial tile -> LDS: lane (g, i) holds rows 4 g + e, column 16 t + i
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) red[(wave * MR + 4 * g + e4) * NC + 16 * t + i] = tot[t][e4];
    __syncthreads();
    if constexpr (SPLIT)
        split_reduce_epilogue<MR, NC, NS, NWV>(p, red, n0, cb, ks, ncb, &s_last);
    else
        reduce_epilogue<MR, NC, NWV>(p, red, n0);
}

// A lane reads, per 32-deep block, 8 consecutive rows of one 8-column chunk
// (8 bytes per row).  Each byte is converted once to fp32 (u8: the code
// itself, 0..255; fp8: the hardware E4M3 conversion, both exact) and pairs of
// rows of one column are packed into bf16 (exact), which forms the MFMA B
// fragments of 8 k values per column directly, with no transpose.  The u8
// zero point z enters as -z * sum(x) over the group, from one extra MFMA per
// block against a fragment of ones.  Per-group scales multiply the fp32
// partial sums: a wave's blocks start on a group boundary and each group's
// partial is folded into the total with the scales of the lane's 8 columns.
// Grid: column blocks x NS K-splits; 8 waves per workgroup split its K range.
template <int WF, int NS>
__global__ __launch_bounds__(S_THREADS) void skinny_w8_kernel(Problem p) {
    constexpr bool SPLIT = NS > 1;
    constexpr int NC = 128, MR = 16;
    __shared__ __attribute__((aligned(16))) float red[S_WAVES * MR * NC];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int ncb = (int)gridDim.x / NS;
    const int cb = (int)blockIdx.x % ncb;
    const int ks = (int)blockIdx.x / ncb;
    const int n0 = cb * NC;

    const int nkb = p.K / 32, gb = p.group / 32;  // blocks, blocks per scale group
    const int nvw = NS * S_WAVES;                 // waves sharing K
    const int per = ((nkb + nvw - 1) / nvw + gb - 1) / gb * gb;
    const int kb0 = (ks * S_WAVES + wave) * per, kb1 = min(nkb, kb0 + per);

    const bool nin = n0 + 8 * i < p.N;
    // raw [K, N] codes: lane (g, i) reads rows 8 g + r of the block, bytes n0 + 8 i ..; prepacked
    // (gemm_w4_prepack): the column block's run of 4 KB blocks, rows r = 2q and 2q + 1 of a block
    // being one 16-byte load per lane (1 KB contiguous over the 64 lanes)
    const bool packed = p.w4_packed != 0;
    const __amdgpu_buffer_rsrc_t rw =
        packed ? make_rsrc((const char *)p.B + (int64_t)cb * nkb * 4096, (int64_t)nkb * 4096)
               : make_rsrc(p.B, (int64_t)(p.K - 1) * p.ldb + p.N);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scales, ((int64_t)(p.K / p.group - 1) * p.ld_s + p.N) * 2);
    // lane parts of the offsets (OOB for lanes past N or M); block parts are uniform
    const uint32_t vw = packed ? (uint32_t)(lane * 16) : nin ? (uint32_t)(8 * g * p.ldb + n0 + 8 * i) : OOB;
    const uint32_t vx = i < p.M ? (uint32_t)((i * p.lda + 8 * g) * 2) : OOB;
    const uint32_t vs = nin ? (uint32_t)((n0 + 8 * i) * 2) : OOB;
    const uint32_t blk_w = packed ? 4096u : (uint32_t)(32 * p.ldb);
    const uint32_t row_w = packed ? 512u : (uint32_t)p.ldb;
    const float zp = (float)p.zero_point;

    f32x4 acc[8], part[8], xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = part[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x2 w[SK_RING][8];
    bf16x8 xr[SK_RING];
    u32x4 sr[SK_RING];
    // Blocks past the wave's share read zeros: their lane offsets become OOB
    // and their uniform offsets 0, so no sum wraps past 2^32 (every in-range
    // sum stays below 2^31, every OOB one between 2^31 and 2^32).
    auto load_blk = [&](int kb, int slot) {
        const bool in = kb < kb1;
        const uint32_t so = in ? (uint32_t)kb * blk_w : 0u;
        const uint32_t lw = in ? vw : OOB;
        if (packed) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, lw, so + (uint32_t)q * 1024u, NT));
                w[slot][2 * q] = u32x2{v[0], v[1]};
                w[slot][2 * q + 1] = u32x2{v[2], v[3]};
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                w[slot][r] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, lw, so + (uint32_t)r * row_w, NT));
        }
        xr[slot] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? vx : OOB, in ? (uint32_t)kb * 64u : 0u, 0));
        sr[slot] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, in ? vs : OOB,
                                                         in ? (uint32_t)((kb / gb) * p.ld_s * 2) : 0u, 0));
    };
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    auto fold = [&](const u32x4 &s8) {  // total += scale * (partial - z * sum x), per column
        float sc[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sc[2 * q] = bf16lo(s8[q]);
            sc[2 * q + 1] = bf16hi(s8[q]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = WF == WFMT_U8 ? fmaf(-zp, xs[e], part[t][e]) : part[t][e];
                acc[t][e] = fmaf(sc[t], v, acc[t][e]);
            }
            part[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        xs = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // one block: bytes -> fp32 -> bf16 fragments (column t: rows 0..7), 8 MFMAs
    auto consume = [&](int slot) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {  // columns 4 hh .. 4 hh + 3
            float f[8][4];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t c = w[slot][r][hh];
                if constexpr (WF == WFMT_FP8) {
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
                    f[r][0] = lo[0], f[r][1] = lo[1], f[r][2] = hi[0], f[r][3] = hi[1];
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b) f[r][b] = (float)((c >> (8 * b)) & 0xffu);
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                u32x4 fr;
#pragma unroll
                for (int q = 0; q < 4; ++q) fr[q] = pack_bf16x2(f[2 * q][b], f[2 * q + 1][b]);
                part[4 * hh + b] = mfma_bf16(xr[slot], __builtin_bit_cast(bf16x8, fr), part[4 * hh + b]);
            }
        }
        if constexpr (WF == WFMT_U8) xs = mfma_bf16(xr[slot], ones, xs);
    };

#pragma unroll
    for (int j = 0; j < SK_RING - 1; ++j) load_blk(kb0 + j, j);
    for (int kb = kb0; kb < kb1; kb += SK_RING) {
#pragma unroll
        for (int u = 0; u < SK_RING; ++u) {
            load_blk(kb + u + SK_RING - 1, (u + SK_RING - 1) % SK_RING);
            consume(u);
            // last block of a scale group: kb - kb0 is a multiple of SK_RING and kb0 of gb
            if (((kb - kb0 + u + 1) % gb) == 0) fold(sr[u]);
        }
    }

    // partial tile -> LDS: lane (g, i) holds rows 4 g + e, columns 8 i + t
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        float *dst = &red[(wave * MR + 4 * g + e4) * NC + 8 * i];
        *(f32x4 *)dst = f32x4{acc[0][e4], acc[1][e4], acc[2][e4], acc[3][e4]};
        *(f32x4 *)(dst + 4) = f32x4{acc[4][e4], acc[5][e4], acc[6][e4], acc[7][e4]};
    }
    __syncthreads();
    if constexpr (SPLIT)
        split_reduce_epilogue<MR, NC, NS>(p, red, n0, cb, ks, ncb, &s_last);
    else
        reduce_epilogue<MR, NC>(p, red, n0);
}

// Prepack: raw [K, N/2] bytes (two codes per byte, order per lo_first) ->
// per (16-column tile, 128-row group): 64 lanes x 16 bytes; lane l, dword kb
// holds the 8 codes of column 16 tile + l % 16 at k = 128 group + 32 kb +
// 8 (l / 16) + j: code j at bits 4 (j/2) + 16 (j%2) ... i.e. even j in the
// low half, odd j in the high half, so that unpack_w4 yields k in order.
__global__ __launch_bounds__(256) void w4_prepack_kernel(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq,
                                                         int32_t lo_first, uint8_t *Wp) {
    const int64_t ngroups = K / 128, ntiles = N / 16;
    const int64_t total = ntiles * ngroups * 64;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(u & 63);
        const int64_t tg = u >> 6;
        const int64_t gi = tg % ngroups, nt = tg / ngroups;
        const int64_t n = nt * 16 + (l & 15);
        const bool even = (n & 1) == 0;
        const bool hi = even != (lo_first != 0);
        u32x4 out;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            uint32_t d = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t k = gi * 128 + kb * 32 + 8 * (l >> 4) + j;
                const uint8_t b = Wq[k * ldq + (n >> 1)];
                const uint32_t code = hi ? (b >> 4) : (b & 0xF);
                d |= code << (4 * (j >> 1) + 16 * (j & 1));
            }
            out[kb] = d;
        }
        *(u32x4 *)(Wp + w4p_frag_offset(nt, gi, ngroups, ntiles) + l * 16) = out;
    }
}

bool al16(const void *q) { return ((uintptr_t)q & 15) == 0; }

}  // namespace

hipError_t launch_w4_prepack(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq, int32_t lo_first, uint8_t *Wp,
                             hipStream_t s) {
    const int64_t total = (int64_t)(N / 16) * (K / 128) * 64;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(w4_prepack_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s, K, N, Wq, ldq,
                       lo_first, Wp);
    return hipGetLastError();
}

// 16-column tiles per block of the prepacked bf16 layout: 7 (112 columns) where that gives every
// CU the same number of blocks and 128-column blocks do not (16 x 28672: 256 blocks of 112 against
// 224 of 128 on 256 CUs), else 8
int bf16p_block_tiles(int N, int cu_count) {
    if (cu_count <= 0 || N % 112) return 8;
    const bool even112 = (N / 112) % cu_count == 0, even128 = N % 128 == 0 && (N / 128) % cu_count == 0;
    return even112 && !even128 ? 7 : 8;
}

// SwiGLU pairs on prepacked weights: the block width that makes the 2 N / (16 TB) workgroups fill
// the CUs (112-column blocks only where N is a multiple of 112)
int swiglu_block_tiles(int N, int cu_count) {
    if (cu_count <= 0 || N % 112) return 8;
    const bool even112 = (2 * (N / 112)) % cu_count == 0, even128 = N % 128 == 0 && (2 * (N / 128)) % cu_count == 0;
    return even112 && !even128 ? 7 : 8;
}

int64_t swiglu_prepacked_scratch_bytes(int M, int N, int cu_count) {
    const int tb = swiglu_block_tiles(N, cu_count);
    const int64_t ncb = N / (16 * tb), mr = M <= 16 ? 16 : 32;
    return 2 * ncb * mr * 16 * tb * 4 + ncb * 4;
}

const char *swiglu_prepacked_name(int N, int cu_count) {
    return swiglu_block_tiles(N, cu_count) == 7 ? "skinny_bf16p_swiglu_112col_pairs" : "skinny_bf16p_swiglu_128col_pairs";
}

// p: mode SWIGLU, B / B2 the prepacked gate and up weights, split_ws / split_cnt the plan's scratch
hipError_t launch_swiglu_prepacked(const Problem &p, int cu_count, hipStream_t s) {
    if (!p.split_ws || !p.split_cnt || p.M > 32) return hipErrorInvalidValue;
    const int tb = swiglu_block_tiles(p.N, cu_count);
    const dim3 grid(2 * (p.N / (16 * tb)));
    if (tb == 7) {
        if (p.M <= 16)
            hipLaunchKernelGGL((skinny_bf16p_swiglu_kernel<1, 7>), grid, dim3(S_THREADS), 0, s, p);
        else
            hipLaunchKernelGGL((skinny_bf16p_swiglu_kernel<2, 7>), grid, dim3(S_THREADS), 0, s, p);
    } else {
        if (p.M <= 16)
            hipLaunchKernelGGL((skinny_bf16p_swiglu_kernel<1, 8>), grid, dim3(S_THREADS), 0, s, p);
        else
            hipLaunchKernelGGL((skinny_bf16p_swiglu_kernel<2, 8>), grid, dim3(S_THREADS), 0, s, p);
    }
    return hipGetLastError();
}

namespace {
int bf16_chunks(int N, int cu_count);
}

// raw weights: 8-column chunks per workgroup (8 or 16) for 2 N columns' worth of workgroups
int swiglu_raw_chunks(int N, int cu_count) { return bf16_chunks(2 * N, cu_count > 0 ? cu_count : 256); }

int64_t swiglu_raw_scratch_bytes(int M, int N, int cu_count) {
    const int nch = swiglu_raw_chunks(N, cu_count);
    const int64_t ncb = (N + 8 * nch - 1) / (8 * nch), mr = M <= 16 ? 16 : 32;
    return 2 * ncb * mr * 8 * nch * 4 + ncb * 4;
}

int64_t swiglu_pair_blocks(int N, int cu_count, bool prepacked) {
    if (prepacked) return N / (16 * swiglu_block_tiles(N, cu_count));
    const int nch = swiglu_raw_chunks(N, cu_count);
    return (N + 8 * nch - 1) / (8 * nch);
}

const char *swiglu_raw_name(int N, int cu_count) {
    return swiglu_raw_chunks(N, cu_count) == 8 ? "skinny_bf16_swiglu_64col_pairs" : "skinny_bf16_swiglu_128col_pairs";
}

// whether the raw pairs can read these operands (the raw decode kernel's conditions, for both weights)
bool swiglu_raw_supported(const Problem &p) {
    Problem g = p, u = p;
    g.mode = u.mode = MODE_GENERIC;
    u.B = p.B2;
    g.b_packed = u.b_packed = 0;
    return p.M <= 32 && skinny_supported(g) && skinny_supported(u);
}

hipError_t launch_swiglu_raw(const Problem &p, int cu_count, hipStream_t s) {
    if (!p.split_ws || !p.split_cnt || p.M > 32) return hipErrorInvalidValue;
    const int nch = swiglu_raw_chunks(p.N, cu_count);
    const dim3 grid(2 * ((p.N + 8 * nch - 1) / (8 * nch)));
    auto go = [&](auto MTC) {
        constexpr int MT = decltype(MTC)::value;
        if (nch == 8)
            hipLaunchKernelGGL((skinny_bf16_swiglu_kernel<MT, 8>), grid, dim3(S_THREADS), 0, s, p);
        else
            hipLaunchKernelGGL((skinny_bf16_swiglu_kernel<MT, 16>), grid, dim3(S_THREADS), 0, s, p);
    };
    if (p.M <= 16)
        go(std::integral_constant<int, 1>{});
    else
        go(std::integral_constant<int, 2>{});
    return hipGetLastError();
}

hipError_t launch_b_prepack(int32_t K, int32_t N, const uint16_t *B, int64_t ldb, uint16_t *Bp, int cu_count,
                            hipStream_t s, int tb_override) {
    const int tb = tb_override ? tb_override : bf16p_block_tiles(N, cu_count);
    const int64_t total = (int64_t)(N / (16 * tb)) * (K / 32) * 64 * tb;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)(blocks > 0 ? blocks : 1));
    if (tb == 7)
        hipLaunchKernelGGL(b_prepack_kernel<7>, grid, dim3(256), 0, s, K, N, B, ldb, Bp);
    else
        hipLaunchKernelGGL(b_prepack_kernel<8>, grid, dim3(256), 0, s, K, N, B, ldb, Bp);
    return hipGetLastError();
}

// raw [K, N] 8-bit codes (row stride ldq) -> the prepacked layout: the 8 bytes of lane l, row r
// (0..7) of 32-row block kb of column block cb, i.e. row 32 kb + 8 (l / 16) + r, columns
// 128 cb + 8 (l % 16) .. + 7, go to byte 1024 (r / 2) + 16 l + 8 (r % 2) of the block's 4 KB
// (block index cb * K / 32 + kb), so one 16-byte load gives a lane rows 2q and 2q + 1
__global__ __launch_bounds__(256) void w8_prepack_kernel(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq,
                                                         uint8_t *Wp) {
    const int64_t nkb = K / 32, total = (int64_t)(N / 128) * nkb * 512;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(u & 63), r = (int)((u >> 6) & 7);
        const int64_t blk = u >> 9, kb = blk % nkb, cb = blk / nkb;
        const int64_t k = kb * 32 + 8 * (l >> 4) + r, n = cb * 128 + 8 * (l & 15);
        *(u32x2 *)(Wp + blk * 4096 + (r >> 1) * 1024 + l * 16 + (r & 1) * 8) = *(const u32x2 *)(Wq + k * ldq + n);
    }
}

hipError_t launch_w8_prepack(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq, uint8_t *Wp, hipStream_t s) {
    const int64_t total = (int64_t)(N / 128) * (K / 32) * 512;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(w8_prepack_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s, K, N, Wq, ldq, Wp);
    return hipGetLastError();
}

bool skinny_supported(const Problem &p) {
    if (p.ab_type != GE_BF16 || p.M > 32) return false;
    if (p.mode == MODE_SWIGLU) return false;
    if (!al16(p.A) || (p.lda & 7) || (p.K & 7)) return false;
    if (p.b_packed)
        return p.mode == MODE_GENERIC && p.M <= 32 && (p.N % 128) == 0 && (p.K % 32) == 0 && al16(p.B) &&
               ((int64_t)(p.M - 1) * p.lda + p.K) * 2 < (1ll << 31) && (int64_t)p.K * 256 < (1ll << 31);
    if (p.mode == MODE_W4 && p.wfmt != WFMT_U4) {
        // 8-bit codes: 8-byte weight loads, 16-byte scale loads, 32-bit offsets
        if (p.w4_packed && ((p.N % 128) || !al16(p.B) || (int64_t)p.K * 128 >= (1ll << 31))) return false;
        return p.M <= 16 && (p.K % 32) == 0 && (p.N % 8) == 0 && ((uintptr_t)p.B & 7) == 0 && (p.ldb % 8) == 0 &&
               al16(p.scales) && (p.ld_s % 8) == 0 && (int64_t)p.K * p.ldb < (1ll << 31) &&
               ((int64_t)(p.M - 1) * p.lda + p.K) * 2 < (1ll << 31);
    }
    if (p.mode == MODE_W4) {
        // codes, scales and activations through 32-bit buffer offsets
        return p.w4_packed && p.M <= 32 && (p.K % 128) == 0 && (p.N % 16) == 0 && al16(p.B) &&
               (p.group == 32 || p.group == 64 || p.group == 128) &&
               ((int64_t)(p.M - 1) * p.lda + p.K) * 2 < (1ll << 31) && (int64_t)p.K * p.N / 2 < (1ll << 31) &&
               ((int64_t)(p.K / p.group - 1) * p.ld_s + p.N) * 2 < (1ll << 31);
    }
    if (p.b_layout != GE_LAYOUT_KN || !al16(p.B) || (p.ldb & 7) || (p.N & 7)) return false;
    // the streaming loop addresses one wave's share of W at a time: at most ceil(K / 32 / 8)
    // blocks of 32 rows (the plain kernel's share; the stream-K shares are no longer)
    const int64_t share_rows = (int64_t)((p.K + 31) / 32 + S_WAVES - 1) / S_WAVES * 32;
    const int64_t b_bytes = ((share_rows - 1) * p.ldb + p.N) * 2;
    const int64_t a_bytes = ((int64_t)(p.M - 1) * p.lda + p.K) * 2;
    return b_bytes < (1ll << 31) && a_bytes < (1ll << 31);
}

namespace {
// 8-column chunks per bf16 workgroup: the choice that minimises the columns
// the busiest CU streams, ceil(workgroups / CUs) * chunks (ties: wider).
// Only 16 and 8 keep every workgroup's row segments on 128-byte boundaries;
// 112- and 96-column blocks share cache lines between neighbours and measured
// slower (the decode shape 16 x 28672 x 8192 went from 98 to 117 us).
int bf16_chunks(int N, int cu_count) {
    static const int opts[] = {16, 8};
    int best = 16;
    int64_t best_cost = -1;
    for (int c : opts) {
        const int64_t wgs = (N + 8 * c - 1) / (8 * c);
        const int64_t cost = (wgs + cu_count - 1) / cu_count * c;
        if (best_cost < 0 || cost < best_cost) best = c, best_cost = cost;
    }
    return best;
}

template <int MT>
void launch_bf16(const Problem &p, int nch, hipStream_t s) {
    const int blocks = (p.N + 8 * nch - 1) / (8 * nch);
    if (nch == 8)
        hipLaunchKernelGGL((skinny_bf16_kernel<MT, 8>), dim3(blocks), dim3(S_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((skinny_bf16_kernel<MT, 16>), dim3(blocks), dim3(S_THREADS), 0, s, p);
}
}  // namespace

// The int4 decode kernel over 64-column blocks (prepacked 128-row groups, M <= 16).
constexpr int W4S_NTW = 8, W4S_WAVES = 8, W4S_MAX_SPLIT = 8;
bool w4s_ok(const Problem &p) {
    return p.mode == MODE_W4 && p.wfmt == WFMT_U4 && p.w4_packed && p.group == 128 && p.M <= 16 &&
           p.N % (16 * W4S_NTW) == 0;
}

// K splits of the 8-bit and the 128-column int4 kernels: the fewest (a power
// of two, at most 8) that give every CU a workgroup, while each wave keeps at
// least one scale group (int4: one 128-row group).
int w8_split(const Problem &p, int cu_count) {
    if (p.mode != MODE_W4 || (p.wfmt == WFMT_U4 && !w4s_ok(p))) return 1;
    const bool u4 = p.wfmt == WFMT_U4;
    const int ncb = split_counters(p), nkb = p.K / 32, gb = u4 ? 4 : p.group / 32;
    const int max_split = u4 ? W4S_MAX_SPLIT : 8, waves = u4 ? W4S_WAVES : S_WAVES;
    int s = 1;
    while (s < max_split && (int64_t)ncb * s < cu_count && nkb / (2 * s * waves) >= gb) s *= 2;
    return s;
}

// column blocks of the split kernels: one counter and one [16][block width] fp32 tile per split each
int split_counters(const Problem &p) { return w4s_ok(p) ? p.N / (16 * W4S_NTW) : (p.N + 127) / 128; }

int64_t w8_split_scratch_bytes(const Problem &p, int split) {
    if (split <= 1) return 0;
    const int64_t ncb = split_counters(p), nc = w4s_ok(p) ? 16 * W4S_NTW : 128;
    return split * ncb * 16 * nc * 4 + ncb * 4;
}

// Tile slots per column block of the stream-K decode kernel, or 0 for the plain kernel.
// Stream-K is used where the plain kernel leaves CUs idle (its workgroups are not a multiple
// of the CU count) and each workgroup's range is one piece of one column block (the ranges
// divide the blocks evenly): a range that straddles two blocks streams two short segments
// with a handoff each, which measured slower than idle CUs (16 x 28672 x 8192: 98 us against
// 93 us for the plain kernel on 224 of 256 CUs).  At 16 x 8192 x 8192 it is a 4-way K split.
int bf16_sk_slots(const Problem &p, int cu_count) {
    if (p.mode != MODE_GENERIC || p.ab_type != GE_BF16 || p.M > 16 || cu_count <= 0) return 0;
    if (p.b_packed) {
        // prepacked: every range is one contiguous run of memory.  Used when one workgroup per
        // column block would leave at least half of the CUs idle (16 x 8192 x 8192: 29.5 us
        // against 52 us), with at most 8 workgroups sharing a block.  With more blocks the
        // plain kernel wins: at 16 x 28672 x 8192 (224 blocks on 256 CUs) 81.9 us against
        // 90.4 us, the ranges' second segments and handoffs costing more than 32 idle CUs.
        const int64_t ncb = p.N / 128, nkb = p.K / 32, U = ncb * nkb;
        if (2 * ncb > cu_count || U < 8ll * cu_count) return 0;
        const int64_t slots = (nkb + U / cu_count - 1) / (U / cu_count) + 1;
        return slots <= 8 ? (int)slots : 0;
    }
    const int nch = bf16_chunks(p.N, cu_count);
    const int64_t plain = (p.N + 8 * nch - 1) / (8 * nch);
    if (plain % cu_count == 0) return 0;
    const int64_t ncb = (p.N + 127) / 128, nkb = (p.K + 31) / 32, U = ncb * nkb;
    if (U % cu_count || U < 8ll * cu_count) return 0;
    const int64_t per = U / cu_count;  // units per workgroup
    if (per >= nkb || nkb % per) return 0;
    const int64_t slots = nkb / per;
    return slots >= 2 && slots <= 8 ? (int)slots : 0;
}

int64_t bf16_sk_scratch_bytes(const Problem &p, int slots) {
    if (slots <= 0) return 0;
    const int64_t ncb = (p.N + 127) / 128;
    return ncb * slots * 16 * 128 * 4 + ncb * 4;
}

const char *skinny_kernel_name(const Problem &p, int cu_count, bool scratch) {
    if (p.mode == MODE_W4 && p.wfmt != WFMT_U4) {
        static const char *names[2][4] = {
            {"skinny_u8_m16_128col", "skinny_u8_m16_128col_split2", "skinny_u8_m16_128col_split4",
             "skinny_u8_m16_128col_split8"},
            {"skinny_fp8_m16_128col", "skinny_fp8_m16_128col_split2", "skinny_fp8_m16_128col_split4",
             "skinny_fp8_m16_128col_split8"}};
        static const char *packed_names[2][4] = {
            {"skinny_u8_m16_128col_prepacked", "skinny_u8_m16_128col_split2_prepacked",
             "skinny_u8_m16_128col_split4_prepacked", "skinny_u8_m16_128col_split8_prepacked"},
            {"skinny_fp8_m16_128col_prepacked", "skinny_fp8_m16_128col_split2_prepacked",
             "skinny_fp8_m16_128col_split4_prepacked", "skinny_fp8_m16_128col_split8_prepacked"}};
        const int s = scratch ? w8_split(p, cu_count) : 1;
        return (p.w4_packed ? packed_names : names)[p.wfmt == WFMT_FP8][s == 1 ? 0 : s == 2 ? 1 : s == 4 ? 2 : 3];
    }
    if (p.mode == MODE_W4) {
        if (w4s_ok(p)) {
            const int sp = w8_split(p, cu_count);
            if (sp == 1) return "skinny_w4_m16_128col";
            if (scratch)
                return sp == 2 ? "skinny_w4_m16_128col_split2" : sp == 4 ? "skinny_w4_m16_128col_split4"
                                                                    : "skinny_w4_m16_128col_split8";
        }
        return p.M <= 16 ? "skinny_w4_m16_32col" : "skinny_w4_m32_32col";
    }
    if (p.b_packed) {
        if (scratch && bf16_sk_slots(p, cu_count) > 0) return "skinny_bf16_m16_prepacked_streamk";
        if (bf16p_block_tiles(p.N, cu_count) == 7)
            return p.M <= 16 ? "skinny_bf16_m16_112col_prepacked" : "skinny_bf16_m32_112col_prepacked";
        return p.M <= 16 ? "skinny_bf16_m16_128col_prepacked" : "skinny_bf16_m32_128col_prepacked";
    }
    if (scratch && bf16_sk_slots(p, cu_count) > 0) return "skinny_bf16_m16_128col_streamk";
    static const char *names[2][2] = {{"skinny_bf16_m16_128col", "skinny_bf16_m16_64col"},
                                      {"skinny_bf16_m32_128col", "skinny_bf16_m32_64col"}};
    return names[p.M > 16][bf16_chunks(p.N, cu_count) == 16 ? 0 : 1];
}

hipError_t launch_skinny(const Problem &p, int cu_count, hipStream_t s) {
    if (!skinny_supported(p)) return hipErrorInvalidValue;
    if (p.mode == MODE_W4 && p.wfmt != WFMT_U4) {
        const int ncb = (p.N + 127) / 128;
        const int ns = (p.split_ws && p.split_cnt) ? p.split : 1;
        if (ns != 1 && ns != 2 && ns != 4 && ns != 8) return hipErrorInvalidValue;
        const dim3 grid(ncb * ns);
        auto go = [&](auto WFC) {
            constexpr int W = decltype(WFC)::value;
            if (ns == 8)
                hipLaunchKernelGGL((skinny_w8_kernel<W, 8>), grid, dim3(S_THREADS), 0, s, p);
            else if (ns == 4)
                hipLaunchKernelGGL((skinny_w8_kernel<W, 4>), grid, dim3(S_THREADS), 0, s, p);
            else if (ns == 2)
                hipLaunchKernelGGL((skinny_w8_kernel<W, 2>), grid, dim3(S_THREADS), 0, s, p);
            else
                hipLaunchKernelGGL((skinny_w8_kernel<W, 1>), grid, dim3(S_THREADS), 0, s, p);
        };
        if (p.wfmt == WFMT_FP8)
            go(std::integral_constant<int, WFMT_FP8>{});
        else
            go(std::integral_constant<int, WFMT_U8>{});
        return hipGetLastError();
    }
    if (p.mode == MODE_W4 && w4s_ok(p)) {
        // the split the plan chose, with its scratch; without scratch the 32-column kernel
        // below, unless the shape needs no split
        const int ns = (p.split_ws && p.split_cnt) ? p.split : 1;
        if (ns > 1 || w8_split(p, cu_count > 0 ? cu_count : 256) == 1) {
            if (ns != 1 && ns != 2 && ns != 4 && ns != 8) return hipErrorInvalidValue;
            const dim3 grid(split_counters(p) * ns);
            const dim3 block(64 * W4S_WAVES);
            if (ns == 8)
                hipLaunchKernelGGL((skinny_w4s_kernel<W4S_NTW, 8, W4S_WAVES>), grid, block, 0, s, p);
            else if (ns == 4)
                hipLaunchKernelGGL((skinny_w4s_kernel<W4S_NTW, 4, W4S_WAVES>), grid, block, 0, s, p);
            else if (ns == 2)
                hipLaunchKernelGGL((skinny_w4s_kernel<W4S_NTW, 2, W4S_WAVES>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((skinny_w4s_kernel<W4S_NTW, 1, W4S_WAVES>), grid, block, 0, s, p);
            return hipGetLastError();
        }
    }
    if (p.mode == MODE_W4) {
        constexpr int NTW = 2;
        const int blocks = (p.N / 16 + NTW - 1) / NTW;
        auto go = [&](auto MTC) {
            constexpr int MT = decltype(MTC)::value;
            if (p.group == 32)
                hipLaunchKernelGGL((skinny_w4_kernel<NTW, 1, MT>), dim3(blocks), dim3(W4_THREADS), 0, s, p);
            else if (p.group == 64)
                hipLaunchKernelGGL((skinny_w4_kernel<NTW, 2, MT>), dim3(blocks), dim3(W4_THREADS), 0, s, p);
            else
                hipLaunchKernelGGL((skinny_w4_kernel<NTW, 4, MT>), dim3(blocks), dim3(W4_THREADS), 0, s, p);
        };
        if (p.M <= 16)
            go(std::integral_constant<int, 1>{});
        else
            go(std::integral_constant<int, 2>{});
        return hipGetLastError();
    }
    if (p.mode == MODE_GENERIC && p.M <= 16 && p.split > 1 && p.split_ws && p.split_cnt) {
        const dim3 grid(cu_count > 0 ? cu_count : 256);
        if (p.b_packed)
            hipLaunchKernelGGL(skinny_bf16_sk_kernel<true>, grid, dim3(S_THREADS), 0, s, p);
        else
            hipLaunchKernelGGL(skinny_bf16_sk_kernel<false>, grid, dim3(S_THREADS), 0, s, p);
        return hipGetLastError();
    }
    if (p.b_packed) {
        const int tb = bf16p_block_tiles(p.N, cu_count);
        const dim3 grid(p.N / (16 * tb));
        if (tb == 7) {
            if (p.M <= 16)
                hipLaunchKernelGGL((skinny_bf16p_kernel<1, 7>), grid, dim3(S_THREADS), 0, s, p);
            else
                hipLaunchKernelGGL((skinny_bf16p_kernel<2, 7>), grid, dim3(S_THREADS), 0, s, p);
        } else {
            if (p.M <= 16)
                hipLaunchKernelGGL((skinny_bf16p_kernel<1, 8>), grid, dim3(S_THREADS), 0, s, p);
            else
                hipLaunchKernelGGL((skinny_bf16p_kernel<2, 8>), grid, dim3(S_THREADS), 0, s, p);
        }
        return hipGetLastError();
    }
    const int nch = bf16_chunks(p.N, cu_count > 0 ? cu_count : 256);
    if (p.M <= 16)
        launch_bf16<1>(p, nch, s);
    else
        launch_bf16<2>(p, nch, s);
    return hipGetLastError();
}

}  // namespace ge
