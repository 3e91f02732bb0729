// ge_tile_w4.hip -- quantised weights, M > 32 (int4 prepacked) or M > 16
// (8-bit codes, raw layout): MFMA tile kernel with the dequantisation in the
// K-loop and the epilogue in the store path (page "Fusion Thinking", Pattern
// 3: packed int4 codes, zero point, per-group scales, dequantised in registers
// on the way into the product; the same loader for INT8 / FP8 codes).

#include "ge_launch.hpp"

namespace ge {
namespace {
#include "ge_tile_common.hpp"

// ---------------------------------------------------------------------------
// int4 weights (prepacked), M > 32: 64 x 128 tiles (two workgroups per CU), bf16 MFMA.
//
// Arithmetic, exact for every finite bf16 X and scale up to fp32 summation
// order (no fp16 range or rounding anywhere).  A code c becomes the bf16 value
// 128 + c by OR-ing it into the mantissa of 0x4300, so for 128-row group g
//   sum_k x[m][k] (c[k][n] - z) s[g][n]
//     = s[g][n] * U_g[m][n]  -  (128 + z) * Sx_g[m] * s[g][n],
//   U_g[m][n] = sum_{k in g} x[m][k] (128 + c[k][n])   (bf16 MFMA, fp32),
//   Sx_g[m]   = sum_{k in g} x[m][k].
// 8-bit codes take the same scheme with the code's own value instead of
// 128 + c: u8 codes 0..255 and fp8 E4M3 values are exact in bf16; for u8 the
// correction is -z * Sx_g * s[g][n], for fp8 there is none.
// The first term is accumulated group by group in fp32 registers (one fma per
// output element per group).  The second term is a small product over the
// groups, Sx (rows x groups) by s (groups x columns), run on the MFMA once per
// 32 groups: -(128 + z) Sx is split exactly into three bf16 parts, the scales
// are bf16 already, so each MFMA product is exact and the sum is fp32.
//
// Waves: the four waves sit side by side (wave w: all 64 rows, columns
// n0 + 32 w .. + 31), so no two waves use the same weights.  Each wave loads
// the codes of its two prepacked 16-column tiles and their 32 scales into a
// private LDS slot by direct loads (no barrier: a wave reads back only what
// it loaded), and every lane turns its own 16 prepacked bytes into B
// fragments in registers, 16 codes per lane per stage (7 instructions per 8
// codes: three shifts and four v_and_or_b32).  The bf16 activations are
// shared through LDS: direct loads from X (its own row stride) six stages
// ahead into a ring of eight swizzled fragment buffers.  Wave w also sums
// rows 16 w .. 16 w + 15 of every stage from that ring (v_dot2 against
// ones), completes Sx_g at the group's last stage and writes its three bf16
// parts to the correction buffer; one barrier per stage orders every LDS
// hand-over.  Two workgroups share a CU, so one's vector work runs beside
// the other's MFMAs.
//
// 8-bit codes stream from the raw [K, N] layout instead: each stage, each wave
// direct-loads its 32 columns x 32 rows (1 KB) three stages ahead into a
// private ring of four slots, and reads its B fragments back with the
// transposing LDS read ds_read_b64_tr_b8 (lane pairs name a 16-byte row, each
// lane receives one column's 8 consecutive k), then converts the bytes to
// bf16 (u8: one conversion per byte and one packing per pair; fp8: one
// scaled conversion per pair).
//
// Pipeline, per stage s (unrolled by 8 = two groups): at a group's first stage
// the previous group's partial products are scaled into the accumulators and
// the stage's MFMAs start new partials (zero C); every 32 groups (and at the
// end) the correction product runs; the direct loads of stage s + 6 and
// (every fourth stage) the codes and scales of the group after next are
// issued; every fourth stage the next group's codes and scales are read into
// registers; the activation fragments of stage s + 1 are read and its B
// fragments made; the 16 MFMAs of stage s run on the fragments prepared one
// stage earlier.
// ---------------------------------------------------------------------------

constexpr int W4_BM = 64;
constexpr int W4_MT = 4, W4_NT = 2;          // 16x16 tiles per wave: 64 rows x 32 columns
constexpr int W4_UNROLL = 8;                 // stages per loop trip (ring sizes divide it)
constexpr int W4_AD = 6;                     // activation loads run this many stages ahead
constexpr int W4_CHUNK = 32;                 // groups per correction product (one MFMA k-step)
static_assert(W4_MT * W4_NT == 8, "one dequantisation piece per MFMA of a stage");
// LDS (bytes): bf16 activations, ring of 8 stages ([64][32] in the swizzled fragment layout);
// per wave, the raw codes of two groups (its two prepacked 16-column tiles, 1 KB each) and the
// raw scales of two groups (one 1 KB slot per group, the wave's 32 columns in its first 64 bytes);
// the correction operands: three bf16 parts of -(128 + z) Sx, [part][m-tile][16 rows][32 groups],
// and per wave the scales, [n-tile][16 columns][32 groups] (both 64-byte rows: fragment order)
constexpr int W4_AS = 0, W4_AS_STAGE = W4_BM * 64;
constexpr int W4_CODES_WAVE = 2 * 2 * 1024, W4_SCALES_WAVE = 2 * 1024;
constexpr int W4_CA_BYTES = 3 * W4_MT * 1024, W4_CB_WAVE = W4_NT * 1024;
// NW waves side by side: a 64 x 32 NW tile.  NW = 4: 76 KB of LDS, two workgroups per CU; NW = 8:
// 108 KB, one workgroup of 8 waves per CU, whose activation tile and row sums serve 256 columns
// (half the activation loads and row sums per CU of two 4-wave workgroups)
template <int NW>
struct W4L {
    static constexpr int BN = 32 * NW, THREADS = 64 * NW;
    static constexpr int CODES = W4_AS + W4_UNROLL * W4_AS_STAGE;
    static constexpr int SCALES = CODES + NW * W4_CODES_WAVE;
    static constexpr int CA = SCALES + NW * W4_SCALES_WAVE;
    static constexpr int CB = CA + W4_CA_BYTES;
    static constexpr int LDS = CB + NW * W4_CB_WAVE;
    static constexpr int RL = NW, RL_LOG = NW == 8 ? 3 : 2;  // lanes per row in the row sums (rows per wave: 64 / NW)
};

// direct loads issued by each wave: per group 3 (int4 codes, scales) or 1 (8-bit: scales); 4-wave
// workgroups: one activation load per stage (stage s + 6 at stage s); 8-wave: one every other stage,
// at even stages s, of the pair s + 6, s + 7 (waves 0-3 the first, 4-7 the second), so that every
// wave of the workgroup issues the same sequence and the wait counts below hold for all of them
constexpr int W4_LB = 3;
// loads a wave may still have in flight at the top of stage u (mod 8) when everything issued up to
// stage u - 4 must have landed: the activations and the group loads (issued at stages = 2 mod 4) of
// stages u-3 .. u-1
constexpr int w4_inflight(int NW, int u) {
    int n = 0;
    for (int k = 1; k <= 3; ++k) {
        const int t = ((u - k) % 8 + 8) % 8;
        if (NW == 4 || (t & 1) == 0) n += 1;
        if (t % 4 == 2) n += W4_LB;
    }
    return n;
}
static_assert(w4_inflight(4, 0) == 6 && w4_inflight(4, 3) == 6, "one group load among three stages");
static_assert(w4_inflight(8, 0) == 4 && w4_inflight(8, 1) == 5 && w4_inflight(8, 2) == 1 && w4_inflight(8, 3) == 5 &&
                  w4_inflight(8, 4) == w4_inflight(8, 0), "8 waves: activation pairs at even stages");

// buffer resource over [base, base + bytes), bytes already known to be in range (no 64-bit compare)
__device__ __forceinline__ i32x4 rsrc32(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// fp32 -> bf16 bits, round to nearest even
__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, 0.0f) & 0xffffu; }

// 8-bit codes: loads a wave may still have in flight at the top of stage u (mod 8) when the codes of
// stage u + 1 (issued last at stage u - 2) must have landed: the activations (if the wave loaded
// any), scales (at stages = 2 mod 4) and codes of stage u - 1
constexpr int w8_inflight(int NW, int u) {
    const int t = ((u - 1) % 8 + 8) % 8;
    return (NW == 4 || (t & 1) == 0 ? 1 : 0) + (t % 4 == 2 ? 1 : 0) + 1;
}
static_assert(w8_inflight(4, 0) == 2 && w8_inflight(4, 3) == 3 && w8_inflight(8, 0) == 1 && w8_inflight(8, 1) == 2 &&
                  w8_inflight(8, 3) == 3,
              "scale loads at stages = 2 mod 4");

// SPLIT: the grid is tiles x p.split K slices (p.split divides K / 128); each workgroup writes its
// fp32 partial tile to p.split_ws and counts itself in on the tile's counter in p.split_cnt; the last
// to arrive sums the slices in slice order (deterministic), runs the epilogue and re-arms the counter.
template <int WF, int NW, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void tile_w4_kernel(Problem p) {
    using L = W4L<NW>;
    constexpr bool U4 = WF == WFMT_U4, FP8 = WF == WFMT_FP8;
    constexpr bool CORR = !FP8;  // a zero-point term (int4: -(128 + z); u8: -z)
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(AS3 void *)smem;
    AS3 char *s3 = (AS3 char *)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int half = NW == 8 ? wave >> 2 : 0;  // 8 waves: which stage of a pair this wave loads
    const int tiles_m = (p.M + W4_BM - 1) / W4_BM, tiles_n = p.N / L::BN;
    const int total = tiles_m * tiles_n;
    const int nsplit = SPLIT ? p.split : 1, grid = total * nsplit;
    int t = blockIdx.x;
    if ((grid & 7) == 0) t = (t & 7) * (grid >> 3) + (t >> 3);
    const int ks = t / total;  // K slice
    t %= total;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (t / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * W4_BM, n0 = tn * L::BN;
    // K slice ks: groups g0 .. g0 + ngroups - 1 of the ngt groups of K (the whole K without a split)
    const int ngt = p.K / 128;
    const int ngroups = ngt / nsplit, nst = 4 * ngroups;
    const int g0 = ks * ngroups;
    const int64_t k0 = (int64_t)g0 * 128;

    // Direct loads.  The lane offsets are fixed; the stage's (or group's) position goes into the
    // buffer resource (scalar arithmetic), whose range is empty past the end of K, so the loop
    // spends no vector instructions on addresses.
    // activations: wave w (mod 4) loads rows 16 w .. 16 w + 15 of a stage, lane l row l / 4 of 16,
    // LDS slot l % 4 of the row holding logical chunk (l % 4) ^ ((row >> 1) & 3)
    const char *a_base = (const char *)p.A + ((int64_t)m0 * p.lda + k0) * 2;
    const int64_t a_bytes = ((int64_t)(p.M - m0 - 1) * p.lda + p.K - k0) * 2;
    const int arow_l = lane >> 2;
    const uint32_t a_src = (uint32_t)((int64_t)((wave & 3) * 16 + arow_l) * p.lda * 2 +
                                      (((lane & 3) ^ ((arow_l >> 1) & 3)) * 16));
    auto load_a = [&](int d, int slot) {
        const i32x4 r = rsrc32(a_base + d * 64, d < nst ? (uint32_t)(a_bytes - d * 64) : 0u);
        load_lds16(r, lds0 + W4_AS + slot * W4_AS_STAGE + (wave & 3) * 1024, a_src);
    };
    // int4: codes of the wave's tiles 2 w, 2 w + 1 and their 32 scales (lanes 0..3) into the wave's
    // slot, once per group; 8-bit: the scales once per group, the codes once per stage
    const int64_t b_bytes = U4 ? (int64_t)p.K * p.N / 2 : (int64_t)(p.K - 1) * p.ldb + p.N;
    const int64_t s_bytes = ((int64_t)(ngt - 1) * p.ld_s + p.N) * 2;
    uint32_t b_src[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        // tile tt of the prepacked layout (N is a multiple of 128, so every 128-column block is
        // whole): a group's eight tiles of one block are 8 KiB in a row
        const int tt = n0 / 16 + wave * 2 + q;
        b_src[q] = (uint32_t)(((int64_t)(tt / W4P_BLOCK_TILES) * ngt * W4P_BLOCK_TILES + tt % W4P_BLOCK_TILES) *
                                  1024 + lane * 16);
    }
    const uint32_t s_src = lane < 4 ? (uint32_t)((n0 + wave * 32) * 2 + lane * 16) : OOB;
    const uint32_t codes_w = L::CODES + wave * W4_CODES_WAVE, scales_w = L::SCALES + wave * W4_SCALES_WAVE;
    auto load_b = [&](int g, int slot) {
        const bool in = g < ngroups;
        if constexpr (U4) {
            const int64_t go = (int64_t)(g0 + g) * W4P_BLOCK_TILES * 1024;
            const i32x4 rb = rsrc32((const char *)p.B + go, in ? (uint32_t)(b_bytes - go) : 0u);
#pragma unroll
            for (int q = 0; q < 2; ++q) load_lds16(rb, lds0 + codes_w + slot * 2048 + q * 1024, b_src[q]);
        }
        const int64_t so = (int64_t)(g0 + g) * p.ld_s * 2;
        const i32x4 rs = rsrc32((const char *)p.scales + so, in ? (uint32_t)(s_bytes - so) : 0u);
        load_lds16(rs, lds0 + scales_w + slot * 1024, s_src);
    };
    // 8-bit codes of stage d (rows 32 d .. 32 d + 31, the workgroup's BN columns) go to slot d % 4 of
    // a ring the waves share: [32 rows][BN bytes], 16-byte chunk c of row r at c ^ q_swz(r), so that
    // the transposing reads of 16 rows hit distinct banks.  Wave w loads rows 1024 / BN of them, whole
    // 128-byte lines (a wave's own 32 columns are a quarter line per row: four times the line
    // requests); lane l row l / (BN / 16) of those, slot l % (BN / 16).  A wave reads other waves'
    // codes, after the stage barrier that follows every wave's wait for them.
    constexpr int QCH = L::BN / 16, Q_STAGE = 32 * L::BN;
    auto q_swz = [](int r) { return NW == 8 ? (r & 15) : ((r >> 1) & 7); };
    const int q_row = (1024 / L::BN) * wave + lane / QCH;
    const uint32_t q_src = (uint32_t)((int64_t)q_row * p.ldb + n0 + (((lane % QCH) ^ q_swz(q_row)) * 16));
    auto load_q = [&](int d) {
        const int64_t ro = (int64_t)(4 * g0 + d) * 32 * p.ldb;
        const i32x4 rq = rsrc32((const char *)p.B + ro, d < nst ? (uint32_t)(b_bytes - ro) : 0u);
        load_lds16(rq, lds0 + L::CODES + (d & 3) * Q_STAGE + wave * 1024, q_src);
    };

    const int frow = lane & 15, fgrp = lane >> 4;
    // a group's codes (the lane's own 16 bytes of each tile) and scales: the four columns
    // 16 j + 4 fgrp .. + 3 of each tile (the accumulator layout, two bf16 per dword) and column
    // 16 j + frow (the correction product's B fragment layout)
    u32x4 craw[2][W4_NT];
    u32x2 sacc[2][W4_NT];
    uint32_t sfrag[2];
    auto read_group = [&](int gp) {  // ring slot gp = group parity (compile-time)
#pragma unroll
        for (int e = 0; e < W4_NT; ++e) {
            if constexpr (U4) craw[gp][e] = *(const AS3 u32x4 *)(s3 + codes_w + gp * 2048 + e * 1024 + lane * 16);
            sacc[gp][e] = *(const AS3 u32x2 *)(s3 + scales_w + gp * 1024 + (16 * e + 4 * fgrp) * 2);
        }
        const uint32_t lo = *(const AS3 uint16_t *)(s3 + scales_w + gp * 1024 + frow * 2);
        const uint32_t hi = *(const AS3 uint16_t *)(s3 + scales_w + gp * 1024 + (16 + frow) * 2);
        sfrag[gp] = lo | (hi << 16);
    };
    // B fragments of stage d (dd = d % 8): piece k = 0..7 makes code pair k % 4 of tile k / 4 (pair
    // w holds the nibbles 4 w .. 4 w + 3 of each half of the dword) into two bf16 128 + c
    bf16x8 fb[2][W4_NT];
    u32x4 dq[W4_NT];
    // (src & mask) | magic in one v_and_or_b32: the mask in a scalar register and the magic in a
    // vector one, since this instruction takes no literal operand (the empty asm statements keep
    // the compiler from folding them back into literals; the arithmetic stays ordinary code, so the
    // compiler keeps track of the MFMAs still reading the registers it reuses)
    uint32_t nib_mask = 0x000f000fu, magic = 0x43004300u;
    asm volatile("" : "+s"(nib_mask));
    asm volatile("" : "+v"(magic));
    auto dequant_piece = [&](int dd, int k) {
        const int gp = (dd >> 2) & 1, q = dd & 3, e = k >> 2, w = k & 3;
        const uint32_t src = craw[gp][e][q] >> (4 * w);
        dq[e][w] = (src & nib_mask) | magic;
        if (w == 3) fb[dd & 1][e] = __builtin_bit_cast(bf16x8, dq[e]);
    };
    // 8-bit: the B fragments of stage d from slot d % 4 of the shared ring (the wave's column blocks
    // 2 w + j, j = 0, 1).  In each 16-lane group (k octet fgrp) lane pair 2 r, 2 r + 1 names row
    // 8 fgrp + r, the 16 bytes of block 2 w + j (wherever the swizzle put them), and lane frow
    // receives column 16 j + frow at k = 8 fgrp .. + 7 (byte order = k order)
    typedef int v2i __attribute__((ext_vector_type(2)));
    v2i qraw[W4_NT];
    uint32_t q_frag[W4_NT];
#pragma unroll
    for (int e = 0; e < W4_NT; ++e) {
        const int r = 8 * fgrp + (frow >> 1);
        q_frag[e] = L::CODES + r * L::BN + (((2 * wave + e) ^ q_swz(r)) * 16) + (frow & 1) * 8;
    }
    auto read_q = [&](int d) {
#pragma unroll
        for (int e = 0; e < W4_NT; ++e)
            qraw[e] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((AS3 v2i *)(s3 + q_frag[e] + (d & 3) * Q_STAGE));
    };
    // bytes -> bf16 fragment e of stage d (in two halves, h = 0, 1: one dword of 4 codes each)
    auto convert_q = [&](int dd, int e, int h) {
        const uint32_t w = (uint32_t)qraw[e][h];
        if constexpr (FP8) {
            dq[e][2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            dq[e][2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
        } else {
            dq[e][2 * h] = pack_bf16x2((float)(w & 0xffu), (float)((w >> 8) & 0xffu));
            dq[e][2 * h + 1] = pack_bf16x2((float)((w >> 16) & 0xffu), (float)(w >> 24));
        }
        if (h == 1) fb[dd & 1][e] = __builtin_bit_cast(bf16x8, dq[e]);
    };
    // piece k = 0..7 of stage dd's B fragments: int4 one dequantisation piece; 8-bit pieces 3 .. 6
    // convert the fragments read at piece 0 (a quarter each)
    auto b_piece = [&](int dd, int k) {
        if constexpr (U4) {
            dequant_piece(dd, k);
        } else {
            if (k == 0) read_q(dd);
            if (k >= 3 && k <= 6) convert_q(dd, (k - 3) >> 1, (k - 3) & 1);
        }
    };

    const int a_frag = W4_AS + swz_a(frow, fgrp);
    bf16x8 fa[2][W4_MT];
    auto read_a = [&](int dd, int i) {
        fa[dd & 1][i] = *(const AS3 bf16x8 *)(s3 + a_frag + dd * W4_AS_STAGE + i * 1024);
    };

    f32x4 acc[W4_MT][W4_NT], U[W4_MT][W4_NT];
#pragma unroll
    for (int i = 0; i < W4_MT; ++i)
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) acc[i][j] = U[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // row sums: wave w sums rows 16 w .. 16 w + 15 of each stage straight from the LDS ring, lane l
    // quarter l % 4 (16 of the row's 64 bytes, whatever logical chunk the swizzle put there) of row
    // 16 w + l / 4, with v_dot2 against bf16 ones
    const float cq = U4 ? -(128.0f + (float)p.zero_point) : -(float)p.zero_point;
    float rsum = 0.f, rsum2 = 0.f;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    // (4 waves: 16 rows per wave, 4 lanes x 16 bytes per row; 8 waves: 8 rows, 8 lanes x 8 bytes)
    constexpr int RB = 64 / L::RL;  // bytes of a row per lane
    const int rs_row = (64 / NW) * wave + (lane >> L::RL_LOG);
    const uint32_t rs_addr = W4_AS + rs_row * 64 + (lane & (L::RL - 1)) * RB;
    // (requested first in a stage and summed last, so that its wait does not cover the stage's
    // fragment reads, which are requested after it)
    using RV = std::conditional_t<NW == 4, u32x4, u32x2>;
    RV rs_v;
    auto row_read = [&](int dd) { rs_v = *(const AS3 RV *)(s3 + rs_addr + dd * W4_AS_STAGE); };
    auto row_sums = [&]() {
        // scalar copies: this compiler reads element 0 for a bit cast of a vector element; two
        // partial sums, so that the dot products form two short chains
        const uint32_t w0 = rs_v[0], w1 = rs_v[1];
        rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, rsum, false);
        rsum2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, rsum2, false);
        if constexpr (NW == 4) {
            const uint32_t w2 = rs_v[2], w3 = rs_v[3];
            rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, rsum, false);
            rsum2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, rsum2, false);
        }
    };
    // group g complete: the four quarters of each row added (lane swaps within each group of four
    // lanes through DPP quad permutations, no LDS round trip), the three bf16 parts of -(128 + z)
    // Sx_g written to the correction buffer (lanes 0, 1, 2 of a row's four write one each)
    auto write_sx = [&](int g) {
        const int gg = g % W4_CHUNK;
        float t2 = rsum + rsum2;
        t2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t2), 0xB1, 0xF, 0xF, false));
        t2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t2), 0x4E, 0xF, 0xF, false));
        if constexpr (NW == 8)  // the two quads of a row of eight lanes: half-row mirror
            t2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t2), 0x141, 0xF, 0xF, false));
        const float v = t2 * cq;
        rsum = 0.f;
        rsum2 = 0.f;
        const uint32_t hi = bf16_bits(v);
        const float r1 = v - __builtin_bit_cast(float, hi << 16);
        const uint32_t mid = bf16_bits(r1);
        const uint32_t lo = bf16_bits(r1 - __builtin_bit_cast(float, mid << 16));
        const uint32_t at = L::CA + (rs_row >> 4) * 1024 + (rs_row & 15) * 64 + gg * 2;
        const int part = lane & (L::RL - 1);
        if (part < 3) *(AS3 uint16_t *)(s3 + at + part * W4_MT * 1024) = (uint16_t)(part == 0 ? hi : part == 1 ? mid : lo);
    };
    // the wave's correction scales: lanes of k-octet 0 put column 16 j + frow of group g in place
    const uint32_t cb_w = L::CB + wave * W4_CB_WAVE;
    auto write_sb = [&](int g, int gp) {
        if (fgrp == 0) {
            const int gg = g % W4_CHUNK;
            *(AS3 uint16_t *)(s3 + cb_w + frow * 64 + gg * 2) = (uint16_t)(sfrag[gp] & 0xffffu);
            *(AS3 uint16_t *)(s3 + cb_w + 1024 + frow * 64 + gg * 2) = (uint16_t)(sfrag[gp] >> 16);
        }
    };
    // correction product of one chunk of groups: acc += Sx-parts (rows x groups) . s (groups x
    // columns), then the wave clears what it wrote (after the next barrier)
    auto correction = [&]() {
        bf16x8 bfr[W4_NT];
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) bfr[j] = *(const AS3 bf16x8 *)(s3 + cb_w + j * 1024 + frow * 64 + fgrp * 16);
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
            for (int i = 0; i < W4_MT; ++i) {
                const bf16x8 af = *(const AS3 bf16x8 *)(s3 + L::CA + (part * W4_MT + i) * 1024 + frow * 64 + fgrp * 16);
#pragma unroll
                for (int j = 0; j < W4_NT; ++j) acc[i][j] = mfma_bf16(bfr[j], af, acc[i][j]);
            }
    };
    auto clear_correction = [&]() {
        // this wave's parts (m-tile w: 3 KB) and its scales (2 KB)
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (wave < 4)  // m-tile w's three parts (8 waves: waves 0-3)
#pragma unroll
            for (int part = 0; part < 3; ++part) *(AS3 u32x4 *)(s3 + L::CA + (part * W4_MT + wave) * 1024 + lane * 16) = z;
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) *(AS3 u32x4 *)(s3 + cb_w + j * 1024 + lane * 16) = z;
    };
    // previous group's partial products into the accumulators: acc += s[n] * U
    auto apply_tile = [&](int gp, int i, int j) {
        const float s0 = bf16lo(sacc[gp][j][0]), s1 = bf16hi(sacc[gp][j][0]);
        const float s2 = bf16lo(sacc[gp][j][1]), s3f = bf16hi(sacc[gp][j][1]);
        acc[i][j][0] = __builtin_fmaf(s0, U[i][j][0], acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(s1, U[i][j][1], acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(s2, U[i][j][2], acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(s3f, U[i][j][3], acc[i][j][3]);
    };

    auto lds_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
#define GE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x70 | 0xF00)

    // prologue: correction buffers cleared; stage 0's activations, group 0 and stage 1's
    // activations landed (8-bit: also the codes of stages 0 .. 2, all of it); group 0 read, stage
    // 0's fragments read and its B fragments made
    if constexpr (CORR) clear_correction();
    // (the loads the loop's stages -6 .. -1 would have issued, in their order)
    if constexpr (NW == 4) {
        load_a(0, 0);
        load_b(0, 0);
        load_a(1, 1);
        load_a(2, 2);
        load_a(3, 3);
        load_a(4, 4);
        load_b(1, 1);
        load_a(5, 5);
    } else {
        load_a(half, half);
        load_b(0, 0);
        load_a(2 + half, 2 + half);
        load_a(4 + half, 4 + half);
        load_b(1, 1);
    }
    if constexpr (U4) {
        // after the activations of stages 0 and 1 come the later activation loads and one group's
        GE_WAIT_VM(NW == 4 ? 4 + W4_LB : 2 + W4_LB);
    } else {
        load_q(0);
        load_q(1);
        load_q(2);
        GE_WAIT_VM(0);
    }
    lds_barrier();
    read_group(0);
#pragma unroll
    for (int i = 0; i < W4_MT; ++i) read_a(0, i);
#pragma unroll
    for (int k = 0; k < 2 * 4; ++k) b_piece(0, k);

    // stage s = s0 + u: wait for the loads of stage s - 4 and earlier, barrier, then the 16 MFMAs
    // of stage s with, between them: (first stage of a group) the previous group scaled into the
    // accumulators, tile by tile; the direct loads of stage s + 6 (and at u % 4 == 2 the group
    // after next), at u % 4 == 2 the read of the next group's codes and scales, the activation
    // fragments of stage s + 1 and its B fragments
    const int nsteps = (nst + W4_UNROLL - 1) / W4_UNROLL * W4_UNROLL;
    for (int s0 = 0; s0 < nsteps; s0 += W4_UNROLL) {
#pragma unroll
        for (int u = 0; u < W4_UNROLL; ++u) {
            const int s = s0 + u;
            // (each branch names its wait count as a constant)
            if constexpr (U4) {
                if ((u & 3) == 0)
                    GE_WAIT_VM(w4_inflight(NW, 0));
                else if ((u & 3) == 1)
                    GE_WAIT_VM(w4_inflight(NW, 1));
                else if ((u & 3) == 2)
                    GE_WAIT_VM(w4_inflight(NW, 2));
                else
                    GE_WAIT_VM(w4_inflight(NW, 3));
            } else {
                if ((u & 3) == 0)
                    GE_WAIT_VM(w8_inflight(NW, 0));
                else if ((u & 3) == 1)
                    GE_WAIT_VM(w8_inflight(NW, 1));
                else if ((u & 3) == 2)
                    GE_WAIT_VM(w8_inflight(NW, 2));
                else
                    GE_WAIT_VM(w8_inflight(NW, 3));
            }
            lds_barrier();
            GE_DEBUG_BARRIER();
            __builtin_amdgcn_sched_barrier(0);
            const int dn = (u + 1) & (W4_UNROLL - 1);
            const bool first = (u & 3) == 0;           // first stage of a group
            const bool apply = first && s > 0;         // group s / 4 - 1 is complete
            if (CORR && apply) write_sb(s / 4 - 1, ((u >> 2) + 1) & 1);
            if (CORR && first && s > 0 && (s / 4) % W4_CHUNK == 0) correction();  // a chunk of groups is complete
            // one barrier later every wave has read it, and the next chunk's first writes (end of
            // this group's last stage) are still to come
            if (CORR && u == 1 && s0 > 0 && s0 % (4 * W4_CHUNK) == 0) clear_correction();
#pragma unroll
            for (int q = 0; q < W4_MT * W4_NT; ++q) {
                const int i = q & (W4_MT - 1), j = q / W4_MT;
                if (CORR && q == 0) row_read(u);
                if (apply) apply_tile(((u >> 2) + 1) & 1, i, j);
                U[i][j] = mfma_bf16(fb[u & 1][j], fa[u & 1][i], first ? f32x4{0.f, 0.f, 0.f, 0.f} : U[i][j]);
                if (q == 0) {
                    if constexpr (NW == 4)
                        load_a(s + W4_AD, (u + W4_AD) & (W4_UNROLL - 1));
                    else if ((u & 1) == 0)  // the pair s + 6, s + 7 (the slots of s - 2, s - 1)
                        load_a(s + W4_AD + half, (u + W4_AD + half) & (W4_UNROLL - 1));
                    if ((u & 3) == 2) {
                        load_b((s + 6) >> 2, ((u + 6) >> 2) & 1);
                        read_group(((u + 2) >> 2) & 1);  // group (s + 2) / 4, loaded at stage s - 4
                    }
                    if constexpr (!U4) load_q(s + 3);  // into the slot of stage s - 1, read at stage s - 2
                }
                if (CORR && q == W4_MT * W4_NT - 1) row_sums();
                if (q >= 1 && q <= W4_MT) read_a(dn, q - 1);
                b_piece(dn, q);  // 8 pieces: one per MFMA
                // keep each MFMA with the work placed beside it (the scheduler would otherwise
                // bunch the MFMAs and the reads and move them across the stage barriers)
                __builtin_amdgcn_sched_barrier(0);
            }
            if (CORR && (u & 3) == 3) write_sx(s / 4);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#undef GE_WAIT_VM
    __builtin_amdgcn_s_waitcnt(0);
    // the last group (stage nsteps - 4 .. nsteps - 1) and the last chunk's correction
    {
        const int g = nsteps / 4 - 1;  // odd: nsteps is a multiple of 8
        if constexpr (CORR) write_sb(g, 1);
#pragma unroll
        for (int i = 0; i < W4_MT; ++i)
#pragma unroll
            for (int j = 0; j < W4_NT; ++j) apply_tile(1, i, j);
        if constexpr (CORR) {
            lds_barrier();
            correction();
        }
    }

    if constexpr (SPLIT) {
        // partial tile -> slot (ks, t) of the scratch, lane-major (each lane's accumulators 16 bytes
        // apart over the lanes, so the last workgroup's lane reads back exactly what the same lane of
        // every slice wrote); device-scope cache policy on the stores and loads, a device-scope
        // counter per tile
        constexpr int SC1 = 16;
        constexpr uint32_t PT = NW * W4_MT * W4_NT * 1024;  // bytes of one partial tile
        __shared__ int s_last;
        const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
            (void *)p.split_ws, (short)0, (int)((uint32_t)grid * PT), 0x00020000);
        const uint32_t lane_off = (uint32_t)(wave * W4_MT * W4_NT * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < W4_MT; ++i)
#pragma unroll
            for (int j = 0; j < W4_NT; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rt,
                                                       (uint32_t)(ks * total + t) * PT + lane_off +
                                                           (uint32_t)(i * W4_NT + j) * 1024,
                                                       0, SC1);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are complete
        GE_DEBUG_FENCE();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(p.split_cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (uint32_t)(nsplit - 1);
        }
        __syncthreads();
        if (!s_last) return;
        GE_DEBUG_FENCE();
#pragma unroll
        for (int i = 0; i < W4_MT; ++i)
#pragma unroll
            for (int j = 0; j < W4_NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < nsplit; ++q) {  // slice order
            f32x4 part[W4_MT][W4_NT];
#pragma unroll
            for (int i = 0; i < W4_MT; ++i)
#pragma unroll
                for (int j = 0; j < W4_NT; ++j)
                    part[i][j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rt, (uint32_t)(q * total + t) * PT + lane_off + (uint32_t)(i * W4_NT + j) * 1024, 0, SC1));
#pragma unroll
            for (int i = 0; i < W4_MT; ++i)
#pragma unroll
                for (int j = 0; j < W4_NT; ++j) acc[i][j] += part[i][j];
        }
        if (threadIdx.x == 0) __hip_atomic_store(p.split_cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const EpiArgs &e = p.epi;
    const int mbase = m0 + frow;
    const int nbase = n0 + wave * 32 + fgrp * 4;
    auto small = [&](int64_t ld) { return ((int64_t)(p.M + 15) * ld + p.N) * 2 < (1ll << 31); };
    const bool all_bf16 = e.d_type == GE_BF16 && small(e.ldd) &&
                          (!(e.flags & GE_FLAG_C) || (e.c_type == GE_BF16 && small(e.ldc))) &&
                          (!(e.flags & GE_FLAG_RESIDUAL) || (e.r_type == GE_BF16 && small(e.ldr))) &&
                          (!(e.flags & GE_FLAG_BIAS) || e.bias_type == GE_BF16);
    with_act(e.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
        if (all_bf16) {
            if (e.flags & GE_FLAG_C)
                epilogue_bf16<ACT, true>(e, acc, p.M, p.N, mbase, n0 + wave * 32 + fgrp * 8);
            else
                epilogue_bf16<ACT, false>(e, acc, p.M, p.N, mbase, n0 + wave * 32 + fgrp * 8);
            return;
        }
#pragma unroll
        for (int i = 0; i < W4_MT; ++i)
#pragma unroll
            for (int j = 0; j < W4_NT; ++j) {
                const int m = mbase + i * 16, n = nbase + j * 16;
                if (m < p.M && n < p.N) {
                    float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    epi4<ACT>(e, v, m, n);
                }
            }
    });
}

}  // namespace

// 8 waves (64 x 256 tiles) where N allows and the tiles still fill the CUs, else 4 (64 x 128).  A
// workgroup's time is set by its own K loop (the loop is latency-bound), not by how many run: at
// 8192 x 8192, 33-256 rows take 79-80 us in 64 x 256 tiles (32-128 workgroups) against 61-62 us
// in 64 x 128 tiles; 512 rows 81 us against 85 us.
static int w4_waves(const Problem &p, int cu_count) {
    const int64_t tiles = (int64_t)((p.M + W4_BM - 1) / W4_BM) * (p.N / W4L<8>::BN);
    return p.N % W4L<8>::BN == 0 && tiles >= cu_count ? 8 : 4;
}

bool tile_w4_supported(const Problem &p) {
    if (p.mode != MODE_W4 || p.group != 128 || !al16(p.scales) || (p.ld_s & 7)) return false;
    if ((p.N % W4L<4>::BN) || (p.K % 128) || (p.lda & 7) || !al16(p.A) || !al16(p.B)) return false;
    if (((int64_t)(p.M - 1) * p.lda + p.K) * 2 >= (1ll << 31)) return false;  // X through 32-bit offsets
    if (((int64_t)(p.K / 128) * p.ld_s + p.N) * 2 >= (1ll << 31)) return false;
    if (p.wfmt == WFMT_U4) {
        // prepacked int4, M > 32 (smaller M streams the weights)
        if (!p.w4_packed || p.M <= 32 || (int64_t)p.K * p.N / 2 >= (1ll << 31)) return false;
    } else {
        // 8-bit codes in the raw [K, N] layout, M > 16: 16-byte rows pieces, 32-bit offsets
        if (p.w4_packed || p.M <= 16 || (p.ldb & 15) || (int64_t)p.K * p.ldb >= (1ll << 31)) return false;
    }
    return epi_ok(p);
}

// K split for too few tiles (33-256 rows): 64 x 128 tiles x S slices, S the largest of 2, 4, 8 that
// keeps tiles x S within the CU count, divides the K / 128 groups and leaves each slice 2 or more
static int tiles4(const Problem &p) { return ((p.M + W4_BM - 1) / W4_BM) * (p.N / W4L<4>::BN); }

int tile_w4_split(const Problem &p, int cu_count) {
    if (!tile_w4_supported(p) || cu_count <= 0) return 1;
    const int tiles = tiles4(p), ngt = p.K / 128;
    int s = 1;
    for (int c = 2; c <= 8; c *= 2)
        if ((int64_t)tiles * c <= cu_count && ngt % c == 0 && ngt / c >= 2) s = c;
    // 32-bit scratch offsets
    while (s > 1 && (int64_t)tiles * s * (4 * W4_MT * W4_NT * 1024) >= (1ll << 31)) s /= 2;
    return s;
}

int tile_w4_split_counters(const Problem &p) { return tiles4(p); }

int64_t tile_w4_split_scratch_bytes(const Problem &p, int split) {
    if (split <= 1) return 0;
    return (int64_t)tiles4(p) * split * (4 * W4_MT * W4_NT * 1024) + (int64_t)tiles4(p) * 4;
}

static bool use_split(const Problem &p) { return p.split > 1 && p.split_ws && p.split_cnt; }

const char *tile_w4_kernel_name(const Problem &p, int cu_count) {
    if (p.split > 1) {  // (named from the plan's choice, before its scratch exists)
        static const char *names[3][4] = {
            {"tile_w4_bf16_64x128x32_split2", "tile_w4_bf16_64x128x32_split4", "tile_w4_bf16_64x128x32_split8", ""},
            {"tile_w8_u8_64x128x32_split2", "tile_w8_u8_64x128x32_split4", "tile_w8_u8_64x128x32_split8", ""},
            {"tile_w8_fp8_64x128x32_split2", "tile_w8_fp8_64x128x32_split4", "tile_w8_fp8_64x128x32_split8", ""}};
        const int si = p.split == 2 ? 0 : p.split == 4 ? 1 : p.split == 8 ? 2 : 3;
        return names[p.wfmt == WFMT_U8 ? 1 : p.wfmt == WFMT_FP8 ? 2 : 0][si];
    }
    const bool w8 = w4_waves(p, cu_count) == 8;
    switch (p.wfmt) {
    case WFMT_U8: return w8 ? "tile_w8_u8_64x256x32" : "tile_w8_u8_64x128x32";
    case WFMT_FP8: return w8 ? "tile_w8_fp8_64x256x32" : "tile_w8_fp8_64x128x32";
    default: return w8 ? "tile_w4_bf16_64x256x32" : "tile_w4_bf16_64x128x32";
    }
}

template <int WF, int NW, bool SPLIT>
static hipError_t launch_wf(const Problem &p, hipStream_t s) {
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)tile_w4_kernel<WF, NW, SPLIT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, W4L<NW>::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((p.M + W4_BM - 1) / W4_BM) * (p.N / W4L<NW>::BN) * (SPLIT ? p.split : 1);
    hipLaunchKernelGGL((tile_w4_kernel<WF, NW, SPLIT>), dim3(tiles), dim3(W4L<NW>::THREADS), W4L<NW>::LDS, s, p);
    return hipGetLastError();
}

template <int WF>
static hipError_t launch_w(const Problem &p, int cu_count, hipStream_t s) {
    if (use_split(p)) {
        if ((p.K / 128) % p.split || p.split > 8) return hipErrorInvalidValue;
        return launch_wf<WF, 4, true>(p, s);
    }
    return w4_waves(p, cu_count) == 8 ? launch_wf<WF, 8, false>(p, s) : launch_wf<WF, 4, false>(p, s);
}

hipError_t launch_tile_w4(const Problem &p, int cu_count, hipStream_t s) {
    if (!tile_w4_supported(p)) return hipErrorInvalidValue;
    if (p.wfmt == WFMT_U8) return launch_w<WFMT_U8>(p, cu_count, s);
    if (p.wfmt == WFMT_FP8) return launch_w<WFMT_FP8>(p, cu_count, s);
    return launch_w<WFMT_U4>(p, cu_count, s);
}

}  // namespace ge
