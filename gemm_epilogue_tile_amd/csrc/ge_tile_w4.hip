// ge_tile_w4.hip -- int4 weights (prepacked), M > 16: MFMA tile kernel with
// the dequantisation in the K-loop and the epilogue in the store path (page
// "Fusion Thinking", Pattern 3: packed int4 codes, zero point, per-group
// scales, dequantised in registers on the way into the product).

#include "ge_launch.hpp"

namespace ge {
namespace {
#include "ge_tile_common.hpp"

// ---------------------------------------------------------------------------
// int4 weights (prepacked), M > 16: 128 x 128 tiles, fp16 MFMA.
//
// (c - z) * s with z = 8 has at most 3 + 8 significant bits, so the
// dequantised weight is exact in fp16 (scales in the fp16 normal range); bf16
// activations convert to fp16 exactly (|x| in the fp16 range).  The products
// are then exact in fp32 and the accumulators need no per-group rescaling.
//
// Activations: a pre-pass converts X to fp16 once per call into the plan's
// scratch (each element is used by all N / 128 column tiles, so converting
// it in every workgroup was the kernel's largest cost); the tile kernel
// streams the fp16 rows by direct loads straight into a ring of swizzled
// fragment buffers, as the bf16 tile kernel does.
//
// Waves: the four waves sit side by side (wave w: all 128 rows, columns
// n0 + 32 w .. + 31), so no two waves use the same weights.  Each wave loads
// the codes of its two prepacked 16-column tiles and their 32 scales into a
// private LDS slot by direct loads (no barrier: a wave reads back only what
// it loaded itself), and every lane dequantises its own B fragments in
// registers, straight from the 16 prepacked bytes its load delivered: 16
// codes per lane per stage, each code converted once per workgroup, with no
// round trip of fp16 weights through LDS.  Only the activations are shared
// through LDS.  (Sharing dequantised fp16 fragments between 2 x 2 waves
// through LDS took 92.5 us per call at 512 x 8192 x 8192; this layout 72.)
//
// Pipeline, per stage s (unrolled by 8 = two 128-row scale groups): the fp16
// activations of stage s + 6 and (every fourth stage) the raw codes and
// scales of the group after next go straight to LDS by direct loads (waits
// counted by hand; the stage's position sits in the buffer resource, so no
// vector instruction computes an address); every fourth stage the codes and
// scales of the next group are read into registers; the activation fragments
// of stage s + 1 are read and its B fragments dequantised; the 16 MFMAs of
// stage s run on the fragments prepared one stage earlier.  One barrier per
// stage.
//
// Dequant: a dword holds 8 codes, pair w (w = 0..3) at bits 4 w .. 4 w + 3 of
// each 16-bit half.  Pairs at bits 0..3 are OR-ed into the mantissa of fp16
// 1024 (ulp 1), pairs at bits 4..7 into that of fp16 64 (ulp 1/16), which
// gives magic + c exactly either way with one v_and_or_b32 (pairs 2 and 3
// after one shift by 8); then a packed subtract of magic + z and a packed
// multiply by s.  13 instructions per 8 codes.
// ---------------------------------------------------------------------------

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void mfma_f16_acc(f32x4 &acc, const f16x8 &a, const f16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 8 bf16 (one u32x4) -> 8 fp16 (exact for values in the fp16 range)
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4 &w) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(w[q]), bf16hi(w[q])));
    return r;
}

constexpr int W4_BM = 128, W4_BN = 128;
constexpr int W4_MT = 8, W4_NT = 2;          // 16x16 tiles per wave: 128 rows x 32 columns
constexpr int W4_UNROLL = 8;                 // stages per loop trip (ring sizes divide it)
constexpr int W4_AD = 6;                     // activation loads run this many stages ahead
// LDS (bytes): fp16 activations, ring of 8 stages ([128][32] in the swizzled fragment layout);
// per wave, the raw codes of two groups (its two prepacked 16-column tiles, 1 KB each) and the
// raw scales of two groups (one 1 KB slot per group, the wave's 32 columns in its first 64 bytes)
constexpr int W4_A16 = 0, W4_A16_STAGE = W4_BM * 64;
constexpr int W4_CODES = W4_A16 + W4_UNROLL * W4_A16_STAGE, W4_CODES_WAVE = 2 * 2 * 1024;
constexpr int W4_SCALES = W4_CODES + 4 * W4_CODES_WAVE, W4_SCALES_WAVE = 2 * 1024;
constexpr int W4_LDS = W4_SCALES + 4 * W4_SCALES_WAVE;  // 88 KB

// direct loads issued by each wave: 2 per stage (activations), 3 per group (codes, scales)
constexpr int W4_LA = 2, W4_LB = 3;
static_assert(W4_LA * 4 * 64 * 16 == W4_A16_STAGE, "four waves load one activation stage");
// loads a wave may still have in flight at the top of stage u (mod 8) when everything issued up to
// stage u - 4 must have landed: the activations of stages u-3 .. u-1 and the group loads among them
// (issued at stages = 2 mod 4)
constexpr int w4_inflight(int u) {
    int n = 3 * W4_LA;
    for (int k = 1; k <= 3; ++k)
        if (((u - k) % 4 + 4) % 4 == 2) n += W4_LB;
    return n;
}
static_assert(w4_inflight(0) == w4_inflight(1) && w4_inflight(1) == w4_inflight(3), "one group load among three stages");

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

__global__ __attribute__((amdgpu_flat_work_group_size(T_THREADS, T_THREADS), amdgpu_waves_per_eu(1, 1)))
void tile_w4_kernel(Problem p) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(AS3 void *)smem;
    const AS3 char *s3 = (const AS3 char *)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int tiles_m = (p.M + W4_BM - 1) / W4_BM, tiles_n = p.N / W4_BN;
    const int total = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (t / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * W4_BM, n0 = tn * W4_BN;
    const int ngroups = p.K / 128, nst = p.K / T_BK;

    // Direct loads.  The lane offsets are fixed; the stage's (or group's) position goes into the
    // buffer resource (scalar arithmetic), whose range is empty past the end of K, so the loop
    // spends no vector instructions on addresses.
    // activations: wave w loads rows 32 w .. 32 w + 31 of each stage, lane l row l / 4 of 16, LDS
    // slot l % 4 of the row holding logical chunk (l % 4) ^ ((row >> 1) & 3)
    const char *a_base = (const char *)p.A16 + (int64_t)m0 * p.K * 2;
    const int64_t a_bytes = (int64_t)(p.M - m0) * p.K * 2;
    uint32_t a_src[W4_LA];
#pragma unroll
    for (int q = 0; q < W4_LA; ++q) {
        const int row_l = lane >> 2;
        const int chunk = (lane & 3) ^ ((row_l >> 1) & 3);
        a_src[q] = (uint32_t)(((wave * W4_LA + q) * 16 + row_l) * p.K * 2 + chunk * 16);
    }
    auto load_a = [&](int d, int slot) {
        const i32x4 r = rsrc32(a_base + d * 64, d < nst ? (uint32_t)(a_bytes - d * 64) : 0u);
#pragma unroll
        for (int q = 0; q < W4_LA; ++q)
            load_lds16(r, lds0 + W4_A16 + slot * W4_A16_STAGE + (wave * W4_LA + q) * 1024, a_src[q]);
    };
    // codes of the wave's tiles 2 w, 2 w + 1 (group g: 1 KB at g KB into each tile's run) and
    // their 32 scales (lanes 0..3) into the wave's slot
    const int64_t b_bytes = (int64_t)p.K * p.N / 2, s_bytes = ((int64_t)(ngroups - 1) * p.ld_s + p.N) * 2;
    uint32_t b_src[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) b_src[q] = (uint32_t)((((int64_t)(n0 / 16 + wave * 2 + q) * ngroups) * 64 + lane) * 16);
    const uint32_t s_src = lane < 4 ? (uint32_t)((n0 + wave * 32) * 2 + lane * 16) : OOB;
    const uint32_t codes_w = W4_CODES + wave * W4_CODES_WAVE, scales_w = W4_SCALES + wave * W4_SCALES_WAVE;
    auto load_b = [&](int g, int slot) {
        const bool in = g < ngroups;
        const i32x4 rb = rsrc32((const char *)p.B + (int64_t)g * 1024, in ? (uint32_t)(b_bytes - (int64_t)g * 1024) : 0u);
#pragma unroll
        for (int q = 0; q < 2; ++q) load_lds16(rb, lds0 + codes_w + slot * 2048 + q * 1024, b_src[q]);
        const int64_t so = (int64_t)g * p.ld_s * 2;
        const i32x4 rs = rsrc32((const char *)p.scales + so, in ? (uint32_t)(s_bytes - so) : 0u);
        load_lds16(rs, lds0 + scales_w + slot * 1024, s_src);
    };

    // a group's codes (lane's own 16 bytes of each tile) and scales (column 16 e + lane % 16)
    const int frow = lane & 15, fgrp = lane >> 4;
    // code pairs at bits 0..3 (of each half) go into the mantissa of fp16 1024 (ulp 1), pairs at
    // bits 4..7 into that of fp16 64 (ulp 1/16): both give magic + c exactly, with one v_and_or_b32
    // and no shift for the latter
    const _Float16 zl = (_Float16)(1024.0f + (float)p.zero_point), zh = (_Float16)(64.0f + (float)p.zero_point);
    const f16x2 zlo2 = f16x2{zl, zl}, zhi2 = f16x2{zh, zh};
    const uint32_t mask_lo = __builtin_amdgcn_readfirstlane(0x000f000fu);
    const uint32_t mask_hi = __builtin_amdgcn_readfirstlane(0x00f000f0u);
    uint32_t magic_lo = 0x64006400u, magic_hi = 0x54005400u;
    asm volatile("" : "+v"(magic_lo), "+v"(magic_hi));
    u32x4 craw[2][2];
    f16x2 cs2[2][2];
    auto read_group = [&](int gp) {  // ring slot gp = group parity (compile-time)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            craw[gp][e] = *(const AS3 u32x4 *)(s3 + codes_w + gp * 2048 + e * 1024 + lane * 16);
            const uint16_t sr = *(const AS3 uint16_t *)(s3 + scales_w + gp * 1024 + (16 * e + frow) * 2);
            const _Float16 sh = (_Float16)bf16_to_f32(sr);
            cs2[gp][e] = f16x2{sh, sh};
        }
    };
    // B fragments of stage d (dd = d % 8): piece k = 0..7 dequantises code pair k % 4 of tile k / 4
    // (pair w holds the nibbles 4 w .. 4 w + 3 of each half of the dword; pairs 2, 3 after a shift by 8)
    f16x8 fb[2][W4_NT];
    u32x4 dq[W4_NT];
    uint32_t csh[W4_NT];
    auto dequant_piece = [&](int dd, int k) {
        const int gp = (dd >> 2) & 1, q = dd & 3, e = k >> 2, w = k & 3;
        uint32_t src;
        if (w < 2) {
            src = craw[gp][e][q];
            asm volatile("" : "+v"(src));
            if (w == 0) csh[e] = src >> 8;
        } else {
            src = csh[e];
        }
        uint32_t tt;
        if (w & 1)
            asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(tt) : "v"(src), "s"(mask_hi), "v"(magic_hi));
        else
            asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(tt) : "v"(src), "s"(mask_lo), "v"(magic_lo));
        uint32_t o = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, tt) - ((w & 1) ? zhi2 : zlo2)) * cs2[gp][e]);
        asm volatile("" : "+v"(o));
        dq[e][w] = o;
        if (w == 3) fb[dd & 1][e] = __builtin_bit_cast(f16x8, dq[e]);
    };

    const int a_frag = W4_A16 + swz_a(frow, fgrp);
    f16x8 fa[2][W4_MT];
    auto read_a = [&](int dd, int i) {
        fa[dd & 1][i] = *(const AS3 f16x8 *)(s3 + a_frag + dd * W4_A16_STAGE + i * 1024);
    };

    f32x4 acc[W4_MT][W4_NT];
#pragma unroll
    for (int i = 0; i < W4_MT; ++i)
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto lds_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
#define GE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x70 | 0xF00)

    // prologue (issue order and waits as in tile_w4_kernel): stage 0's activations, group 0 and
    // stage 1's activations landed; group 0 read, stage 0's fragments read and dequantised
    load_a(0, 0);
    load_b(0, 0);
    load_a(1, 1);
    load_a(2, 2);
    load_a(3, 3);
    load_a(4, 4);
    load_b(1, 1);
    load_a(5, 5);
    GE_WAIT_VM(4 * W4_LA + W4_LB);
    lds_barrier();
    read_group(0);
#pragma unroll
    for (int i = 0; i < W4_MT; ++i) read_a(0, i);
#pragma unroll
    for (int k = 0; k < 2 * 4; ++k) dequant_piece(0, k);

    // stage s = s0 + u: wait for the loads of stage s - 4 and earlier, barrier, then the 16 MFMAs
    // of stage s with, between them: the direct loads of stage s + 6 (and at u % 4 == 2 the group
    // after next), at u % 4 == 2 the read of the next group's codes, the activation fragments of
    // stage s + 1 and its B fragments
    const int nsteps = (nst + W4_UNROLL - 1) / W4_UNROLL * W4_UNROLL;
    for (int s0 = 0; s0 < nsteps; s0 += W4_UNROLL) {
#pragma unroll
        for (int u = 0; u < W4_UNROLL; ++u) {
            const int s = s0 + u;
            if ((u & 3) == 2)
                GE_WAIT_VM(w4_inflight(2));
            else
                GE_WAIT_VM(w4_inflight(0));
            lds_barrier();
            const int dn = (u + 1) & (W4_UNROLL - 1);
#pragma unroll
            for (int q = 0; q < W4_MT * W4_NT; ++q) {
                const int i = q & (W4_MT - 1), j = q / W4_MT;
                mfma_f16_acc(acc[i][j], fb[u & 1][j], fa[u & 1][i]);
                asm volatile("" ::: "memory");
                if (q == 0) {
                    load_a(s + W4_AD, (u + W4_AD) & (W4_UNROLL - 1));
                    if ((u & 3) == 2) {
                        load_b((s + 6) >> 2, ((u + 6) >> 2) & 1);
                        read_group(((u + 2) >> 2) & 1);  // group (s + 2) / 4, loaded at stage s - 4
                    }
                }
                if (q >= 1 && q <= W4_MT) read_a(dn, q - 1);
                if (q >= W4_MT) dequant_piece(dn, q - W4_MT);
                asm volatile("" ::: "memory");
            }
        }
    }
#undef GE_WAIT_VM
    __builtin_amdgcn_s_waitcnt(0);
    mfma_drain();
#pragma unroll
    for (int i = 0; i < W4_MT; ++i)
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) asm volatile("" : "+a"(acc[i][j]));

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

// X (bf16, [M][K] with row stride lda) -> dense fp16 [M][K]: exact for |x| in the fp16 normal range
__global__ __launch_bounds__(256) void a16_convert_kernel(int32_t M, int32_t K, const uint16_t *A, int64_t lda,
                                                          uint16_t *A16) {
    const int64_t cpr = K / 8, chunks = (int64_t)M * cpr;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
        const int64_t m = c / cpr, kc = c - m * cpr;
        const u32x4 w = *(const u32x4 *)(A + m * lda + kc * 8);
        *(u32x4 *)(A16 + m * K + kc * 8) = bf16x8_to_f16x8(w);
    }
}

}  // namespace

bool tile_w4_supported(const Problem &p) {
    if (p.mode != MODE_W4 || !p.w4_packed || p.M <= 16) return false;
    if ((p.N % W4_BN) || (p.K % 128) || (p.lda & 7) || !al16(p.A) || !al16(p.B)) return false;
    if (p.group != 128 || !al16(p.scales) || (p.ld_s & 7)) return false;
    if ((int64_t)p.M * p.K * 2 >= (1ll << 31)) return false;  // the fp16 copy of X
    if ((int64_t)p.K * p.N / 2 >= (1ll << 31) || ((int64_t)(p.K / 128) * p.ld_s + p.N) * 2 >= (1ll << 31)) return false;
    return epi_ok(p);
}

int64_t tile_w4_scratch_bytes(const Problem &p) { return (int64_t)p.M * p.K * 2; }

const char *tile_w4_kernel_name() { return "tile_w4_f16_128x128x32"; }

hipError_t launch_tile_w4(const Problem &p, hipStream_t s) {
    if (!tile_w4_supported(p) || !p.A16) return hipErrorInvalidValue;
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)tile_w4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           W4_LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t chunks = (int64_t)p.M * (p.K / 8);
    const int cblocks = (int)((chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096);
    hipLaunchKernelGGL(a16_convert_kernel, dim3(cblocks), dim3(256), 0, s, p.M, p.K, (const uint16_t *)p.A, p.lda,
                       (uint16_t *)p.A16);
    const int tiles = ((p.M + W4_BM - 1) / W4_BM) * (p.N / W4_BN);
    hipLaunchKernelGGL(tile_w4_kernel, dim3(tiles), dim3(T_THREADS), W4_LDS, s, p);
    return hipGetLastError();
}

}  // namespace ge
