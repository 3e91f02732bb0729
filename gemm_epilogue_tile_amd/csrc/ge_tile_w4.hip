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
// (code - z) * s has at most 3 + 8 significant bits, so the dequantised
// weight is exact in fp16 (for scales with |8 s| in the fp16 normal range);
// the bf16 activations convert to fp16 exactly (for |x| in the fp16 range).
// The products are then exact in fp32 and no per-group rescaling of the
// accumulators is needed.  Dequant per pair of codes: the codes are OR-ed into
// the mantissa of fp16 1024 (giving 1024 + c), then a packed subtract of
// 1024 + z and a packed multiply by s (exact for z = 8).  Scale groups of
// 128 rows.
//
// A: direct loads into 4 LDS stages of 32 k, as in the bf16 tile kernel.
// B: per 128-row group, the workgroup's 8 column tiles (8 KB, lane-major as
//    prepacked) go to one of two LDS group buffers by direct loads; each wave
//    reads its 4 tiles' 16 bytes per lane once per group.
// ---------------------------------------------------------------------------

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void mfma_f16_acc(f32x4 &acc, const f16x8 &a, const f16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// bf16 x8 -> fp16 x8 (exact for values in the fp16 range)
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(const bf16x8 &x) {
    const u32x4 w = __builtin_bit_cast(u32x4, x);
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = bf16lo(w[q]), hi = bf16hi(w[q]);
        r[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    return __builtin_bit_cast(f16x8, r);
}

// one packed dword of 8 codes -> fp16 B fragment (k in order), (c - z) * s:
// (1024 + c) - (1024 + z) is an exact small integer; with z = 8 it has at
// most 3 significant bits, so its product with a bf16 scale (8 bits) is exact
// in fp16.  Other zero points may round the product by half an fp16 ulp.
__device__ __forceinline__ f16x8 dequant_w4_f16(uint32_t w, f16x2 s2, f16x2 z2) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t t = ((w >> (4 * q)) & 0x000f000fu) | 0x64006400u;  // fp16 1024 + c
        const f16x2 v = (__builtin_bit_cast(f16x2, t) - z2) * s2;
        r[q] = __builtin_bit_cast(uint32_t, v);
    }
    return __builtin_bit_cast(f16x8, r);
}

constexpr int W4_BM = 128, W4_BN = 128, W4_MT = 4, W4_NT = 4;
constexpr int W4_A_STAGE = W4_BM * T_BK * 2;        // 8 KB
constexpr int W4_A_INSTR = W4_A_STAGE / 1024 / 4;   // 2 per wave per stage
constexpr int W4_B_GROUP = (W4_BN / 16) * 1024;     // 8 KB: 8 tiles x 64 lanes x 16 B
constexpr int W4_B_INSTR = W4_B_GROUP / 1024 / 4;   // 2 per wave per group
constexpr int W4_B_BASE = T_NS * W4_A_STAGE;        // 32 KB
constexpr int W4_S_BASE = W4_B_BASE + 2 * W4_B_GROUP;  // scales: 2 group buffers x 4 waves x 1 KB
constexpr int W4_S_GROUP = 4 * 1024;
constexpr int W4_LDS = W4_S_BASE + 2 * W4_S_GROUP;  // 56 KB

__global__ __attribute__((amdgpu_flat_work_group_size(T_THREADS, T_THREADS)))
void tile_w4_kernel(Problem p) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(AS3 void *)smem;
    const AS3 char *s3 = (const AS3 char *)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

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
    const int ngroups = p.K / 128;

    // A direct loads: [128][32] per stage, 16 rows x 4 chunks per instruction
    const int arow_l = lane >> 2;
    const int achunk = (lane & 3) ^ ((arow_l >> 1) & 3);
    uint32_t a_off[W4_A_INSTR];
#pragma unroll
    for (int q = 0; q < W4_A_INSTR; ++q)
        a_off[q] = (uint32_t)(((wave * W4_A_INSTR + q) * 16 + arow_l) * p.lda * 2) + achunk * 16;
    auto load_a = [&](int s) {
        const int k0 = s * T_BK;
        const i32x4 r = make_rsrc((const char *)p.A + ((int64_t)m0 * p.lda + k0) * 2,
                                  ((int64_t)(p.M - 1 - m0) * p.lda + (p.K - k0)) * 2);
        const bool kin = k0 + achunk * 8 < p.K;
        const uint32_t dst = lds0 + (s & (T_NS - 1)) * W4_A_STAGE + wave * W4_A_INSTR * 1024;
#pragma unroll
        for (int q = 0; q < W4_A_INSTR; ++q) load_lds16(r, dst + q * 1024, kin ? a_off[q] : OOB);
    };
    // B direct loads: group gi of the workgroup's 8 column tiles (1 KB per tile and group), and
    // the group's bf16 scales: wave w brings columns n0 + 32w .. n0 + 32w + 31 (lanes 0..3; the
    // other lanes read out of range and fill the rest of the wave's 1 KB slot with zeros).
    const i32x4 rb = make_rsrc(p.B, (int64_t)p.K * p.N / 2);
    const i32x4 rs = make_rsrc(p.scales, ((int64_t)(ngroups - 1) * p.ld_s + p.N) * 2);
    auto load_b = [&](int gi) {
        const bool gin = gi < ngroups;
        const uint32_t dst = lds0 + W4_B_BASE + (gi & 1) * W4_B_GROUP + wave * W4_B_INSTR * 1024;
#pragma unroll
        for (int q = 0; q < W4_B_INSTR; ++q) {
            const int nt = n0 / 16 + wave * W4_B_INSTR + q;
            const uint32_t off = (uint32_t)(((nt * ngroups + gi) * 64 + lane) * 16);
            load_lds16(rb, dst + q * 1024, gin ? off : OOB);
        }
        const uint32_t soff = (uint32_t)(((int64_t)gi * p.ld_s + n0 + wave * 32) * 2) + lane * 16;
        load_lds16(rs, lds0 + W4_S_BASE + (gi & 1) * W4_S_GROUP + wave * 1024, gin && lane < 4 ? soff : OOB);
    };

    const int frow = lane & 15, fgrp = lane >> 4;
    const int a_frag = swz_a(wm * 64 + frow, fgrp);
    const uint32_t b_raw = W4_B_BASE + (wn * W4_NT) * 1024 + lane * 16;  // + group buffer

    // fp16 scale pairs for this lane's 4 columns of one group (scale groups of 128 rows), from the
    // group's LDS buffer: column c of the tile sits in wave c / 32's slot at byte 2 (c % 32)
    auto scales_of = [&](int gb, f16x2 (&s2)[W4_NT]) {
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) {
            const int c = (wn * W4_NT + j) * 16 + frow;
            const uint16_t raw = *(const AS3 uint16_t *)(s3 + W4_S_BASE + gb * W4_S_GROUP + (c >> 5) * 1024 +
                                                         (c & 31) * 2);
            const _Float16 h = (_Float16)bf16_to_f32(raw);
            s2[j] = f16x2{h, h};
        }
    };
    const _Float16 zh = (_Float16)(1024.0f + (float)p.zero_point);
    const f16x2 z2 = f16x2{zh, zh};

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
    constexpr int LA = W4_A_INSTR, LB = W4_B_INSTR + 1;  // per wave: A loads per stage, B + scale loads per group

    // issue order: B(g0), A(0), A(1), A(2), A(3); then per stage s: A(s+4), and at the first stage
    // of a group also B(next group).  Waits below count the loads issued after the ones needed.
    load_b(0);
#pragma unroll
    for (int s = 0; s < T_NS; ++s) load_a(s);
    GE_WAIT_VM(3 * LA);  // A(0) and B(0) landed
    lds_barrier();

    bf16x8 fa[2][W4_MT];
    u32x4 braw[W4_NT], braw_n[W4_NT];  // this group's / the next group's packed codes
    f16x2 sc2[W4_NT], sc2_n[W4_NT];
#pragma unroll
    for (int i = 0; i < W4_MT; ++i) fa[0][i] = *(const AS3 bf16x8 *)(s3 + a_frag + i * 1024);
#pragma unroll
    for (int j = 0; j < W4_NT; ++j) braw[j] = *(const AS3 u32x4 *)(s3 + b_raw + j * 1024);
    scales_of(0, sc2);

    for (int gi = 0; gi < ngroups; ++gi) {
        const int gb = gi & 1;
#pragma unroll
        for (int b = 0; b < T_NS; ++b) {
            const int s = gi * T_NS + b;
            // stage s+1 (and at b == 3 the next group's B) must have landed
            if (b == 0) GE_WAIT_VM(2 * LA);
            else if (b == 3) GE_WAIT_VM(2 * LA);
            else GE_WAIT_VM(2 * LA + LB);
            lds_barrier();
            load_a(s + T_NS);
            if (b == 0) load_b(gi + 1);
            // next stage's fragments (the next group's raw B and scales at b == 3)
            const int sn = (b + 1) & (T_NS - 1);
#pragma unroll
            for (int i = 0; i < W4_MT; ++i)
                fa[(b + 1) & 1][i] = *(const AS3 bf16x8 *)(s3 + a_frag + sn * W4_A_STAGE + i * 1024);
            if (b == 3) {
#pragma unroll
                for (int j = 0; j < W4_NT; ++j)
                    braw_n[j] = *(const AS3 u32x4 *)(s3 + b_raw + (gb ^ 1) * W4_B_GROUP + j * 1024);
                scales_of(gb ^ 1, sc2_n);
            }
            // this stage
            f16x8 ah[W4_MT];
#pragma unroll
            for (int i = 0; i < W4_MT; ++i) ah[i] = bf16x8_to_f16x8(fa[b & 1][i]);
#pragma unroll
            for (int j = 0; j < W4_NT; ++j) {
                const f16x8 bh = dequant_w4_f16(braw[j][b], sc2[j], z2);
#pragma unroll
                for (int i = 0; i < W4_MT; ++i) mfma_f16_acc(acc[i][j], bh, ah[i]);
            }
        }
#pragma unroll
        for (int j = 0; j < W4_NT; ++j) {
            braw[j] = braw_n[j];
            sc2[j] = sc2_n[j];
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
    const int mbase = m0 + wm * 64 + frow;
    const int nbase = n0 + wn * 64 + fgrp * 4;
    auto small = [&](int64_t ld) { return ((int64_t)(p.M + 15) * ld + p.N) * 2 < (1ll << 31); };
    const bool all_bf16 = e.d_type == GE_BF16 && small(e.ldd) &&
                          (!(e.flags & GE_FLAG_C) || (e.c_type == GE_BF16 && small(e.ldc))) &&
                          (!(e.flags & GE_FLAG_RESIDUAL) || (e.r_type == GE_BF16 && small(e.ldr))) &&
                          (!(e.flags & GE_FLAG_BIAS) || e.bias_type == GE_BF16);
    with_act(e.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
        if (all_bf16) {
            if (e.flags & GE_FLAG_C)
                epilogue_bf16<ACT, true>(e, acc, p.M, p.N, mbase, n0 + wn * 64 + fgrp * 8);
            else
                epilogue_bf16<ACT, false>(e, acc, p.M, p.N, mbase, n0 + wn * 64 + fgrp * 8);
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

bool tile_w4_supported(const Problem &p) {
    if (p.mode != MODE_W4 || !p.w4_packed || p.M <= 16) return false;
    if ((p.N % W4_BN) || (p.K % 128) || (p.lda & 7) || !al16(p.A) || !al16(p.B)) return false;
    if (p.group != 128 || !al16(p.scales) || (p.ld_s & 7)) return false;
    if (((int64_t)(p.M - 1) * p.lda + p.K) * 2 >= (1ll << 31)) return false;
    if ((int64_t)p.K * p.N / 2 >= (1ll << 31) || (int64_t)p.K / 128 * p.ld_s * 2 >= (1ll << 31)) return false;
    return epi_ok(p);
}

const char *tile_w4_kernel_name() { return "tile_w4_f16_128x128x32"; }

hipError_t launch_tile_w4(const Problem &p, hipStream_t s) {
    if (!tile_w4_supported(p)) return hipErrorInvalidValue;
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)tile_w4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           W4_LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((p.M + W4_BM - 1) / W4_BM) * (p.N / W4_BN);
    hipLaunchKernelGGL(tile_w4_kernel, dim3(tiles), dim3(T_THREADS), W4_LDS, s, p);
    return hipGetLastError();
}

}  // namespace ge
