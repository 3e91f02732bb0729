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
// Weights: every 32-deep stage, each of the 256 threads dequantises 16 codes
// (one lane in each of two prepacked 16-column tiles) and writes them to LDS
// in MFMA fragment order, so every code is converted once per workgroup
// instead of once per wave that uses it.
//
// Pipeline, per stage s (unrolled by 8 = two 128-row scale groups): the fp16
// activations of stage s + 6 and (every fourth stage) the raw codes and
// scales of the group after next go straight to LDS by direct loads (their
// waits are counted by hand); the codes of stage s + 2 are dequantised into
// LDS buffer (s + 2) % 2; the fragments of stage s + 1 are read; the 16 MFMAs
// of stage s run on the fragments read one stage earlier.  The side work is
// spread between the MFMAs; one barrier per stage.
//
// Dequant per pair of codes: the codes are OR-ed into the mantissa of fp16
// 1024 (giving 1024 + c), then a packed subtract of 1024 + z and a packed
// multiply by s.
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

// one packed dword of 8 codes -> 8 fp16 weights (k in order), (c - z) * s
__device__ __forceinline__ u32x4 dequant_w4_f16(uint32_t w, f16x2 s2, f16x2 z2) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t t = ((w >> (4 * q)) & 0x000f000fu) | 0x64006400u;  // fp16 1024 + c
        const f16x2 v = (__builtin_bit_cast(f16x2, t) - z2) * s2;
        r[q] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
}

constexpr int W4_BM = 128, W4_BN = 128, W4_MT = 4, W4_NT = 4;
constexpr int W4_UNROLL = 8;                   // stages per loop trip (ring sizes divide it)
constexpr int W4_AD = 6;                       // activation loads run this many stages ahead
// LDS (bytes): fp16 activations, ring of 8 stages ([128][32] in the swizzled fragment layout); raw
// codes of two groups (prepacked blocks of the 8 tiles); raw scales of two groups (one 1 KB slot
// per wave, the wave's 32 columns in its first 64 bytes); dequantised fp16 B of two stages
constexpr int W4_A16 = 0, W4_A16_STAGE = W4_BM * 64;
constexpr int W4_RAWB = W4_A16 + W4_UNROLL * W4_A16_STAGE, W4_RAWB_GROUP = (W4_BN / 16) * 1024;
constexpr int W4_RAWS = W4_RAWB + 2 * W4_RAWB_GROUP, W4_RAWS_GROUP = 4 * 1024;
constexpr int W4_B16 = W4_RAWS + 2 * W4_RAWS_GROUP, W4_B16_STAGE = (W4_BN / 16) * 1024;
constexpr int W4_LDS = W4_B16 + 2 * W4_B16_STAGE;  // 104 KB

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

__global__ __attribute__((amdgpu_flat_work_group_size(T_THREADS, T_THREADS), amdgpu_waves_per_eu(1, 1)))
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
    const int ngroups = p.K / 128, nst = p.K / T_BK;

    // ---- direct loads (into LDS) ----
    // fp16 activations (dense [M][K] rows): wave w, instruction q -> rows 16 (2 w + q) + lane/4;
    // LDS slot lane % 4 of the row holds logical chunk (lane % 4) ^ ((row >> 1) & 3)
    const i32x4 rA = make_rsrc((const char *)p.A16 + (int64_t)m0 * p.K * 2, (int64_t)(p.M - m0) * p.K * 2);
    uint32_t a_src[W4_LA];
#pragma unroll
    for (int q = 0; q < W4_LA; ++q) {
        const int row_l = lane >> 2;
        const int chunk = (lane & 3) ^ ((row_l >> 1) & 3);
        a_src[q] = (uint32_t)(((wave * W4_LA + q) * 16 + row_l) * p.K * 2 + chunk * 16);
    }
    auto load_a = [&](int d, int slot) {  // stage d (runtime) into ring slot d % 8 (compile-time)
        const bool in = d < nst;
#pragma unroll
        for (int q = 0; q < W4_LA; ++q)
            load_lds16(rA, lds0 + W4_A16 + slot * W4_A16_STAGE + (wave * W4_LA + q) * 1024,
                       in ? a_src[q] + d * 64 : OOB);
    };
    // codes: wave w, instruction q -> tile 2 w + q (1 KB block of the group); scales: the wave's
    // 32 columns (lanes 0..3; the other lanes read zeros into the rest of its 1 KB slot)
    const i32x4 rB = make_rsrc(p.B, (int64_t)p.K * p.N / 2);
    const i32x4 rS = make_rsrc(p.scales, ((int64_t)(ngroups - 1) * p.ld_s + p.N) * 2);
    auto load_b = [&](int g, int slot) {  // group g into ring slot g % 2
        const bool in = g < ngroups;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = wave * 2 + q;
            load_lds16(rB, lds0 + W4_RAWB + slot * W4_RAWB_GROUP + tt * 1024,
                       in ? (uint32_t)((((int64_t)(n0 / 16 + tt) * ngroups + g) * 64 + lane) * 16) : OOB);
        }
        load_lds16(rS, lds0 + W4_RAWS + slot * W4_RAWS_GROUP + wave * 1024,
                   in && lane < 4 ? (uint32_t)(((int64_t)g * p.ld_s + n0 + wave * 32) * 2) + lane * 16 : OOB);
    };

    // ---- per-thread dequantisation: code blocks bi and bi + 256 (tile bi / 64, lane bi % 64);
    //      consecutive threads touch consecutive 16-byte LDS chunks, free of bank conflicts ----
    const int bi = tid;  // second block: bi + 256 (tile + 4, same lane)
    const int sc_col = (bi >> 6) * 16 + (bi & 15);  // second block: sc_col + 64
    const _Float16 zh = (_Float16)(1024.0f + (float)p.zero_point);
    const f16x2 z2 = f16x2{zh, zh};
    const uint32_t nib_mask = __builtin_amdgcn_readfirstlane(0x000f000fu);
    uint32_t f16_magic = 0x64006400u;
    asm volatile("" : "+v"(f16_magic));
    u32x4 craw[2];   // the two code blocks of the current group (read once per group)
    f16x2 cs2[2];    // their scales
    // dequantisation of one stage in 9 pieces, so that it can be spread between the MFMAs:
    // piece 0 reads the codes and scales at a group's first stage; pieces 1..8 dequantise one
    // code pair each (writing a lane fragment after every fourth)
    u32x4 dq_out;
    auto convert_piece = [&](int dd, int k) {  // stage d, dd = d % 8 (compile-time)
        const int buf = dd & 1, gs = (dd >> 2) & 1, q = dd & 3;
        AS3 char *w3 = (AS3 char *)smem;
        if (k == 0) {
            if (q == 0) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    craw[e] = *(const AS3 u32x4 *)(s3 + W4_RAWB + gs * W4_RAWB_GROUP + (bi + 256 * e) * 16);
                    const int col = sc_col + 64 * e;
                    const uint16_t sr =
                        *(const AS3 uint16_t *)(s3 + W4_RAWS + gs * W4_RAWS_GROUP + (col >> 5) * 1024 + (col & 31) * 2);
                    const _Float16 sh = (_Float16)bf16_to_f32(sr);
                    cs2[e] = f16x2{sh, sh};
                }
            }
        } else {
            const int e = (k - 1) >> 2, w = (k - 1) & 3;  // code block e, pair w
            // (empty asm ties on the piece's input and output keep it between its two MFMAs)
            uint32_t cin = craw[e][q];
            asm volatile("" : "+v"(cin));
            // fp16 1024 + c: (codes & 0x000f000f) | 0x64006400 in one v_and_or_b32 (VOP3 takes no
            // literals here, so the mask sits in an SGPR and the magic number in a VGPR)
            uint32_t tt;
            asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(tt) : "v"(w ? cin >> (4 * w) : cin), "s"(nib_mask), "v"(f16_magic));
            uint32_t o = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, tt) - z2) * cs2[e]);
            asm volatile("" : "+v"(o));
            dq_out[w] = o;
            if (w == 3) *(AS3 u32x4 *)(w3 + W4_B16 + buf * W4_B16_STAGE + (bi + 256 * e) * 16) = dq_out;
        }
    };
    auto convert = [&](int dd) {
#pragma unroll
        for (int k = 0; k <= 8; ++k) convert_piece(dd, k);
    };

    // ---- fragments ----
    const int frow = lane & 15, fgrp = lane >> 4;
    const int a_frag = W4_A16 + swz_a(wm * 64 + frow, fgrp);
    const int b_frag = W4_B16 + (wn * W4_NT * 64 + lane) * 16;
    f16x8 fa[2][W4_MT], fb[2][W4_NT];
    // read r of stage d (dd = d % 8): A and B fragments alternate; registers d % 2
    auto read_frag = [&](int dd, int r) {
        const int i = r >> 1, buf = dd & 1;
        if ((r & 1) == 0)
            fa[buf][i] = *(const AS3 f16x8 *)(s3 + a_frag + dd * W4_A16_STAGE + i * 1024);
        else
            fb[buf][i] = *(const AS3 f16x8 *)(s3 + b_frag + buf * W4_B16_STAGE + i * 1024);
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

    // prologue, in the order the loop would have issued it: activations of stage d at "stage" d - 6,
    // group 0 at -6 and group 1 at -2 (after that stage's activations)
    load_a(0, 0);
    load_b(0, 0);
    load_a(1, 1);
    load_a(2, 2);
    load_a(3, 3);
    load_a(4, 4);
    load_b(1, 1);
    load_a(5, 5);
    GE_WAIT_VM(4 * W4_LA + W4_LB);  // everything up to "stage" -5 (A0, B0, A1) landed
    lds_barrier();
    convert(0);
    convert(1);
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 2 * W4_MT; ++r) read_frag(0, r);

    // main loop, stage s = s0 + u: wait for the loads of stage s - 4 and earlier, barrier, then the
    // 16 MFMAs of stage s with, between them: the direct loads of stage s + 6 (and at u % 4 == 2 the
    // group after next), the dequantisation of stage s + 2 and the fragment reads of stage s + 1
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
            // side work after MFMA q: q = 0 direct loads and the code reads of the dequantisation,
            // q = 1..8 one fragment read each, q = 2..15 the dequantisation pieces
            const int dd = (u + 2) & (W4_UNROLL - 1);
#pragma unroll
            for (int q = 0; q < W4_MT * W4_NT; ++q) {
                const int i = q & (W4_MT - 1), j = q / W4_MT;
                mfma_f16_acc(acc[i][j], fb[u & 1][j], fa[u & 1][i]);
                asm volatile("" ::: "memory");
                if (q == 0) {
                    load_a(s + W4_AD, (u + W4_AD) & (W4_UNROLL - 1));
                    // s0 is a multiple of 8, so the ring slots are compile-time
                    if ((u & 3) == 2) load_b((s + 6) >> 2, ((u + 6) >> 2) & 1);
                    convert_piece(dd, 0);
                }
                if (q >= 1 && q <= 2 * W4_MT) read_frag((u + 1) & (W4_UNROLL - 1), q - 1);
#pragma unroll
                for (int k = 1; k <= 8; ++k)
                    if (q >= 2 && 2 + ((k - 1) * 14) / 8 == q) convert_piece(dd, k);
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
