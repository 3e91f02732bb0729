// ge_general.hip -- the fallback tile kernel.
//
// Covers every request the planner accepts: any M, N, K >= 1, any leading
// dimension and alignment, fp32 or bf16 operands, B in KN or NK layout, the
// SwiGLU dual product and packed int4 weights.  Loads are element-wise with
// bounds checks, so ragged edges read zeros and nothing outside the matrices
// is touched.  It is the slow, simple path; the large-tile and skinny kernels
// take the shapes that matter for speed.
//
// Tile: 64 x 64 outputs per 256-thread workgroup, 32-deep K steps staged in
// LDS with the reduction index contiguous; four waves in a 2 x 2 grid, each
// owning 32 x 32 outputs = 2 x 2 MFMA tiles of 16 x 16.
//   bf16 operands -> v_mfma_f32_16x16x32_bf16
//   fp32 operands, and quantised weights -> v_mfma_f32_16x16x4f32 (the
//   weights dequantise exactly: (code - zero_point) * scale has at most 16
//   significant bits for 4- and 8-bit codes, fp8 value * scale at most 12,
//   so they are exact in fp32, and so are bf16 activations).

#include "ge_launch.hpp"

namespace ge {
namespace {

constexpr int GB_M = 64, GB_N = 64, GB_K = 32;
constexpr int G_THREADS = 256;

// element (k, n) of the second operand as fp32, zero outside the matrix
__device__ __forceinline__ float load_b(const Problem &p, const void *B, int k, int n) {
    if (k >= p.K || n >= p.N) return 0.0f;
    if (p.mode == MODE_W4) {
        const float s = bf16_to_f32(((const uint16_t *)p.scales)[(int64_t)(k / p.group) * p.ld_s + n]);
        if (p.wfmt != WFMT_U4) {  // one code per byte
            const uint8_t q = ((const uint8_t *)B)[(int64_t)k * p.ldb + n];
            return (p.wfmt == WFMT_U8 ? (float)((int)q - p.zero_point) : fp8e4m3_to_f32(q)) * s;
        }
        const uint8_t byte = ((const uint8_t *)B)[(int64_t)k * p.ldb + (n >> 1)];
        const bool even = (n & 1) == 0;
        const int code = (even != (p.lo_first != 0)) ? (byte >> 4) : (byte & 0xF);
        return (float)(code - p.zero_point) * s;
    }
    const int64_t off = p.b_layout == GE_LAYOUT_KN ? (int64_t)k * p.ldb + n : (int64_t)n * p.ldb + k;
    return load_elem(B, p.ab_type, off);
}

__device__ __forceinline__ float load_a(const Problem &p, int m, int k) {
    if (m >= p.M || k >= p.K) return 0.0f;
    return load_elem(p.A, p.ab_type, (int64_t)m * p.lda + k);
}

// USE_BF16: operands staged as bf16 and multiplied with the bf16 MFMA;
// otherwise staged as fp32 and multiplied with the fp32 MFMA.
template <bool USE_BF16, bool DUAL>
__global__ __launch_bounds__(G_THREADS) void general_kernel(Problem p) {
    constexpr int PADK = USE_BF16 ? GB_K + 8 : GB_K + 1;
    using S = typename std::conditional<USE_BF16, uint16_t, float>::type;
    __shared__ __attribute__((aligned(16))) S As[GB_M][PADK];
    __shared__ __attribute__((aligned(16))) S Bs[DUAL ? 2 : 1][GB_N][PADK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * GB_M, n0 = blockIdx.x * GB_N;

    f32x4 acc[2][2][2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[d][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the next K step's elements are loaded into registers while the current one is multiplied
    // (A: thread -> row tid/4, 8 consecutive k; B: thread -> k row tid/8, 8 consecutive n)
    constexpr int NBT = DUAL ? 2 : 1;
    const int ar = tid >> 2, akc = (tid & 3) * 8;
    const int bkr = tid >> 3, bnc = (tid & 7) * 8;
    float ra[8], rb[NBT][8];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ra[i] = load_a(p, m0 + ar, k0 + akc + i);
#pragma unroll
        for (int d = 0; d < NBT; ++d) {
            const void *B = d == 0 ? p.B : p.B2;
#pragma unroll
            for (int i = 0; i < 8; ++i) rb[d][i] = load_b(p, B, k0 + bkr, n0 + bnc + i);
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < p.K; k0 += GB_K) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (USE_BF16) As[ar][akc + i] = f32_to_bf16(ra[i]); else As[ar][akc + i] = ra[i];
        }
#pragma unroll
        for (int d = 0; d < NBT; ++d)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (USE_BF16) Bs[d][bnc + i][bkr] = f32_to_bf16(rb[d][i]); else Bs[d][bnc + i][bkr] = rb[d][i];
            }
        __syncthreads();
        if (k0 + GB_K < p.K) fetch(k0 + GB_K);

        if constexpr (USE_BF16) {
            const int kk = (lane >> 4) * 8;
            bf16x8 af[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *(const bf16x8 *)&As[wm * 32 + i * 16 + (lane & 15)][kk];
#pragma unroll
            for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16x8 bfr = *(const bf16x8 *)&Bs[d][wn * 32 + j * 16 + (lane & 15)][kk];
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[d][i][j] = mfma_bf16(af[i], bfr, acc[d][i][j]);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < GB_K; ks += 4) {
                const int kk = ks + (lane >> 4);
                float af[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) af[i] = As[wm * 32 + i * 16 + (lane & 15)][kk];
#pragma unroll
                for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float bv = Bs[d][wn * 32 + j * 16 + (lane & 15)][kk];
#pragma unroll
                        for (int i = 0; i < 2; ++i) acc[d][i][j] = mfma_f32(af[i], bv, acc[d][i][j]);
                    }
            }
        }
        __syncthreads();
    }

    // epilogue straight from the MFMA fragment layout, element by element
    const EpiArgs &e = p.epi;
    with_act(DUAL ? GE_ACT_NONE : e.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
                    const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                    if (m < p.M && n < p.N) {
                        float v;
                        if constexpr (DUAL) {
                            const float g = acc[0][i][j][r], u = acc[1][i][j][r];
                            v = activate<GE_ACT_SILU>(g) * u;
                        } else {
                            v = epi_scalar<ACT>(e, acc[0][i][j][r], m, n);
                        }
                        store_elem(e.D, e.d_type, (int64_t)m * e.ldd + n, v);
                    }
                }
    });
}

}  // namespace

hipError_t launch_general(const Problem &p, hipStream_t s) {
    const dim3 grid((p.N + GB_N - 1) / GB_N, (p.M + GB_M - 1) / GB_M);
    const bool bf16 = p.ab_type == GE_BF16 && p.mode != MODE_W4;
    const bool dual = p.mode == MODE_SWIGLU;
    if (bf16 && dual)
        hipLaunchKernelGGL((general_kernel<true, true>), grid, dim3(G_THREADS), 0, s, p);
    else if (bf16)
        hipLaunchKernelGGL((general_kernel<true, false>), grid, dim3(G_THREADS), 0, s, p);
    else if (dual)
        hipLaunchKernelGGL((general_kernel<false, true>), grid, dim3(G_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((general_kernel<false, false>), grid, dim3(G_THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace ge
