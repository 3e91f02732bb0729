// ge_general.hip -- the fallback tile kernel.
//
// Covers every request the planner accepts: any M, N, K >= 1, any leading
// dimension and alignment, fp32 or bf16 operands, B in KN or NK layout, the
// SwiGLU dual product and packed int4 weights.  Loads are element-wise; an
// element outside the matrix is read as zero (its address clamped to element
// 0, so nothing outside the matrices is touched and no load waits on a
// branch).  It is the slow, simple path; the large-tile and skinny kernels
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

// Raw bits of element i of a bf16 (T = uint16_t, zero-extended) or fp32 (T = float) array, with
// the index clamped to 0 when !ok (every operand has an element 0), so the load is unconditional.
// The bits are turned into a value (and zeroed when out of range) only where they are used, so a
// thread's loads stay in flight together until then.
template <typename T>
__device__ __forceinline__ uint32_t ld_raw(const void *p, int64_t i, bool ok) {
    const int64_t j = ok ? i : 0;
    if constexpr (std::is_same<T, uint16_t>::value)
        return ((const uint16_t *)p)[j];
    else
        return __builtin_bit_cast(uint32_t, ((const float *)p)[j]);
}
__device__ __forceinline__ float raw_value(uint32_t bits, bool bf16, bool ok) {
    const float v = bf16 ? __builtin_bit_cast(float, bits << 16) : __builtin_bit_cast(float, bits);
    return ok ? v : 0.0f;
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

    // K steps are fetched into registers two ahead of the step being multiplied, as raw bits with
    // an in-range mask (bit i: A element i; bit 8 + 8 d + i: element i of B operand d)
    // (A: thread -> row tid/4, 8 consecutive k; B: thread -> k row tid/8, 8 consecutive n)
    constexpr int NBT = DUAL ? 2 : 1;
    const int ar = tid >> 2, akc = (tid & 3) * 8;
    const int bkr = tid >> 3, bnc = (tid & 7) * 8;
    const bool quant = p.mode == MODE_W4, a16 = p.ab_type == GE_BF16;
    const bool kn = p.b_layout == GE_LAYOUT_KN;
    uint32_t ra[2][8], rb[2][NBT][8], rsc[2][8], okm[2];
    auto fetch = [&](int k0, auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        uint32_t mask = 0;
        auto fetch_a = [&](auto tag) {
            using T = decltype(tag);
            const int m = m0 + ar;
            const int64_t row = (int64_t)m * p.lda;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = k0 + akc + i;
                const bool ok = m < p.M && k < p.K;
                mask |= (uint32_t)ok << i;
                ra[sl][i] = ld_raw<T>(p.A, row + k, ok);
            }
        };
        auto fetch_b = [&](auto tag) {
            using T = decltype(tag);
            const int k = k0 + bkr;
#pragma unroll
            for (int d = 0; d < NBT; ++d) {
                const void *B = d == 0 ? p.B : p.B2;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int n = n0 + bnc + i;
                    const bool ok = k < p.K && n < p.N;
                    mask |= (uint32_t)ok << (8 + 8 * d + i);
                    rb[sl][d][i] = ld_raw<T>(B, kn ? (int64_t)k * p.ldb + n : (int64_t)n * p.ldb + k, ok);
                }
            }
        };
        // quantised weights: the code byte and the bf16 scale of each element
        auto fetch_q = [&]() {
            const int k = k0 + bkr;
            const bool kok = k < p.K;
            const int64_t srow = (int64_t)((kok ? k : 0) / p.group) * p.ld_s;
            const int64_t crow = (int64_t)(kok ? k : 0) * p.ldb;
            const bool u4 = p.wfmt == WFMT_U4;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int n = n0 + bnc + i;
                const bool ok = kok && n < p.N;
                const int nn = ok ? n : 0;
                mask |= (uint32_t)ok << (8 + i);
                rsc[sl][i] = ((const uint16_t *)p.scales)[srow + nn];
                rb[sl][0][i] = ((const uint8_t *)p.B)[crow + (u4 ? nn >> 1 : nn)];
            }
        };
        if (a16) fetch_a(uint16_t{}); else fetch_a(float{});
        if constexpr (!DUAL && !USE_BF16) {  // (quantised weights: never dual, staged as fp32)
            if (quant) {
                fetch_q();
                okm[sl] = mask;
                return;
            }
        }
        if (a16) fetch_b(uint16_t{}); else fetch_b(float{});
        okm[sl] = mask;
    };
    // registers of a slot -> LDS values: zero out of range; quantised weights decoded,
    // (code - zero_point) * scale or fp8 value * scale, exact in fp32
    auto commit = [&](auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        const uint32_t mask = okm[sl];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = (mask >> i) & 1;
            if constexpr (USE_BF16) As[ar][akc + i] = ok ? (uint16_t)ra[sl][i] : (uint16_t)0;
            else As[ar][akc + i] = raw_value(ra[sl][i], a16, ok);
        }
        if constexpr (USE_BF16) {
#pragma unroll
            for (int d = 0; d < NBT; ++d)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const bool ok = (mask >> (8 + 8 * d + i)) & 1;
                    Bs[d][bnc + i][bkr] = ok ? (uint16_t)rb[sl][d][i] : (uint16_t)0;
                }
        } else if (!DUAL && quant) {
            const bool u4 = p.wfmt == WFMT_U4, u8 = p.wfmt == WFMT_U8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = (mask >> (8 + i)) & 1;
                const uint32_t byte = rb[sl][0][i];
                float w;
                if (u4) {
                    // column n0 + bnc + i: its parity is that of i
                    const bool even = (i & 1) == 0;
                    const int code = (even != (p.lo_first != 0)) ? (int)(byte >> 4) : (int)(byte & 0xF);
                    w = (float)(code - p.zero_point);
                } else {
                    w = u8 ? (float)((int)byte - p.zero_point) : fp8e4m3_to_f32(byte);
                }
                Bs[0][bnc + i][bkr] = ok ? w * bf16_to_f32((uint16_t)rsc[sl][i]) : 0.0f;
            }
        } else {
#pragma unroll
            for (int d = 0; d < NBT; ++d)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const bool ok = (mask >> (8 + 8 * d + i)) & 1;
                    Bs[d][bnc + i][bkr] = raw_value(rb[sl][d][i], a16, ok);
                }
        }
    };

    // one K step: registers -> LDS, the step two ahead into the same registers, the MFMAs
    auto step = [&](int k0, auto SLOT) {
        commit(SLOT);
        __syncthreads();
        if (k0 + 2 * GB_K < p.K) fetch(k0 + 2 * GB_K, SLOT);

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
    };

    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    fetch(0, Slot0{});
    if (GB_K < p.K) fetch(GB_K, Slot1{});
    for (int k0 = 0; k0 < p.K; k0 += 2 * GB_K) {
        step(k0, Slot0{});
        if (k0 + GB_K < p.K) step(k0 + GB_K, Slot1{});
    }

    // epilogue from the MFMA fragment layout: lane l, element r of tile (i, j) is row
    // 16 i + 4 (l / 16) + r, column 16 j + l % 16 of the wave's 32 x 32.  Every operand the
    // epilogue reads is requested first (branch-free), then each element is finished and stored.
    const EpiArgs &e = p.epi;
    const bool hc = !DUAL && (e.flags & GE_FLAG_C), hb = !DUAL && (e.flags & GE_FLAG_BIAS);
    const bool hr = !DUAL && (e.flags & GE_FLAG_RESIDUAL);
    auto row_of = [&](int i, int r) { return m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r; };
    auto col_of = [&](int j) { return n0 + wn * 32 + j * 16 + (lane & 15); };
    uint32_t cv[2][2][4], rv[2][2][4], bv[2], em = 0;  // raw bits; em bit 4 (2 i + j) + r: in range
    auto load_mat = [&](auto tag, const void *P, int64_t ld, uint32_t (&out)[2][2][4]) {
        using T = decltype(tag);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = row_of(i, r), n = col_of(j);
                    out[i][j][r] = ld_raw<T>(P, (int64_t)m * ld + n, m < p.M && n < p.N);
                }
    };
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) em |= (uint32_t)(row_of(i, r) < p.M && col_of(j) < p.N) << (8 * i + 4 * j + r);
    if (hc) {
        if (e.c_type == GE_BF16) load_mat(uint16_t{}, e.C, e.ldc, cv); else load_mat(float{}, e.C, e.ldc, cv);
    }
    if (hr) {
        if (e.r_type == GE_BF16) load_mat(uint16_t{}, e.R, e.ldr, rv); else load_mat(float{}, e.R, e.ldr, rv);
    }
    if (hb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = col_of(j);
            bv[j] = e.bias_type == GE_BF16 ? ld_raw<uint16_t>(e.bias, n, n < p.N) : ld_raw<float>(e.bias, n, n < p.N);
        }
    }
    with_act(DUAL ? GE_ACT_NONE : e.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = row_of(i, r), n = col_of(j);
                    if ((em >> (8 * i + 4 * j + r)) & 1) {
                        float v;
                        if constexpr (DUAL) {
                            const float g = acc[0][i][j][r], u = acc[1][i][j][r];
                            v = activate<GE_ACT_SILU>(g) * u;
                        } else {
                            // act(alpha acc + beta C + bias) + R, in that order
                            float t = e.alpha * acc[0][i][j][r];
                            if (hc) t = fmaf(e.beta, raw_value(cv[i][j][r], e.c_type == GE_BF16, true), t);
                            if (hb) t += raw_value(bv[j], e.bias_type == GE_BF16, true);
                            v = activate<ACT>(t);
                            if (hr) v += raw_value(rv[i][j][r], e.r_type == GE_BF16, true);
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
