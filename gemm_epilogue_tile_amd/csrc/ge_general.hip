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
// Tile: T x T outputs per 256-thread workgroup (T = 64, or 32 when 64 x 64
// tiles would leave most CUs idle), 32-deep K steps staged in LDS with the
// reduction index contiguous; four waves in a 2 x 2 grid, each owning
// T/2 x T/2 outputs = MFMA tiles of 16 x 16.
//   bf16 operands -> v_mfma_f32_16x16x32_bf16
//   fp32 operands, and quantised weights -> v_mfma_f32_16x16x4f32 (the
//   weights dequantise exactly: (code - zero_point) * scale has at most 16
//   significant bits for 4- and 8-bit codes, fp8 value * scale at most 12,
//   so they are exact in fp32, and so are bf16 activations).

#include "ge_launch.hpp"

namespace ge {
namespace {

constexpr int GB_K = 32;
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
template <bool USE_BF16, bool DUAL, int T>
__global__ __launch_bounds__(G_THREADS) void general_kernel(Problem p) {
    static_assert(T == 32 || T == 64, "tile size");
    constexpr int PADK = USE_BF16 ? GB_K + 8 : GB_K + 1;
    constexpr int W = T / 2, MT = W / 16;  // wave tile W x W, MT x MT MFMA tiles
    constexpr int E = T / 8;               // A and B elements per thread per K step
    using S = typename std::conditional<USE_BF16, uint16_t, float>::type;
    __shared__ __attribute__((aligned(16))) S As[T][PADK];
    __shared__ __attribute__((aligned(16))) S Bs[DUAL ? 2 : 1][T][PADK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;

    f32x4 acc[2][MT][MT];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j) acc[d][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The epilogue's operands (C, R, bias) do not depend on the product: they are requested
    // first, so their latency overlaps the K loop.  Fragment layout: lane l, element r of tile
    // (i, j) is row 16 i + 4 (l / 16) + r, column 16 j + l % 16 of the wave's W x W.
    const EpiArgs &e = p.epi;
    const bool hc = !DUAL && (e.flags & GE_FLAG_C), hb = !DUAL && (e.flags & GE_FLAG_BIAS);
    const bool hr = !DUAL && (e.flags & GE_FLAG_RESIDUAL);
    auto row_of = [&](int i, int r) { return m0 + wm * W + i * 16 + (lane >> 4) * 4 + r; };
    auto col_of = [&](int j) { return n0 + wn * W + j * 16 + (lane & 15); };
    // raw bits; em bit 4 (MT i + j) + r: output in range
    uint32_t cv[MT][MT][4], rv[MT][MT][4], bv[MT], em = 0;
    auto load_mat = [&](auto tag, const void *P, int64_t ld, uint32_t (&out)[MT][MT][4]) {
        using TT = decltype(tag);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = row_of(i, r), n = col_of(j);
                    out[i][j][r] = ld_raw<TT>(P, (int64_t)m * ld + n, m < p.M && n < p.N);
                }
    };
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                em |= (uint32_t)(row_of(i, r) < p.M && col_of(j) < p.N) << (4 * (MT * i + j) + r);
    if (hc) {
        if (e.c_type == GE_BF16) load_mat(uint16_t{}, e.C, e.ldc, cv); else load_mat(float{}, e.C, e.ldc, cv);
    }
    if (hr) {
        if (e.r_type == GE_BF16) load_mat(uint16_t{}, e.R, e.ldr, rv); else load_mat(float{}, e.R, e.ldr, rv);
    }
    if (hb) {
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int n = col_of(j);
            bv[j] = e.bias_type == GE_BF16 ? ld_raw<uint16_t>(e.bias, n, n < p.N) : ld_raw<float>(e.bias, n, n < p.N);
        }
    }

    // K steps are fetched into registers two ahead of the step being multiplied, as raw bits with
    // an in-range mask (bit i: A element i; bit 8 + 8 d + i: element i of B operand d)
    // (A: thread -> one row, E consecutive k; B: thread -> k row tid / 8, E consecutive n)
    constexpr int NBT = DUAL ? 2 : 1;
    const int ar = tid / (GB_K / E), akc = (tid % (GB_K / E)) * E;
    const int bkr = tid >> 3, bnc = (tid & 7) * E;
    const bool quant = p.mode == MODE_W4, a16 = p.ab_type == GE_BF16;
    const bool kn = p.b_layout == GE_LAYOUT_KN;
    uint32_t ra[2][E], rb[2][NBT][E], rsc[2][E], okm[2];
    auto fetch = [&](int k0, auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        uint32_t mask = 0;
        auto fetch_a = [&](auto tag) {
            using ET = decltype(tag);
            const int m = m0 + ar;
            const int64_t row = (int64_t)m * p.lda;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const int k = k0 + akc + i;
                const bool ok = m < p.M && k < p.K;
                mask |= (uint32_t)ok << i;
                ra[sl][i] = ld_raw<ET>(p.A, row + k, ok);
            }
        };
        auto fetch_b = [&](auto tag) {
            using ET = decltype(tag);
            const int k = k0 + bkr;
#pragma unroll
            for (int d = 0; d < NBT; ++d) {
                const void *B = d == 0 ? p.B : p.B2;
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const int n = n0 + bnc + i;
                    const bool ok = k < p.K && n < p.N;
                    mask |= (uint32_t)ok << (8 + 8 * d + i);
                    rb[sl][d][i] = ld_raw<ET>(B, kn ? (int64_t)k * p.ldb + n : (int64_t)n * p.ldb + k, ok);
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
            for (int i = 0; i < E; ++i) {
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
        for (int i = 0; i < E; ++i) {
            const bool ok = (mask >> i) & 1;
            if constexpr (USE_BF16) As[ar][akc + i] = ok ? (uint16_t)ra[sl][i] : (uint16_t)0;
            else As[ar][akc + i] = raw_value(ra[sl][i], a16, ok);
        }
        if constexpr (USE_BF16) {
#pragma unroll
            for (int d = 0; d < NBT; ++d)
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const bool ok = (mask >> (8 + 8 * d + i)) & 1;
                    Bs[d][bnc + i][bkr] = ok ? (uint16_t)rb[sl][d][i] : (uint16_t)0;
                }
        } else if (!DUAL && quant) {
            const bool u4 = p.wfmt == WFMT_U4, u8 = p.wfmt == WFMT_U8;
#pragma unroll
            for (int i = 0; i < E; ++i) {
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
                for (int i = 0; i < E; ++i) {
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
            bf16x8 af[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = *(const bf16x8 *)&As[wm * W + i * 16 + (lane & 15)][kk];
#pragma unroll
            for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const bf16x8 bfr = *(const bf16x8 *)&Bs[d][wn * W + j * 16 + (lane & 15)][kk];
#pragma unroll
                    for (int i = 0; i < MT; ++i) acc[d][i][j] = mfma_bf16(af[i], bfr, acc[d][i][j]);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < GB_K; ks += 4) {
                const int kk = ks + (lane >> 4);
                float af[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i) af[i] = As[wm * W + i * 16 + (lane & 15)][kk];
#pragma unroll
                for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
                    for (int j = 0; j < MT; ++j) {
                        const float bf = Bs[d][wn * W + j * 16 + (lane & 15)][kk];
#pragma unroll
                        for (int i = 0; i < MT; ++i) acc[d][i][j] = mfma_f32(af[i], bf, acc[d][i][j]);
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

    // epilogue: each in-range element finished in fp32 and stored
    with_act(DUAL ? GE_ACT_NONE : e.act, [&](auto ACTC) {
        constexpr int ACT = decltype(ACTC)::value;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = row_of(i, r), n = col_of(j);
                    if ((em >> (4 * (MT * i + j) + r)) & 1) {
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

// 32 x 32 tiles when 64 x 64 ones would fill fewer than half the CUs (small problems: four times
// the workgroups, each a quarter of the MFMA work per K step), 64 x 64 otherwise
int general_tile(const Problem &p, int cu_count) {
    const int64_t tiles64 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    return 2 * tiles64 < cu_count ? 32 : 64;
}

const char *general_kernel_name(const Problem &p, int cu_count) {
    return general_tile(p, cu_count) == 32 ? "general_32x32" : "general_64x64";
}

template <int T>
static hipError_t launch_general_t(const Problem &p, hipStream_t s) {
    const dim3 grid((p.N + T - 1) / T, (p.M + T - 1) / T);
    const bool bf16 = p.ab_type == GE_BF16 && p.mode != MODE_W4;
    const bool dual = p.mode == MODE_SWIGLU;
    if (bf16 && dual)
        hipLaunchKernelGGL((general_kernel<true, true, T>), grid, dim3(G_THREADS), 0, s, p);
    else if (bf16)
        hipLaunchKernelGGL((general_kernel<true, false, T>), grid, dim3(G_THREADS), 0, s, p);
    else if (dual)
        hipLaunchKernelGGL((general_kernel<false, true, T>), grid, dim3(G_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((general_kernel<false, false, T>), grid, dim3(G_THREADS), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_general(const Problem &p, int cu_count, hipStream_t s) {
    return general_tile(p, cu_count) == 32 ? launch_general_t<32>(p, s) : launch_general_t<64>(p, s);
}

}  // namespace ge
