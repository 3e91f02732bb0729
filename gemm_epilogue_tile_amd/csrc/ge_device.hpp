// ge_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// vector types, bf16 conversion, activations, the epilogue functor and the
// fragment layout of the 16x16 MFMA tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_epi.h"

namespace ge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// low / high bf16 half of a packed dword, widened exactly
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
// Race-guard build (-DGE_DEBUG_SYNC, libgemm_epi_debug.so): each pipeline stage of the tile
// kernels also waits for all of its wave's outstanding memory operations and meets a full
// workgroup barrier, and the cross-workgroup handoffs add device-scope fences.  The extra
// ordering can only remove races, never add them, so the normal build's outputs must equal the
// debug build's bit for bit; a difference points at a missing wait or barrier.
#ifdef GE_DEBUG_SYNC
#define GE_DEBUG_BARRIER()             \
    do {                               \
        __builtin_amdgcn_s_waitcnt(0); \
        __syncthreads();               \
    } while (0)
#define GE_DEBUG_FENCE() __threadfence()
#else
#define GE_DEBUG_BARRIER() \
    do {                   \
    } while (0)
#define GE_DEBUG_FENCE() \
    do {                 \
    } while (0)
#endif

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// One OCP fp8 E4M3 code (low byte of q) -> fp32, exactly (NaN codes give
// NaN).  The gfx950 conversion instruction implements this format; checked
// for all 256 codes against the format's definition.
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t q) { return __builtin_amdgcn_cvt_f32_fp8((int)q, 0); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// activations (fp32).  exp is taken as 2^(x log2 e) on the hardware exp2 unit;
// the reciprocal is the hardware one.  Identities used:
//   sigmoid(x) = 1 / (1 + e^-x)
//   silu(x)    = x * sigmoid(x)
//   gelu_tanh(x) = 0.5 x (1 + tanh(u)) = x * sigmoid(2u),
//                  u = sqrt(2/pi) (x + 0.044715 x^3)   (Hendrycks & Gimpel)
// For large |x| the exponential saturates to 0 or inf and the formulas return
// x or (-)0 as the limits require.
// ---------------------------------------------------------------------------

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;

__device__ __forceinline__ float fast_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <int ACT>
__device__ __forceinline__ float activate(float t) {
    if constexpr (ACT == GE_ACT_RELU) {
        return fmaxf(t, 0.0f);
    } else if constexpr (ACT == GE_ACT_GELU_TANH) {
        // -2u log2(e) = t (a + b t^2): one exponent argument in three operations
        constexpr float a = -2.0f * kSqrt2OverPi * kLog2e, b = a * kGeluCubic;
        const float arg = t * fmaf(b, t * t, a);
        return t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(arg));
    } else if constexpr (ACT == GE_ACT_SILU) {
        return t * fast_sigmoid(t);
    } else {
        return t;
    }
}

// ---------------------------------------------------------------------------
// epilogue parameters (passed by value to every kernel)
// ---------------------------------------------------------------------------

struct EpiArgs {
    float alpha, beta;
    const void *C;
    const void *bias;
    const void *R;
    void *D;
    int64_t ldc, ldr, ldd;
    int32_t c_type, bias_type, r_type, d_type;
    int32_t act;
    uint32_t flags;  // GE_FLAG_BIAS / GE_FLAG_C (only when beta != 0) / GE_FLAG_RESIDUAL
};

__device__ __forceinline__ float load_elem(const void *p, int32_t type, int64_t i) {
    return type == GE_BF16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

__device__ __forceinline__ void store_elem(void *p, int32_t type, int64_t i, float v) {
    if (type == GE_BF16)
        ((uint16_t *)p)[i] = f32_to_bf16(v);
    else
        ((float *)p)[i] = v;
}

// one element of the epilogue: act(alpha*acc + beta*C + bias) + R
template <int ACT>
__device__ __forceinline__ float epi_scalar(const EpiArgs &e, float acc, int64_t m, int64_t n) {
    float t = e.alpha * acc;
    if (e.flags & GE_FLAG_C) t = fmaf(e.beta, load_elem(e.C, e.c_type, m * e.ldc + n), t);
    if (e.flags & GE_FLAG_BIAS) t += load_elem(e.bias, e.bias_type, n);
    float u = activate<ACT>(t);
    if (e.flags & GE_FLAG_RESIDUAL) u += load_elem(e.R, e.r_type, m * e.ldr + n);
    return u;
}

// Load 8 consecutive elements (columns n..n+7 of row m) of a bf16 or fp32
// matrix as fp32.  Requires 16-byte alignment of the chunk.
__device__ __forceinline__ void load8(const void *p, int32_t type, int64_t off, float v[8]) {
    if (type == GE_BF16) {
        const u32x4 w = *(const u32x4 *)((const uint16_t *)p + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16lo(w[i]);
            v[2 * i + 1] = bf16hi(w[i]);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)p + off);
        const f32x4 b = *(const f32x4 *)((const float *)p + off + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    }
}

__device__ __forceinline__ void store8(void *p, int32_t type, int64_t off, const float v[8]) {
    if (type == GE_BF16) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        *(u32x4 *)((uint16_t *)p + off) = w;
    } else {
        f32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = v[i];
            b[i] = v[4 + i];
        }
        *(f32x4 *)((float *)p + off) = a;
        *(f32x4 *)((float *)p + off + 4) = b;
    }
}

// Epilogue on 8 consecutive columns n..n+7 of row m (all in bounds, 16-byte
// aligned chunks).  acc holds the fp32 accumulators; the result goes to D.
template <int ACT>
__device__ __forceinline__ void epi_row8(const EpiArgs &e, const float acc[8], int64_t m, int64_t n) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = e.alpha * acc[i];
    if (e.flags & GE_FLAG_C) {
        float c[8];
        load8(e.C, e.c_type, m * e.ldc + n, c);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = fmaf(e.beta, c[i], t[i]);
    }
    if (e.flags & GE_FLAG_BIAS) {
        float b[8];
        load8(e.bias, e.bias_type, n, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] += b[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = activate<ACT>(t[i]);
    if (e.flags & GE_FLAG_RESIDUAL) {
        float r[8];
        load8(e.R, e.r_type, m * e.ldr + n, r);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] += r[i];
    }
    store8(e.D, e.d_type, m * e.ldd + n, t);
}

// Dispatch a functor templated on the activation.
template <typename F>
__device__ __forceinline__ void with_act(int32_t act, F &&f) {
    switch (act) {
    case GE_ACT_RELU: f(std::integral_constant<int, GE_ACT_RELU>{}); break;
    case GE_ACT_GELU_TANH: f(std::integral_constant<int, GE_ACT_GELU_TANH>{}); break;
    case GE_ACT_SILU: f(std::integral_constant<int, GE_ACT_SILU>{}); break;
    default: f(std::integral_constant<int, GE_ACT_NONE>{}); break;
    }
}

// ---------------------------------------------------------------------------
// MFMA wrappers.  Output fragment of a 16x16 tile (both instructions):
// lane l, element j holds row 4*(l/16) + j, column l % 16.
// bf16 16x16x32: lane l supplies row (A) / column (B) l % 16 and 8 values of
// the reduction index from group l / 16; A and B use the same assignment, so
// any fixed map from (group, element) to k gives the same sum.
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// In-place form for hot loops: the accumulator is tied to the destination in
// AGPRs, so it never moves between registers from one step to the next (the
// builtin form lets the register allocator rotate accumulators through
// copies, which halves the MFMA issue rate of a lone wave).  The hazard
// between the last MFMA and a later read of the accumulator is covered by
// mfma_drain().
__device__ __forceinline__ void mfma_bf16_acc(f32x4 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states after the last in-place MFMA before its accumulators are read.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::); }
// fp32 16x16x4: lane l supplies row / column l % 16 at reduction index l / 16.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace ge
