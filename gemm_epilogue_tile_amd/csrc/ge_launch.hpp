// ge_launch.hpp -- internal interface between the host planner (ge_api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ge_device.hpp"

namespace ge {

enum Mode : int32_t { MODE_GENERIC = 0, MODE_SWIGLU = 1, MODE_W4 = 2 };
enum WFmt : int32_t { WFMT_U4 = 0, WFMT_U8 = 1, WFMT_FP8 = 2 };

// Prepacked int4 layout (gemm_w4_prepack): 128-column blocks (outer), 128-row
// groups, then the block's 16-column tiles (inner), one 1 KiB fragment each
// (64 lanes x 16 bytes); the last block of a width that is not a multiple of
// 128 holds the remaining tiles.  A block's groups are thus one contiguous run,
// and its eight tiles of one group are 8 KiB in a row.  Byte offset of the
// fragment of tile t, group g:
constexpr int W4P_BLOCK_TILES = 8;
__host__ __device__ inline int64_t w4p_frag_offset(int64_t t, int64_t g, int64_t ngroups, int64_t ntiles) {
    const int64_t b = t / W4P_BLOCK_TILES;
    const int64_t ntb = ntiles - W4P_BLOCK_TILES * b < W4P_BLOCK_TILES ? ntiles - W4P_BLOCK_TILES * b : W4P_BLOCK_TILES;
    return (b * ngroups * W4P_BLOCK_TILES + g * ntb + t % W4P_BLOCK_TILES) * 1024;
}

// A fully described product + epilogue, pointers included.
struct Problem {
    int32_t M, N, K;
    int32_t mode;       // Mode
    int32_t ab_type;    // GE_F32 / GE_BF16 storage of A (and of dense B)
    int32_t b_layout;   // GE_LAYOUT_KN / GE_LAYOUT_NK (dense B only)
    const void *A;
    const void *B;      // dense B, Wg (swiglu) or Wq (w4)
    const void *B2;     // Wu (swiglu)
    const void *scales; // w4 scales (bf16)
    int64_t lda, ldb, ld_s;
    int32_t group, zero_point, lo_first;
    int32_t w4_packed;  // B holds int4 weights in the prepacked layout
    int32_t b_packed;   // B holds bf16 weights in the prepacked decode layout (gemm_b_prepack)
    int32_t wfmt;       // MODE_W4 code format: WFMT_U4 (packed pairs), WFMT_U8, WFMT_FP8
    // cross-workgroup K split of the 8-bit streaming kernel (split > 1): fp32
    // tiles and per-column-block arrival counters, owned by the plan
    int32_t split;
    float *split_ws;
    uint32_t *split_cnt;
    EpiArgs epi;
};

// Fallback tile kernel: any shape, stride and alignment.
hipError_t launch_general(const Problem &p, int cu_count, hipStream_t s);
int general_tile(const Problem &p, int cu_count);  // 32 or 64
const char *general_kernel_name(const Problem &p, int cu_count);

// Large-tile bf16 MFMA kernel (M large).  Returns hipErrorInvalidValue when
// the problem does not meet its preconditions (see tile_supported()).
bool tile_supported(const Problem &p);
hipError_t launch_tile(const Problem &p, int cu_count, hipStream_t s);
const char *tile_kernel_name(const Problem &p, int cu_count);

// Quantised-weight tile kernel (prepacked int4 with M > 32, or raw 8-bit codes with M > 16),
// dispatched through launch_tile.
bool tile_w4_supported(const Problem &p);
hipError_t launch_tile_w4(const Problem &p, int cu_count, hipStream_t s);
const char *tile_w4_kernel_name(const Problem &p, int cu_count);

// K split of the quantised tile kernel when its tiles do not fill the CUs (1: none), the scratch
// bytes it needs (partial tiles, then one counter per tile that must start at zero; the kernel
// re-arms them) and the number of those counters.  The kernel runs split when p.split > 1 with
// p.split_ws / p.split_cnt set.
int tile_w4_split(const Problem &p, int cu_count);
int64_t tile_w4_split_scratch_bytes(const Problem &p, int split);
int tile_w4_split_counters(const Problem &p);

// One-time conversion of raw [K, N/2] int4 weights to the prepacked layout.
hipError_t launch_w4_prepack(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq, int32_t lo_first, uint8_t *Wp,
                             hipStream_t s);

// One-time conversion of raw [K, N] 8-bit codes to the prepacked decode layout.
hipError_t launch_w8_prepack(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq, uint8_t *Wp, hipStream_t s);

// One-time conversion of raw [K, N] bf16 weights to the prepacked decode layout.
hipError_t launch_b_prepack(int32_t K, int32_t N, const uint16_t *B, int64_t ldb, uint16_t *Bp, int cu_count,
                            hipStream_t s, int tb_override = 0);
// SwiGLU on prepacked weights (M <= 32): gate and up column blocks on workgroup pairs; the block
// width (the layout gemm_b_prepack writes for a SwiGLU plan), the plan scratch (the pairs' fp32
// tiles, then one counter per block) and the kernel's name
int swiglu_block_tiles(int N, int cu_count);
int64_t swiglu_prepacked_scratch_bytes(int M, int N, int cu_count);
const char *swiglu_prepacked_name(int N, int cu_count);
hipError_t launch_swiglu_prepacked(const Problem &p, int cu_count, hipStream_t s);
// the same pairs on raw [K, N] weights (M <= 32, when the raw decode kernel takes both weights)
bool swiglu_raw_supported(const Problem &p);
int64_t swiglu_raw_scratch_bytes(int M, int N, int cu_count);
const char *swiglu_raw_name(int N, int cu_count);
int64_t swiglu_pair_blocks(int N, int cu_count, bool prepacked);  // column blocks (one counter each)
hipError_t launch_swiglu_raw(const Problem &p, int cu_count, hipStream_t s);
// 16-column tiles per block of the prepacked bf16 layout (7 or 8), a function of N and the CU count
int bf16p_block_tiles(int N, int cu_count);

// Rotary position embedding at Q / K tile load, with the scores product as the consumer.
struct RopeArgs {
    int32_t batch, Sq, Sk, D;
    int32_t q_pos0, k_pos0;
    const uint16_t *Q, *K;      // [batch][Sq][D], [batch][Sk][D] bf16
    const float *cos, *sin;     // [positions][D / 2]; NULL: no rotation
    float alpha;
    void *S;                    // [batch][Sq][Sk], fp32 or bf16
};
// exact: each rotated coordinate is the exact rotation rounded once (else fp32 with one fused
// multiply-add, within one bf16 unit of it)
hipError_t launch_rope_qk(const RopeArgs &a, bool interleaved, bool f32out, bool exact, hipStream_t s);
// The rotation alone (the unfused chain's first step): X [batch * S][D] -> Y.
hipError_t launch_rope(int32_t batch, int32_t S, int32_t D, const uint16_t *X, const float *cosT, const float *sinT,
                       int32_t pos0, bool interleaved, bool exact, uint16_t *Y, hipStream_t s);

// Small-M weight-streaming kernel (decode shapes).
bool skinny_supported(const Problem &p);
hipError_t launch_skinny(const Problem &p, int cu_count, hipStream_t s);
// scratch: the plan may own device scratch (false: the variants that need none)
const char *skinny_kernel_name(const Problem &p, int cu_count, bool scratch = true);
// K splits of the 8-bit and the 128-column int4 streaming kernels and the
// scratch bytes they need (tiles, then counters that must start at zero; the
// kernel re-arms them).
int w8_split(const Problem &p, int cu_count);
int64_t w8_split_scratch_bytes(const Problem &p, int split);
// counters (column blocks) at the end of that scratch
int split_counters(const Problem &p);
// Stream-K bf16 decode kernel: tile slots per column block (0: the plain kernel) and the
// scratch bytes they need (tiles, then counters that must start at zero).  It is launched
// when p.split > 1 with p.split_ws / p.split_cnt set, on cu_count workgroups.
int bf16_sk_slots(const Problem &p, int cu_count);
int64_t bf16_sk_scratch_bytes(const Problem &p, int slots);

// Elementwise kernels of the unfused chain.  All tensors dense [M, N] of the
// given storage type unless noted.
hipError_t launch_ew_axpby(int64_t M, int64_t N, float alpha, const void *X, int32_t x_type,
                           float beta, const void *C, int32_t c_type, int64_t ldc, void *Y,
                           int32_t y_type, hipStream_t s);
hipError_t launch_ew_bias(int64_t M, int64_t N, const void *X, int32_t x_type, const void *bias,
                          int32_t bias_type, void *Y, int32_t y_type, hipStream_t s);
hipError_t launch_ew_act(int64_t M, int64_t N, int32_t act, const void *X, int32_t x_type, void *Y,
                         int32_t y_type, hipStream_t s);
hipError_t launch_ew_add(int64_t M, int64_t N, const void *X, int32_t x_type, const void *R,
                         int32_t r_type, int64_t ldr, void *Y, int32_t y_type, int64_t ldy,
                         hipStream_t s);
hipError_t launch_ew_sigmoid(int64_t count, const void *X, void *Y, hipStream_t s);   // bf16
hipError_t launch_ew_mul(int64_t count, const void *X, const void *Z, void *Y, hipStream_t s);  // bf16
hipError_t launch_ew_copy(int64_t M, int64_t N, const void *X, int32_t x_type, void *Y,
                          int32_t y_type, int64_t ldy, hipStream_t s);
hipError_t launch_w4_dequant(int32_t K, int32_t N, const uint8_t *Wq, int64_t ldq,
                             const void *scales, int64_t ld_s, int32_t group, int32_t zero_point,
                             int32_t lo_first, void *W, hipStream_t s, int32_t wfmt = WFMT_U4);

// Fused residual add + RMSNorm (bf16 rows).
hipError_t launch_add_rmsnorm(int32_t M, int32_t N, const void *a, const void *x, const void *w,
                              float eps, void *resid, void *out, hipStream_t s);
// The same step as two kernels (add, then RMSNorm over the stored residual), for measurement.
hipError_t launch_add_rmsnorm_unfused(int32_t M, int32_t N, const void *a, const void *x, const void *w,
                                      float eps, void *resid, void *out, hipStream_t s);

}  // namespace ge
