/*
 * gemm_epi.h -- C ABI of the fused GEMM + epilogue engine for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * What is computed (pages "Fusion and Epilogues" (Epilogue fusion), "Kernel
 * fusion" (Concept, Check yourself) and "Fusion Thinking" (Patterns 2 and 3)):
 *
 *   generic   D = act(alpha * A.B + beta * C + bias) + R
 *   swiglu    D = silu(X.Wg) * (X.Wu)
 *   w4        D = act(alpha * X.deq(Wq, s) + beta * C + bias) + R,
 *             deq(Wq, s)[k][n] = (code[k][n] - zero_point) * s[k / group][n]
 *
 * The whole epilogue is applied to the fp32 accumulator tile while it is
 * still on chip, so D is written to memory exactly once.  The unfused entry
 * points compute the same results as a chain of separate kernels (one memory
 * round trip per step); they exist to measure what fusion saves.
 *
 * Conventions common to every entry point
 *   - Matrices are row-major.  Element (i, j) of a matrix with leading
 *     dimension ld lives at base[i * ld + j]; ld is counted in elements
 *     (bytes for packed int4), 0 means dense.
 *   - A is [M, K].  B is [K, N] (GE_LAYOUT_KN) or stored transposed as [N, K]
 *     (GE_LAYOUT_NK).  C, R and D are [M, N]; bias is [N].
 *   - Packed int4 weights Wq are [K, N/2] bytes: byte j of row k holds the
 *     codes of columns 2j and 2j+1, high nibble first unless the flag
 *     GE_FLAG_NIBBLE_LO_FIRST is set.  Scales are [K / group, N].
 *   - All device pointers belong to the caller and must be device memory of
 *     the device that was current when the plan was made.  The library never
 *     allocates, frees or synchronises in a run call: runs are asynchronous on
 *     the given stream (a hipStream_t passed as void*, NULL = null stream) and
 *     may be captured into a HIP graph.
 *   - D may alias C or R exactly (same pointer, same leading dimension); any
 *     other overlap between D and an input is undefined.
 *   - Arithmetic: products in bf16 x bf16 (or fp32 x fp32) with fp32
 *     accumulation, epilogue in fp32, one round-to-nearest-even conversion to
 *     the output type.
 *   - Errors: every function returns a ge_status; nothing is thrown across the
 *     ABI.  On an error no work has been queued; a thread-local message is
 *     available from ge_last_error().
 *
 * Plans are immutable once made: one plan may be used from several threads
 * and streams at once, with one exception: a plan that owns device scratch
 * (gemm_epi_plan_scratch_bytes() > 0: quantised-weight plans whose K is split
 * over workgroups -- M <= 16 streaming, or the tile kernel at M > 16 (8-bit)
 * or M > 32 (int4) when its tiles leave CUs idle -- and bf16 generic plans
 * with M <= 16 whose K is split the same way (stream-K), and SwiGLU plans
 * with M <= 32 on the gate / up workgroup pairs) must not run on two
 * streams at once, since its launches share that scratch.
 */
#ifndef GEMM_EPI_H
#define GEMM_EPI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define GE_API __attribute__((visibility("default")))
#else
#define GE_API
#endif

typedef int32_t ge_status;
#define GE_OK 0
#define GE_ERR_INVALID_ARG 1 /* bad shape, stride, pointer or enum value */
#define GE_ERR_UNSUPPORTED 2 /* valid request that no kernel instance covers */
#define GE_ERR_NO_DEVICE 3   /* no usable HIP device (or not a gfx950) */
#define GE_ERR_HIP 4         /* HIP runtime or launch error; see ge_last_error() */
#define GE_ERR_ALIGN 5       /* a pointer / stride breaks the alignment the kernel needs */

/* storage types */
#define GE_F32 0
#define GE_BF16 1
#define GE_U4X2 2     /* two 4-bit codes per byte (packed int4 weights) */
#define GE_U8 3       /* one unsigned 8-bit code per byte (weights, with a zero point) */
#define GE_FP8E4M3 4  /* one OCP fp8 E4M3 ("fn": no infinities) value per byte (weights) */

/* layout of the second operand */
#define GE_LAYOUT_KN 0 /* B[k][n] at B[k * ldb + n] */
#define GE_LAYOUT_NK 1 /* B[k][n] at B[n * ldb + k] */

/* activations (applied after alpha, beta * C and bias; before R) */
#define GE_ACT_NONE 0
#define GE_ACT_RELU 1      /* max(t, 0) */
#define GE_ACT_GELU_TANH 2 /* 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))) */
#define GE_ACT_SILU 3      /* t / (1 + exp(-t)) */

/* plan kinds */
#define GE_KIND_GENERIC 0
#define GE_KIND_SWIGLU 1
#define GE_KIND_W4 2

/* flags */
#define GE_FLAG_BIAS 1u            /* add bias[n] */
#define GE_FLAG_C 2u               /* add beta * C (ignored when beta == 0) */
#define GE_FLAG_RESIDUAL 4u        /* add R after the activation */
#define GE_FLAG_NIBBLE_LO_FIRST 8u /* W4: low nibble is the even column */
#define GE_FLAG_W4_PREPACKED 16u   /* W4: Wq is in the layout gemm_w4_prepack writes */
#define GE_FLAG_B_PREPACKED 32u    /* GENERIC bf16 or SWIGLU, M <= 32: B (Wg, Wu) in the layout gemm_b_prepack writes */

/* rope flags (ge_rope_qk_run, ge_rope_run) */
#define GE_ROPE_INTERLEAVED 1 /* pair i is (2i, 2i + 1); else (i, i + D/2), rotate-half */
#define GE_ROPE_EXACT 2       /* each rotated coordinate is the exact rotation rounded once to bf16 */
#define GE_FLAG_NO_SCRATCH 64u     /* the plan allocates no device memory (see gemm_epi_run_noalloc) */

/*
 * Problem descriptor.  Unused fields must be zero.  dtype fields take
 * GE_F32 / GE_BF16 (b_type may be GE_U4X2, GE_U8 or GE_FP8E4M3 for
 * GE_KIND_W4, the weight-only quantised kind).
 *
 * Supported combinations:
 *   GENERIC  a_type == b_type in {F32, BF16}; c/bias/r/d types in {F32, BF16};
 *            b_layout KN or NK; any act; any flags except NIBBLE_LO_FIRST and
 *            W4_PREPACKED.  With GE_FLAG_B_PREPACKED (a decode-time weight
 *            layout): a = b = BF16, b_layout KN, M <= 32, N % 128 == 0,
 *            K % 32 == 0; the unfused entry points reject such plans.
 *   SWIGLU   a, b, d = BF16, b_layout KN, act = NONE, alpha = 1, no flags
 *            other than none; Wg and Wu share ldb.
 *   W4       a = BF16, b = U4X2, scale_type = BF16, d/bias/c/r in {F32, BF16},
 *            K % group == 0, N even, group in {32, 64, 128, 256},
 *            zero_point in [0, 15].
 *            With GE_FLAG_W4_PREPACKED additionally: K % 128 == 0, and
 *            either M <= 32, N % 16 == 0, group in {32, 64, 128}, or N % 128
 *            == 0, group == 128; the unfused entry points take raw weights
 *            and reject such plans.
 *            The fused int4 kernels take every finite bf16 x and scale:
 *            codes enter the products as exact bf16 integers, scales as
 *            their exact bf16 values, and all sums (and the scaling of each
 *            group's partial sums) are carried out in fp32; nothing passes
 *            through fp16.
 *   W4 with 8-bit codes: b = U8 (W = (q - zero_point) * s, zero_point in
 *            [0, 255]) or FP8E4M3 (W = e4m3(q) * s, zero_point 0; NaN codes
 *            give NaN), Wq [K, N] bytes with ldb >= N, scales [K/group, N]
 *            bf16, group in {32, 64, 128, 256}, K % group == 0; flag
 *            NIBBLE_LO_FIRST is invalid, W4_PREPACKED (Wq in the layout
 *            gemm_w4_prepack writes for 8-bit codes) needs M <= 16,
 *            N % 128 == 0 and K % 32 == 0.  The dequantised weights are exact
 *            in the product (bf16 / fp32 arithmetic).
 */
typedef struct ge_desc {
    int32_t M, N, K;         /* > 0; M * N and K * N below 2^31 */
    int32_t a_type, b_type;  /* operand storage types */
    int32_t c_type, d_type;  /* C and D storage types */
    int32_t bias_type, r_type, scale_type;
    int32_t b_layout;        /* GE_LAYOUT_KN or GE_LAYOUT_NK */
    int64_t lda, ldb, ldc, ldd, ldr; /* leading dimensions (elements; bytes for Wq); 0 = dense */
    float alpha, beta;
    int32_t act;             /* GE_ACT_* */
    uint32_t flags;          /* GE_FLAG_* */
    int32_t group_size;      /* W4 scale group along K (0 = 128) */
    int32_t zero_point;      /* W4 code offset (the pages use 8) */
} ge_desc;

typedef struct ge_plan ge_plan;

/* Fill *d with the defaults: alpha 1, everything else 0 / dense / KN. */
GE_API void ge_desc_init(ge_desc *d);

/*
 * Validate d for the given kind and choose a kernel instance.  On success
 * *out receives a library-owned plan that the caller releases with
 * gemm_epi_plan_destroy().  Queries the current device (architecture and
 * compute-unit count); allocates host memory, and a zeroed device scratch
 * for these plans: quantised-weight plans with M <= 16 whose column blocks
 * alone do not fill the GPU (the cross-workgroup K split: S * ceil(N/128) *
 * 8 KiB of fp32 tiles plus 4 * ceil(N/128) bytes of counters, S in {2, 4,
 * 8}); quantised-weight plans on the tile kernel (prepacked int4 with M > 32,
 * 8-bit with M > 16) whose 64 x 128 tiles leave CUs idle (K split S ways, S
 * in {2, 4, 8} dividing K / 128 with 2 or more groups per slice: S * tiles *
 * 32 KiB of fp32 partial tiles plus 4 * tiles bytes of counters, tiles =
 * ceil(M / 64) * N / 128); bf16 generic plans with M <= 16 whose column blocks leave
 * CUs idle and whose (column block, 32-row K block) units divide evenly into
 * one K piece of one column block per CU (stream-K: the same tiles and
 * counters, S = pieces per block in {2..8}; e.g. 16 x 8192 x 8192 on 256
 * CUs, S = 4); SwiGLU plans with M <= 32 that take the gate / up
 * workgroup pairs (prepacked weights, or raw weights without
 * GE_FLAG_NO_SCRATCH: two fp32 tiles of 16 or 32 rows per column block plus
 * 4 bytes of counter per block).  Such a call waits for the zeroing of its scratch on a
 * stream of the library's own (the callers' streams keep running); device
 * allocation is not allowed during graph capture, so make such plans before
 * capturing (the call fails with GE_ERR_HIP and says so otherwise).
 * Errors: INVALID_ARG (bad descriptor or null out), UNSUPPORTED, NO_DEVICE.
 */
GE_API ge_status gemm_epi_plan(const ge_desc *d, int32_t kind, ge_plan **out);

/* Release a plan and its device scratch, if any (NULL is accepted). */
GE_API ge_status gemm_epi_plan_destroy(ge_plan *plan);

/* Bytes of device scratch the plan owns (0 for most plans; NULL gives 0). */
GE_API size_t gemm_epi_plan_scratch_bytes(const ge_plan *plan);

/* Name of the fused kernel instance a plan launches (static string). */
GE_API const char *gemm_epi_plan_kernel(const ge_plan *plan);

/*
 * Fused generic GEMM + epilogue:  D = act(alpha * A.B + beta * C + bias) + R.
 * C is read only when GE_FLAG_C is set and beta != 0; bias only with
 * GE_FLAG_BIAS; R only with GE_FLAG_RESIDUAL (pointers that are not read may
 * be NULL).  Fast paths need 16-byte aligned bases and leading dimensions
 * that are multiples of 8 elements; other inputs run a general kernel.
 */
GE_API ge_status gemm_epi_run(const ge_plan *plan, const void *A, const void *B, const void *C,
                       const void *bias, const void *R, void *D, void *stream);

/*
 * gemm_epi_run for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as gemm_epi_run, and the same kernel that a
 * plan owning scratch would launch; where that kernel needs device scratch
 * (bf16 decode shapes, M <= 16, whose K is split over workgroups: partial
 * fp32 tiles and per-column-block counters), it uses a static buffer that the
 * library holds on each GPU until the process ends: 64 KiB of counters
 * (16384 column blocks of 128) and 8 MiB of tiles; a shape that needs more
 * returns GE_ERR_UNSUPPORTED.  The call allocates nothing and never
 * synchronises; its first call on a GPU also queues a small kernel that
 * clears the counters.  Every call on one GPU shares that buffer: calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads) race and give wrong results.  A plan made with GE_FLAG_NO_SCRATCH
 * allocates no device memory, so neither making nor running it allocates
 * (gemm_epi_run on such a plan launches the variant that needs no scratch).
 */
GE_API ge_status gemm_epi_run_noalloc(const ge_plan *plan, const void *A, const void *B, const void *C,
                                      const void *bias, const void *R, void *D, void *stream);

/*
 * Fused SwiGLU dual GEMM:  D = silu(X.Wg) * (X.Wu).  X is [M, K]; Wg and Wu
 * are [K, N] with the plan's ldb.  Each X tile is read once and feeds both
 * products (page "Fusion Thinking", Pattern 2, Level 2).
 *
 * At M <= 32 each column block of Wg and of Wu streams on a workgroup of
 * its own through the decode loop, and the second of the two to finish
 * combines silu(gate) * up for the block: the pair's fp32 tiles and a
 * counter per block live in device scratch that the plan owns, so calls on
 * one such plan must not overlap in time.  Raw weights take this route when
 * the raw decode loop can read them (N % 8 == 0, 16-byte aligned X, Wg, Wu,
 * lda and ldb multiples of 8; otherwise the tile or general kernel runs),
 * unless the plan is made with GE_FLAG_NO_SCRATCH: then it allocates nothing
 * and runs the tile kernel.
 * A SwiGLU plan made with GE_FLAG_B_PREPACKED (M <= 32, N % 128 == 0,
 * K % 32 == 0, dense weights) takes Wg and Wu each converted by
 * gemm_b_prepack on a SwiGLU plan of the same N and K (that layout's column
 * blocks are sized so that the pairs fill the GPU); X, Wg and Wu must then
 * be 16-byte aligned (GE_ERR_ALIGN otherwise), and the unfused chain is
 * refused (it reads raw weights).
 */
GE_API ge_status gemm_swiglu_run(const ge_plan *plan, const void *X, const void *Wg, const void *Wu,
                          void *D, void *stream);

/*
 * Fused GEMM on weight-only quantised weights (packed int4, or 8-bit codes:
 * u8 with a zero point, fp8 E4M3): the codes are decoded and dequantised
 * inside the K loop and never exist in memory as bf16 (page "Fusion
 * Thinking", Pattern 3).  D = act(alpha * X.deq(Wq, s) + beta*C + bias) + R.
 */
GE_API ge_status gemm_w4_run(const ge_plan *plan, const void *X, const uint8_t *Wq, const void *scales,
                      const void *C, const void *bias, const void *R, void *D, void *stream);

/*
 * One-time weight conversion for the fused W4 kernels (the way a weight
 * loader would store quantised weights): reads raw packed int4 weights Wq
 * [K, N/2] (nibble order from the plan's flags, row stride = the plan's ldb)
 * and writes the same K*N/2 bytes to Wp in the kernel-native layout: for each
 * 64-column block (outer), 128-row K group, and 16-column tile of the block
 * (inner; the last block of an N that is not a multiple of 64 holds the
 * remaining tiles), 1 KiB = 64 lanes x 16 bytes, lane l holding the codes of
 * column 16*tile + l%16 for k = 128*group + 32*b + 8*(l/16) + j (b = 0..3,
 * one dword per b; code j at bit 4*(j/2) + 16*(j%2)).  So the fragment of
 * tile t and group g starts at byte 1024 * (4*ngroups*(t/4) + nt*g + t%4),
 * nt being the number of tiles in t's block.  Needs N % 16 == 0, K % 128 == 0
 * and a 16-byte aligned Wp that does not overlap Wq.  Asynchronous on the
 * stream.
 * For a plan with 8-bit codes (b_type U8 or FP8E4M3) it reads Wq [K, N]
 * bytes (row stride ldb, a multiple of 8, 8-byte aligned) and writes the K*N
 * bytes in the layout the 8-bit decode kernel streams: for each 128-column
 * block (outer) and 32-row K block (inner), 4 KiB holding 4 loads of 1 KiB;
 * load q holds, for lane l = 0..63 at byte 16*l, the codes of rows
 * 32*kb + 8*(l/16) + 2q and + 2q + 1 (8 bytes each, in that order), columns
 * 128*cb + 8*(l%16) .. + 7.  Needs N % 128 == 0 and K % 32 == 0.
 */
GE_API ge_status gemm_w4_prepack(const ge_plan *plan, const uint8_t *Wq, uint8_t *Wp, void *stream);

/*
 * One-time weight conversion for the prepacked bf16 decode kernels (M <= 32;
 * the way a weight loader would store decode weights): reads B [K, N] bf16
 * (row stride = the plan's ldb) and writes the same K*N*2 bytes to Bp in the
 * kernel-native layout: for each column block cb of T 16-column tiles
 * (outer) and 32-row K block kb (inner), T KiB holding the MFMA B fragments
 * of the block's tiles t, 1 KiB each, lane l's 16 bytes at byte 16*l of tile
 * t holding column 16*T*cb + 16*t + l%16 at k = 32*kb + 8*(l/16) + j,
 * j = 0..7 in order.  T is 8 (128-column blocks), or 7 where N / 112 is a
 * multiple of the device's CU count and N / 128 is not (so that every CU
 * streams the same number of blocks, e.g. N = 28672 on 256 CUs): the layout
 * depends on N and on the device the plan was made on, which must be the
 * device that runs it.  So each column block's K range is one contiguous
 * run of memory and every 16-byte load is a finished fragment (no transpose
 * in the kernel).  Any GENERIC bf16 KN plan of the same N, K and ldb serves
 * (M and the epilogue are ignored).  On a SWIGLU plan, T is chosen the same
 * way for 2 N columns (the gate and the up blocks together: T = 7 where
 * N % 112 == 0 and 2 N / 112 is a multiple of the CU count while 2 N / 128
 * is not, e.g. N = 14336 on 256 CUs), and the result serves the SwiGLU
 * plans made with GE_FLAG_B_PREPACKED.  Needs N % 128 == 0, K % 32 == 0, a
 * 2-byte aligned B and a 16-byte aligned Bp that does not overlap B.
 * Asynchronous on the stream.
 */
GE_API ge_status gemm_b_prepack(const ge_plan *plan, const void *B, void *Bp, void *stream);

/*
 * Rotary position embedding applied as the Q and K tiles are loaded, with the
 * attention scores product as the consumer (page "Fusion Thinking", Pattern
 * 4: RoPE computed at Q-tile and K-tile load time instead of by two kernels
 * that write q' and k' back to memory):
 *   S[b, m, n] = alpha * sum_d rope(Q[b, m, :], q_pos0 + m)[d] * rope(K[b, n, :], k_pos0 + n)[d]
 * Q [batch, Sq, D] and K [batch, Sk, D] bf16, dense, 16-byte aligned; cos and
 * sin fp32 [n_pos, D/2] (row p: cos(p theta_i), sin(p theta_i)), 16-byte
 * aligned, covering every position used; S [batch, Sq, Sk] of s_type (GE_F32
 * or GE_BF16), dense, not overlapping Q or K.  Pair i of a row is (i, i + D/2)
 * (rotate-half, the Llama layout), or (2i, 2i + 1) with GE_ROPE_INTERLEAVED in
 * flags: x'_a = x_a cos - x_b sin, x'_b = x_a sin + x_b cos, the values the
 * unfused chain stores (bf16, RNE).  With GE_ROPE_EXACT each x' is the exact
 * rotated value rounded once; without it each is computed in fp32 (one rounded
 * product, one fused multiply-add) and rounded to bf16: within one bf16 unit of
 * the exactly rounded value, or within 2^-23 (|x_a cos| + |x_b sin|) of the
 * exact rotation where the two products cancel (the exact rounding costs about
 * a third more time here: the key tiles are rotated once per query tile).  The
 * product is bf16 x bf16 with fp32 accumulation, alpha applied in fp32, one
 * rounding to s_type.  cos == sin == NULL: no rotation (the plain product, the
 * unfused chain's last step).  D in {64, 128}, batch <= 65535.
 * Errors: INVALID_ARG (sizes, NULLs, positions outside the tables, overlap,
 * unknown flag bits), UNSUPPORTED (D), ALIGN, NO_DEVICE, HIP.  Asynchronous on
 * the stream.
 */
GE_API ge_status ge_rope_qk_run(int32_t batch, int32_t Sq, int32_t Sk, int32_t D, const void *Q, const void *K,
                                const float *cos_t, const float *sin_t, int32_t n_pos, int32_t q_pos0,
                                int32_t k_pos0, int32_t flags, float alpha, int32_t s_type, void *S,
                                void *stream);

/*
 * The rotation alone (the unfused chain's first kernels, rope(q, cos, sin) of
 * the same page): Y = rope(X) for X, Y [batch, S, D] bf16, row s of each batch
 * at position pos0 + s, with the pairing and rounding of ge_rope_qk_run (the
 * same flags).  X and Y 16-byte aligned, not overlapping; cos, sin as above
 * (required).
 */
GE_API ge_status ge_rope_run(int32_t batch, int32_t S, int32_t D, const void *X, const float *cos_t,
                             const float *sin_t, int32_t n_pos, int32_t pos0, int32_t flags, void *Y,
                             void *stream);

/*
 * Deliberately unfused chains, for measurement only: the plain GEMM writes
 * its fp32-accumulated result to the workspace in the output type (bf16 or
 * fp32), then one elementwise kernel per epilogue step reads and writes
 * memory (generic: scale / C, bias, activation, residual; swiglu: gate GEMM,
 * up GEMM, then sigmoid, multiply, multiply, as separate kernels; w4: a
 * dequant kernel writes the bf16 weights to the workspace first).  The
 * caller owns the workspace, of at least gemm_epi_unfused_workspace_bytes()
 * bytes, 256-byte aligned.
 */
GE_API ge_status gemm_epi_unfused_workspace_bytes(const ge_plan *plan, size_t *bytes);
GE_API ge_status gemm_epi_run_unfused(const ge_plan *plan, const void *A, const void *B, const void *C,
                               const void *bias, const void *R, void *D, void *workspace,
                               void *stream);
GE_API ge_status gemm_swiglu_run_unfused(const ge_plan *plan, const void *X, const void *Wg,
                                  const void *Wu, void *D, void *workspace, void *stream);
GE_API ge_status gemm_w4_run_unfused(const ge_plan *plan, const void *X, const uint8_t *Wq,
                              const void *scales, const void *C, const void *bias, const void *R,
                              void *D, void *workspace, void *stream);

/*
 * First step of the unfused W4 chain on its own: W[k][n] =
 * bf16_rne((code[k][n] - zero_point) * s[k / group][n]), W dense [K, N] bf16.
 */
GE_API ge_status gemm_w4_dequant_run(const ge_plan *plan, const uint8_t *Wq, const void *scales, void *W,
                              void *stream);

/*
 * Fused residual add + RMSNorm over rows of length N (page "Fusion
 * Thinking", Pattern 1): resid = a + x; out = resid / sqrt(mean(resid^2) +
 * eps) * w.  a, x, resid, out are [M, N] bf16 (dense), w is [N] bf16.  resid
 * may alias a or x exactly.
 */
GE_API ge_status ge_add_rmsnorm_run(int32_t M, int32_t N, const void *a, const void *x, const void *w,
                             float eps, void *resid, void *out, void *stream);

/*
 * The same step deliberately unfused, for measurement only (page "Fusion
 * Thinking", Pattern 1: the separate add and normalisation kernels that the
 * fused one replaces): one elementwise kernel writes resid = bf16(a + x),
 * then a second one reads the stored resid back and writes out = resid /
 * sqrt(mean(resid^2) + eps) * w, so the norm is taken over the rounded
 * residual.  Same arguments, checks, aliasing rules and status codes as
 * ge_add_rmsnorm_run; resid is written before it is read, on the same stream.
 */
GE_API ge_status ge_add_rmsnorm_run_unfused(int32_t M, int32_t N, const void *a, const void *x, const void *w,
                                     float eps, void *resid, void *out, void *stream);

/* Static text for a status code. */
GE_API const char *ge_status_string(ge_status s);

/* Detail of the last error on the calling thread ("" if none). */
GE_API const char *ge_last_error(void);

/* Library version, "major.minor.patch". */
GE_API const char *ge_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPI_H */
