// ge_rope.hip -- rotary position embedding applied as the Q and K tiles are
// loaded, with the scores product S = alpha * rope(Q) rope(K)^T as the
// consumer (page "Fusion Thinking", Pattern 4: the rotation is computed at
// Q-tile and K-tile load time instead of by two kernels that write q' and k'
// back to memory just before the product reads them).
//
// One 256-thread workgroup per (head, 128-query tile), walking the key tiles:
//   1. the tiles are read from memory in 16-byte chunks and rotated -- the
//      values the unfused chain would have stored, each coordinate in fp32
//      (one product and one fused multiply-add) rounded to bf16 (RNE), or
//      (EX) the exact rotation rounded once -- and written to LDS rows
//      padded by 16 bytes, so that the MFMA fragment reads
//      of 16 rows hit 16 distinct bank groups;
//   2. four waves (2 x 2, 64 x 64 each) run v_mfma_f32_16x16x32_bf16 over
//      the head dimension, K' fragments as the first operand so that each
//      lane holds four consecutive key columns of one query row;
//   3. the scale alpha is applied in fp32 and S is stored once (fp32 or bf16).
// The query tile is rotated once per workgroup; the next key tile's loads
// are in flight while the current one is multiplied and its scores stored.
// Pairs: (i, i + D/2) (rotate-half) or (2i, 2i + 1) (interleaved); the pair
// rotates by the angle of the row's position p: cos and sin come from tables
// [P][D/2], row p.

#include "ge_launch.hpp"

namespace ge {
namespace {

constexpr int RT = 128;  // query rows and key rows per tile

// Rounding of a rotated coordinate.  The stored value is the exact rotation rounded once to bf16
// (nearest, ties to even).  Fast path, in fp32: Kahan's difference of products, w = b t,
// e = fma(b, t, -w) (exactly b t - w), f = fma(a, c, -+w), r = f -+ e, for x' = a c -+ b t.  Its error
// is below 2 units in the last place of r (2^-23 |r|), so r rounds to the bf16 number the exact
// value rounds to when r lies 4 or more of those units away from every point halfway between two
// bf16 numbers (low 16 bits of r outside 0x7ffd .. 0x8003) and is neither tiny (|r| < 2^-100, where
// underflow would void the bound) nor huge or not finite.  Other elements are redone by rot_exact.
__device__ __forceinline__ bool rot_unsure(float r) {
    const uint16_t lo = (uint16_t)__builtin_bit_cast(uint32_t, r);
    const float m = __builtin_fabsf(r);
    // 16-bit subtract and compare on the low half; !(m >= 2^-100 && m <= max) also catches NaN
    return (uint16_t)(lo - (uint16_t)0x7ffd) <= (uint16_t)6 || !(m >= 0x1p-100f && m <= 0x1.fffffep127f);
}

// EX: the fast path of the exact rounding above.  Otherwise one rounded product and one fused
// multiply-add, r = fma(a, c, -+ rn(b t)): |r - (a c -+ b t)| <= 2^-24 (|b t| + |r|), so after the
// rounding to bf16 the value is within one bf16 unit of the exactly rounded one, or, where the two
// products cancel, within 2^-23 (|a c| + |b t|) of the exact rotation (a quarter of the exact
// rounding's cost: the rotation of every key tile for every query tile is the fused kernel's main
// vector work).
template <bool EX>
__device__ __forceinline__ float rot_fast(float a, float c, float b, float t, bool neg, bool &slow) {
    if constexpr (EX) {
        const float w = b * t;
        const float e = __builtin_fmaf(b, t, -w);
        const float r = neg ? __builtin_fmaf(a, c, -w) - e : __builtin_fmaf(a, c, w) + e;
        slow |= rot_unsure(r);
        return r;
    } else {
        return neg ? __builtin_fmaf(a, c, -(b * t)) : __builtin_fmaf(a, c, b * t);
    }
}

// bf16 bits of a c -+ b t computed exactly: both products are exact in fp64 (8 and 24 significant
// bits), their sum s is rounded once, and the TwoSum residual err (s + err is the exact value)
// decides a tie that the fp64 rounding may have created.  The magnitude is scaled by a power of two
// so that the bf16 spacing becomes 1 (2^-133 below 2^-126, the subnormal spacing).
__device__ __noinline__ uint32_t rot_exact(float a, float c, float b, float t, bool neg) {
    const double p = (double)a * (double)c;
    const double q = neg ? -((double)b * (double)t) : (double)b * (double)t;
    const double s = p + q;
    const double bb = s - p;
    const double err = (p - (s - bb)) + (q - bb);
    const uint32_t sign = s < 0.0 ? 0x8000u : 0u;
    if (s == 0.0) return (uint32_t)(__builtin_bit_cast(uint64_t, s) >> 48) & 0x8000u;
    const double mag = __builtin_fabs(s);
    int e2 = 0;
    (void)__builtin_frexp(mag, &e2);  // 2^(e2 - 1) <= mag < 2^e2
    const int sh = e2 - 8 > -133 ? e2 - 8 : -133;
    const double v = __builtin_ldexp(mag, -sh);  // exact
    const double fl = __builtin_floor(v);
    const double frac = v - fl;                  // exact
    bool up;
    if (frac != 0.5)
        up = frac > 0.5;
    else if (err != 0.0)
        up = (err > 0.0) == (s > 0.0);  // the exact magnitude lies above the halfway point
    else
        up = ((uint64_t)fl & 1u) != 0;  // exact tie: to even
    const uint32_t f = (uint32_t)fl + (up ? 1u : 0u);
    uint32_t mb = sh == -133 ? f : ((uint32_t)(e2 - 1 + 127) << 7) + (f - 128u);
    if (mb > 0x7f80u) mb = 0x7f80u;  // beyond the largest bf16: infinity
    return sign | mb;
}

// Rotate chunk c of one row from registers.  Rotate-half: x[0] = elements 8c .. 8c+7 of the first
// half, x[1] the same elements of the second half (D/2 + 8c ..), c4 / s4 the 8 angles 8c .. 8c+7;
// o0, o1 the rotated chunks.  Interleaved: x[0] = elements 8c .. 8c+7, i.e. the pairs 4c .. 4c+3
// with the 4 angles in c4[0] / s4[0]; o0 the rotated chunk.  Every coordinate is the exact rotation
// rounded once to bf16 (fast path above, flagged elements redone exactly).
template <int D, bool INTER, bool EX>
__device__ __forceinline__ void rope_regs(const u32x4 *x, const f32x4 *c4, const f32x4 *s4, u32x4 &o0, u32x4 &o1) {
    // elements whose fast result is not certain (rare) are redone one by one, only in the lanes
    // that hold them
    auto fix = [](uint32_t o, int half, float r, float a, float c, float b, float t, bool neg) -> uint32_t {
        if (rot_unsure(r)) {
            const uint32_t v = rot_exact(a, c, b, t, neg);
            o = half ? (o & 0xffffu) | (v << 16) : (o & 0xffff0000u) | v;
        }
        return o;
    };
    if constexpr (INTER) {
        bool slow = false;
        float ya[4], yb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = bf16lo(x[0][j]), b = bf16hi(x[0][j]);
            ya[j] = rot_fast<EX>(a, c4[0][j], b, s4[0][j], true, slow);
            yb[j] = rot_fast<EX>(a, s4[0][j], b, c4[0][j], false, slow);
            o0[j] = pack_bf16x2(ya[j], yb[j]);
        }
        if (__builtin_expect(slow, 0)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = bf16lo(x[0][j]), b = bf16hi(x[0][j]);
                o0[j] = fix(o0[j], 0, ya[j], a, c4[0][j], b, s4[0][j], true);
                o0[j] = fix(o0[j], 1, yb[j], a, s4[0][j], b, c4[0][j], false);
            }
        }
    } else {
        bool slow = false;
        float ya[8], yb[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float c0 = c4[j >> 1][(2 * j) & 3], c1 = c4[j >> 1][(2 * j + 1) & 3];
            const float s0 = s4[j >> 1][(2 * j) & 3], s1 = s4[j >> 1][(2 * j + 1) & 3];
            const float a0 = bf16lo(x[0][j]), a1 = bf16hi(x[0][j]);  // first-half elements 8c + 2j, + 1
            const float b0 = bf16lo(x[1][j]), b1 = bf16hi(x[1][j]);  // their partners in the second half
            ya[2 * j] = rot_fast<EX>(a0, c0, b0, s0, true, slow);
            yb[2 * j] = rot_fast<EX>(a0, s0, b0, c0, false, slow);
            ya[2 * j + 1] = rot_fast<EX>(a1, c1, b1, s1, true, slow);
            yb[2 * j + 1] = rot_fast<EX>(a1, s1, b1, c1, false, slow);
            o0[j] = pack_bf16x2(ya[2 * j], ya[2 * j + 1]);
            o1[j] = pack_bf16x2(yb[2 * j], yb[2 * j + 1]);
        }
        if (__builtin_expect(slow, 0)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float c0 = c4[j >> 1][(2 * j) & 3], c1 = c4[j >> 1][(2 * j + 1) & 3];
                const float s0 = s4[j >> 1][(2 * j) & 3], s1 = s4[j >> 1][(2 * j + 1) & 3];
                const float a0 = bf16lo(x[0][j]), a1 = bf16hi(x[0][j]);
                const float b0 = bf16lo(x[1][j]), b1 = bf16hi(x[1][j]);
                o0[j] = fix(o0[j], 0, ya[2 * j], a0, c0, b0, s0, true);
                o0[j] = fix(o0[j], 1, ya[2 * j + 1], a1, c1, b1, s1, true);
                o1[j] = fix(o1[j], 0, yb[2 * j], a0, s0, b0, c0, false);
                o1[j] = fix(o1[j], 1, yb[2 * j + 1], a1, s1, b1, c1, false);
            }
        }
    }
}

// The same from memory: chunk c of the row at xrow with its position's table rows.
template <int D, bool INTER, bool EX>
__device__ __forceinline__ void rope_chunk(const uint16_t *xrow, const float *crow, const float *srow, int c,
                                           u32x4 &o0, u32x4 &o1) {
    constexpr int NV = INTER ? 1 : 2, NT = INTER ? 1 : 2;
    u32x4 x[NV];
    f32x4 c4[NT], s4[NT];
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] = *(const u32x4 *)(xrow + v * (D / 2) + 8 * c);
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        c4[q] = *(const f32x4 *)(crow + NT * 4 * c + 4 * q);
        s4[q] = *(const f32x4 *)(srow + NT * 4 * c + 4 * q);
    }
    rope_regs<D, INTER, EX>(x, c4, s4, o0, o1);
}

// chunks per row handled by one work item
template <int D, bool INTER>
constexpr int chunks_per_row() { return INTER ? D / 8 : D / 16; }

// One 128-row tile of X (rows r0 .. r0 + 127 of a [rows][D] head, row r at position pos0 + r): each
// thread's chunks and their cos / sin requested into registers (rows past the end read nothing and
// stage zeros), then rotated when ROT and written to LDS rows of D + 8 elements.
template <int D, bool INTER, bool ROT, bool EX>
struct TileRegs {
    static constexpr int CPR = ROT ? chunks_per_row<D, INTER>() : D / 8;
    static constexpr int ITEMS = RT * CPR / 256;               // per thread
    static constexpr int NV = (ROT && !INTER) ? 2 : 1;         // 16-byte chunks of X per item
    static constexpr int NT = ROT ? (INTER ? 1 : 2) : 1;       // 16-byte chunks of each table per item
    static_assert(RT * CPR % 256 == 0, "items per thread");
    u32x4 x[ITEMS][NV];
    f32x4 c[ITEMS][NT], s[ITEMS][NT];

    __device__ __forceinline__ void load(const uint16_t *X, int rows, int r0, int pos0, const float *cosT,
                                         const float *sinT) {
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            const int it = threadIdx.x + 256 * u, r = it / CPR, ch = it % CPR;
            const bool in = r0 + r < rows;
            const uint16_t *xrow = X + (int64_t)(in ? r0 + r : 0) * D;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                x[u][v] = in ? *(const u32x4 *)(xrow + v * (D / 2) + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
            if constexpr (ROT) {
                const int64_t p = in ? pos0 + r0 + r : 0;
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    c[u][q] = *(const f32x4 *)(cosT + p * (D / 2) + NT * 4 * ch + 4 * q);
                    s[u][q] = *(const f32x4 *)(sinT + p * (D / 2) + NT * 4 * ch + 4 * q);
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t *dst) const {
        constexpr int LD = D + 8;
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            const int it = threadIdx.x + 256 * u, r = it / CPR, ch = it % CPR;
            if constexpr (!ROT) {
                *(u32x4 *)(dst + r * LD + 8 * ch) = x[u][0];
            } else {
                u32x4 o0, o1;
                rope_regs<D, INTER, EX>(x[u], c[u], s[u], o0, o1);
                *(u32x4 *)(dst + r * LD + 8 * ch) = o0;
                if constexpr (!INTER) *(u32x4 *)(dst + r * LD + D / 2 + 8 * ch) = o1;
            }
        }
    }
};

// One workgroup per (head, 128-query tile), XCD-aware: the query tile is rotated once into LDS; the key tiles
// follow one another through two LDS buffers, the next one's chunks and tables requested into
// registers before the current one is multiplied and its scores stored.
template <int D, bool INTER, bool ROT, bool F32OUT, bool EX>
__global__ __launch_bounds__(256) void rope_qk_kernel(RopeArgs a) {
    constexpr int LD = D + 8;
    extern __shared__ __attribute__((aligned(16))) uint16_t rsm[];
    uint16_t *qs = rsm;
    // workgroup -> (head, query tile): consecutive ids land on different XCDs (round-robin), so ids
    // are regrouped so that each XCD owns a contiguous run of (head, query tile) pairs, i.e. whole
    // heads, whose key tiles its L2 then fetches once instead of once per query tile
    const int nq = (a.Sq + RT - 1) / RT, total = nq * a.batch;
    int pair = blockIdx.x;
    if ((total & 7) == 0) pair = (pair & 7) * (total >> 3) + (pair >> 3);
    const int b = pair / nq, m0 = (pair % nq) * RT;
    const uint16_t *Kb = a.K + (int64_t)b * a.Sk * D;
    const int ntiles = (a.Sk + RT - 1) / RT;

    TileRegs<D, INTER, ROT, EX> t;
    t.load(a.Q + (int64_t)b * a.Sq * D, a.Sq, m0, a.q_pos0, a.cos, a.sin);
    t.store(qs);
    t.load(Kb, a.Sk, 0, a.k_pos0, a.cos, a.sin);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, fr = lane & 15, fg = lane >> 4;
    const bool vec = (a.Sk & 3) == 0;
    for (int jt = 0; jt < ntiles; ++jt) {
        uint16_t *ks = rsm + (1 + (jt & 1)) * RT * LD;
        const int n0 = jt * RT;
        t.store(ks);
        if (jt + 1 < ntiles) t.load(Kb, a.Sk, n0 + RT, a.k_pos0, a.cos, a.sin);
        __syncthreads();  // this key tile (and, first time, the query tile) visible; buffer jt-1 done with

        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            bf16x8 qa[4], kf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qa[i] = *(const bf16x8 *)(qs + (wm * 64 + 16 * i + fr) * LD + 32 * kk + 8 * fg);
#pragma unroll
            for (int j = 0; j < 4; ++j) kf[j] = *(const bf16x8 *)(ks + (wn * 64 + 16 * j + fr) * LD + 32 * kk + 8 * fg);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(kf[j], qa[i], acc[i][j]);
        }

        // lane holds S[m][n .. n + 3], m = m0 + 64 wm + 16 i + fr, n = n0 + 64 wn + 16 j + 4 fg
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 64 + 16 * i + fr;
            if (m >= a.Sq) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + wn * 64 + 16 * j + 4 * fg;
                if (n >= a.Sk) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = a.alpha * acc[i][j][e];
                const int64_t off = ((int64_t)b * a.Sq + m) * a.Sk + n;
                if (vec && n + 4 <= a.Sk) {
                    if constexpr (F32OUT)
                        *(f32x4 *)((float *)a.S + off) = f32x4{v[0], v[1], v[2], v[3]};
                    else
                        *(u32x2 *)((uint16_t *)a.S + off) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.Sk) {
                            if constexpr (F32OUT)
                                ((float *)a.S)[off + e] = v[e];
                            else
                                ((uint16_t *)a.S)[off + e] = (uint16_t)(pack_bf16x2(v[e], 0.0f) & 0xffffu);
                        }
                }
            }
        }
    }
}

// the rotation alone: X [batch * S][D] -> Y, row r at position pos0 + r % S
template <int D, bool INTER, bool EX>
__global__ __launch_bounds__(256) void rope_kernel(int64_t rows, int32_t S, const uint16_t *X, const float *cosT,
                                                   const float *sinT, int32_t pos0, uint16_t *Y) {
    constexpr int CPR = chunks_per_row<D, INTER>();
    const int64_t items = rows * CPR;
    for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
        const int64_t r = it / CPR;
        const int c = (int)(it % CPR);
        const int64_t p = pos0 + r % S;
        u32x4 o0, o1;
        rope_chunk<D, INTER, EX>(X + r * D, cosT + p * (D / 2), sinT + p * (D / 2), c, o0, o1);
        *(u32x4 *)(Y + r * D + 8 * c) = o0;
        if constexpr (!INTER) *(u32x4 *)(Y + r * D + D / 2 + 8 * c) = o1;
    }
}

template <int D, bool INTER, bool ROT, bool F32OUT, bool EX>
hipError_t go_qk(const RopeArgs &a, hipStream_t s) {
    auto k = rope_qk_kernel<D, INTER, ROT, F32OUT, EX>;
    constexpr int lds = 3 * RT * (D + 8) * 2;  // the query tile and two key tiles
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 grid((unsigned)(((a.Sq + RT - 1) / RT) * a.batch));
    hipLaunchKernelGGL(k, grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int D, bool EX>
hipError_t qk_for_d(const RopeArgs &a, bool inter, bool rot, bool f32out, hipStream_t s) {
    if (!rot) return f32out ? go_qk<D, false, false, true, false>(a, s) : go_qk<D, false, false, false, false>(a, s);
    if (inter) return f32out ? go_qk<D, true, true, true, EX>(a, s) : go_qk<D, true, true, false, EX>(a, s);
    return f32out ? go_qk<D, false, true, true, EX>(a, s) : go_qk<D, false, true, false, EX>(a, s);
}

}  // namespace

hipError_t launch_rope_qk(const RopeArgs &a, bool interleaved, bool f32out, bool exact, hipStream_t s) {
    const bool rot = a.cos != nullptr;
    if (a.D == 64) return exact ? qk_for_d<64, true>(a, interleaved, rot, f32out, s) : qk_for_d<64, false>(a, interleaved, rot, f32out, s);
    if (a.D == 128) return exact ? qk_for_d<128, true>(a, interleaved, rot, f32out, s) : qk_for_d<128, false>(a, interleaved, rot, f32out, s);
    return hipErrorInvalidValue;
}

hipError_t launch_rope(int32_t batch, int32_t S, int32_t D, const uint16_t *X, const float *cosT, const float *sinT,
                       int32_t pos0, bool interleaved, bool exact, uint16_t *Y, hipStream_t s) {
    const int64_t rows = (int64_t)batch * S;
    const int64_t items = rows * (interleaved ? D / 8 : D / 16);
    const int blocks = (int)((items + 255) / 256 < 8192 ? (items + 255) / 256 : 8192);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, rows, S, X, cosT, sinT, pos0, Y);
        return hipGetLastError();
    };
    if (exact) {
        if (D == 64) return interleaved ? go(rope_kernel<64, true, true>) : go(rope_kernel<64, false, true>);
        if (D == 128) return interleaved ? go(rope_kernel<128, true, true>) : go(rope_kernel<128, false, true>);
    } else {
        if (D == 64) return interleaved ? go(rope_kernel<64, true, false>) : go(rope_kernel<64, false, false>);
        if (D == 128) return interleaved ? go(rope_kernel<128, true, false>) : go(rope_kernel<128, false, false>);
    }
    return hipErrorInvalidValue;
}

}  // namespace ge
