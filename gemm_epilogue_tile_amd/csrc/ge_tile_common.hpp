// ge_tile_common.hpp -- pieces shared by the MFMA tile kernels (bf16 and int4):
// direct-to-LDS buffer loads, buffer resources, LDS swizzles, stage sizes and
// the alignment checks of the epilogue operands.  Included inside
// namespace ge { namespace { ... } } of each kernel source.
#pragma once

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define AS3 __attribute__((address_space(3)))

constexpr int T_THREADS = 256;
constexpr int T_BK = 32;   // K depth of one stage
constexpr int T_NS = 4;    // LDS stages
constexpr int GROUP_M = 4;
constexpr uint32_t OOB = 0x80000000u;  // beyond any buffer this kernel builds (< 2^31 bytes)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (base, size in bytes, stride 0): lanes whose offset is
// at or past `bytes` read zeros.  The fields are wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, int64_t bytes) {
    const uint32_t n = bytes > 0 ? (uint32_t)bytes : 0u;
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from memory straight into LDS at lds + 16 * lane.  Issued
// as inline assembly so the compiler does not track it: its LDS writes are
// ordered by the explicit vmcnt waits and barriers of the main loop.  (The
// tracked builtin makes the compiler wait for every outstanding direct load
// before any LDS read, which would undo the prefetch.)
__device__ __forceinline__ void load_lds16(const i32x4 &r, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(r) : "memory", "m0");
}

// [rows][32] tiles (64-byte rows): 16-byte chunk c of row r lives at c ^ ((r >> 1) & 3)
__device__ __forceinline__ int swz_a(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }
// [32][BN] tiles (BN >= 128): 16-byte chunk c of row k lives at c ^ swz_b_key(k).  The transposing
// fragment read covers rows k0 .. k0 + 3 and k0 + 8 .. k0 + 11 in one half-wave: bits 0-1 of k spread
// the first four rows over 8 chunks, bit 3 moves the other four to the next 8 (without it the two
// sets share banks; 1.74 against 1.10 ns per read per CU in an LDS-bound probe).
__device__ __forceinline__ int swz_b_key(int k) { return ((k & 3) << 1) ^ (((k >> 3) & 1) << 3); }
template <int BN>
__device__ __forceinline__ int swz_b(int k, int chunk) { return k * (BN * 2) + ((chunk ^ swz_b_key(k)) << 4); }

// 4 consecutive elements as fp32 (8-byte bf16 or 16-byte fp32 access)
__device__ __forceinline__ void load4(const void *p, int32_t type, int64_t off, float v[4]) {
    if (type == GE_BF16) {
        const u32x2 w = *(const u32x2 *)((const uint16_t *)p + off);
        v[0] = bf16lo(w[0]);
        v[1] = bf16hi(w[0]);
        v[2] = bf16lo(w[1]);
        v[3] = bf16hi(w[1]);
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)p + off);
        v[0] = a[0];
        v[1] = a[1];
        v[2] = a[2];
        v[3] = a[3];
    }
}

__device__ __forceinline__ void store4(void *p, int32_t type, int64_t off, const float v[4]) {
    if (type == GE_BF16) {
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        *(u32x2 *)((uint16_t *)p + off) = w;
    } else {
        *(f32x4 *)((float *)p + off) = f32x4{v[0], v[1], v[2], v[3]};
    }
}

template <int ACT>
__device__ __forceinline__ void epi4(const EpiArgs &e, float v[4], int64_t m, int64_t n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= e.alpha;
    if (e.flags & GE_FLAG_C) {
        float c[4];
        load4(e.C, e.c_type, m * e.ldc + n, c);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf(e.beta, c[i], v[i]);
    }
    if (e.flags & GE_FLAG_BIAS) {
        float b[4];
        load4(e.bias, e.bias_type, n, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += b[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = activate<ACT>(v[i]);
    if (e.flags & GE_FLAG_RESIDUAL) {
        float r[4];
        load4(e.R, e.r_type, m * e.ldr + n, r);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += r[i];
    }
    store4(e.D, e.d_type, m * e.ldd + n, v);
}

// Two horizontally adjacent 16x16 accumulator tiles x (columns c..c+15) and
// y (c+16..c+31), in the fragment layout where lane row g = lane / 16 holds
// columns 4g..4g+3 of its tile, become eight consecutive columns per lane:
// lane row g ends up with columns c + 8g .. c + 8g + 7.  Two lane-row swaps
// per register do it: rows 2,3 of x trade with rows 0,1 of y, then odd rows
// of the first result trade with even rows of the second.
// Inline assembly: each swap rewrites both of its registers, as the operands
// state (this compiler's two-result swap builtins keep only the first).
__device__ __forceinline__ void pair_to_cols8(const f32x4 &x, const f32x4 &y, float v[8]) {
    // (scalar copies: neither vector elements nor single-element bit casts are used as asm or
    // bit-cast operands, since this compiler reads element 0 for both)
    const u32x4 xu = __builtin_bit_cast(u32x4, x), yu = __builtin_bit_cast(u32x4, y);
    uint32_t a0 = xu[0], a1 = xu[1], a2 = xu[2], a3 = xu[3], b0 = yu[0], b1 = yu[1], b2 = yu[2], b3 = yu[3];
    asm volatile("s_nop 1\n\t"
                 "v_permlane32_swap_b32 %0, %4\n\tv_permlane32_swap_b32 %1, %5\n\t"
                 "v_permlane32_swap_b32 %2, %6\n\tv_permlane32_swap_b32 %3, %7\n\t"
                 "v_permlane16_swap_b32 %0, %4\n\tv_permlane16_swap_b32 %1, %5\n\t"
                 "v_permlane16_swap_b32 %2, %6\n\tv_permlane16_swap_b32 %3, %7"
                 : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3));
    v[0] = __builtin_bit_cast(float, a0);
    v[1] = __builtin_bit_cast(float, a1);
    v[2] = __builtin_bit_cast(float, a2);
    v[3] = __builtin_bit_cast(float, a3);
    v[4] = __builtin_bit_cast(float, b0);
    v[5] = __builtin_bit_cast(float, b1);
    v[6] = __builtin_bit_cast(float, b2);
    v[7] = __builtin_bit_cast(float, b3);
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 &w, float v[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16lo(w[i]);
        v[2 * i + 1] = bf16hi(w[i]);
    }
}

// Buffer resource over a row-major bf16 matrix: rows below M, reads past it
// give zeros and writes past it are dropped.  Absent operands get an empty
// range, so their loads return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mat_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Epilogue of a wave's MT x NT grid of 16x16 tiles when D, C, R and bias are
// all bf16 (the common case): each lane owns 8 consecutive columns per tile
// pair, so every access is 16 bytes.  The C and R rows of tile row i + 2 are
// fetched while tile row i is computed; the code has no branches, so the
// memory waits count exactly (absent terms read zeros from empty buffers and
// add nothing).  mrow: this lane's row in tile row 0; ncol: its first column
// in tile pair 0 (tile pairs are 32 columns apart).  Needs the byte extent of
// C, R and D below 2^31 (checked by the caller).
template <int ACT, bool HAS_C, int MT, int NT>
__device__ __forceinline__ void epilogue_bf16(const EpiArgs &e, f32x4 (&acc)[MT][NT], int M, int N, int mrow,
                                              int ncol) {
    constexpr int NP = NT / 2, DEPTH = 2;
    static_assert(NT % 2 == 0, "tile pairs");
    const bool has_b = e.flags & GE_FLAG_BIAS, has_r = e.flags & GE_FLAG_RESIDUAL;
    const auto rc = mat_rsrc(e.C, HAS_C ? ((int64_t)(M - 1) * e.ldc + N) * 2 : 0);
    const auto rr = mat_rsrc(e.R, has_r ? ((int64_t)(M - 1) * e.ldr + N) * 2 : 0);
    const auto rb = mat_rsrc(e.bias, has_b ? (int64_t)N * 2 : 0);
    const auto rd = mat_rsrc(e.D, ((int64_t)(M - 1) * e.ldd + N) * 2);
    u32x4 cv[DEPTH + 1][NP], rv[DEPTH + 1][NP];
    auto fetch = [&](int i, u32x4 (&c)[NP], u32x4 (&r)[NP]) {
        const int m = mrow + 16 * i;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int n = ncol + 32 * q;
            const bool ok = m < M && n < N;
            if constexpr (HAS_C)
                c[q] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? (int)(((int64_t)m * e.ldc + n) * 2) : (int)OOB, 0, 0);
            r[q] = __builtin_amdgcn_raw_buffer_load_b128(rr, ok ? (int)(((int64_t)m * e.ldr + n) * 2) : (int)OOB, 0, 0);
        }
    };
    u32x4 braw[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int n = ncol + 32 * q;
        braw[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, n < N ? n * 2 : (int)OOB, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < DEPTH && i < MT; ++i) fetch(i, cv[i], rv[i]);
    float bias[NP][8];  // widened once
#pragma unroll
    for (int q = 0; q < NP; ++q) bf16x8_to_f32(braw[q], bias[q]);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        if (i + DEPTH < MT) fetch(i + DEPTH, cv[(i + DEPTH) % (DEPTH + 1)], rv[(i + DEPTH) % (DEPTH + 1)]);
        const int m = mrow + 16 * i;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int n = ncol + 32 * q;
            float v[8], r[8];
            pair_to_cols8(acc[i][2 * q], acc[i][2 * q + 1], v);
            bf16x8_to_f32(rv[i % (DEPTH + 1)][q], r);
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = fmaf(e.alpha, v[t], bias[q][t]);
            if constexpr (HAS_C) {
                float c[8];
                bf16x8_to_f32(cv[i % (DEPTH + 1)][q], c);
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = fmaf(e.beta, c[t], v[t]);
            }
            u32x4 w;
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = activate<ACT>(v[t]) + r[t];
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(v[2 * t], v[2 * t + 1]);
            const bool ok = m < M && n < N;
            __builtin_amdgcn_raw_buffer_store_b128(w, rd, ok ? (int)(((int64_t)m * e.ldd + n) * 2) : (int)OOB, 0, 0);
        }
    }
}

// SwiGLU store: silu(g) * u over the same 16-byte column groups.
template <int MT, int NT>
__device__ __forceinline__ void epilogue_swiglu(const EpiArgs &e, f32x4 (&g)[MT][NT], f32x4 (&u)[MT][NT], int M,
                                                int N, int mrow, int ncol) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = mrow + 16 * i;
#pragma unroll
        for (int q = 0; q < NT / 2; ++q) {
            const int n = ncol + 32 * q;
            float vg[8], vu[8];
            pair_to_cols8(g[i][2 * q], g[i][2 * q + 1], vg);
            pair_to_cols8(u[i][2 * q], u[i][2 * q + 1], vu);
            u32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                w[t] = pack_bf16x2(activate<GE_ACT_SILU>(vg[2 * t]) * vu[2 * t],
                                   activate<GE_ACT_SILU>(vg[2 * t + 1]) * vu[2 * t + 1]);
            if (m < M && n < N) *(u32x4 *)((uint16_t *)e.D + (int64_t)m * e.ldd + n) = w;
        }
    }
}

__host__ __device__ inline bool al16(const void *q) { return ((uintptr_t)q & 15) == 0; }

// the epilogue operands allow 16-byte accesses
inline bool epi_ok(const Problem &p) {
    const EpiArgs &e = p.epi;
    auto ok_mat = [](const void *q, int32_t type, int64_t ld) {
        return al16(q) && ((ld * (type == GE_BF16 ? 2 : 4)) % 16) == 0;
    };
    if (!ok_mat(e.D, e.d_type, e.ldd)) return false;
    if ((e.flags & GE_FLAG_C) && !ok_mat(e.C, e.c_type, e.ldc)) return false;
    if ((e.flags & GE_FLAG_RESIDUAL) && !ok_mat(e.R, e.r_type, e.ldr)) return false;
    if ((e.flags & GE_FLAG_BIAS) && !al16(e.bias)) return false;
    return true;
}
