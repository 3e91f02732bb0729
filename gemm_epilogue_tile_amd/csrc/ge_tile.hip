// ge_tile.hip -- large-tile bf16 MFMA kernel with the epilogue in the store path.
//
// One 256-thread workgroup (four waves) owns a BM x BN output tile and its
// whole K reduction, so the epilogue needs nothing from other workgroups
// (page "kernel fusion" wiki: the activation is applied to each output tile
// before it leaves the compute unit; page "Fusion and Epilogues": the ending
// is applied to the accumulators on the way to their single store).
//
// Main loop, per 64-deep K step:
//   global -> registers  128-bit buffer loads (out-of-range rows/chunks read 0)
//                        of the NEXT step, issued before this step's MFMAs;
//   registers -> LDS     A rows stored as-is; B ([K, N] row-major) is
//                        transposed 8x8 in registers so that LDS holds B^T
//                        with the reduction index contiguous, like A;
//                        16-byte chunks XOR-swizzled (chunk ^ f(row),
//                        f(row) = (row ^ row >> 3) & 7) so that both the
//                        128-bit writes and the fragment reads are free of
//                        bank conflicts;
//   LDS -> MFMA          ds_read_b128 fragments, v_mfma_f32_16x16x32_bf16
//                        with fp32 accumulators.  B is the first MFMA
//                        operand, so each lane ends up holding four
//                        consecutive output columns of one row.
// Two LDS stages (double buffering), one barrier per K step.
//
// Epilogue: alpha*acc + beta*C + bias -> activation -> + R (or silu(g)*u for
// the dual product), 4 consecutive columns per lane, one rounding to the
// output type, one store.
//
// Workgroup -> tile map: consecutive workgroup ids land on different XCDs
// (round-robin dispatch), so ids are first regrouped so that each XCD owns a
// contiguous run of tiles, then runs are laid out in bands of GROUP_M tile
// rows: the tiles one XCD works on at a time share A rows and B columns in
// that XCD's L2.

#include "ge_launch.hpp"

namespace ge {
namespace {

constexpr int T_THREADS = 256;
constexpr int T_BK = 64;
constexpr int GROUP_M = 4;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

constexpr uint32_t OOB = 0x80000000u;  // beyond any buffer this kernel builds (< 2^31 bytes)

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

// even / odd bf16 halves of two dwords, packed (x supplies the low half)
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return (x & 0xffffu) | (y << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return (x >> 16) | (y & 0xffff0000u); }

template <int BM, int BN, int WM, int WN, bool DUAL, bool B_NK>
struct Cfg {
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int MT = WTM / 16, NT = WTN / 16;   // 16x16 MFMA tiles per wave
    static constexpr int NB = DUAL ? 2 : 1;
    static constexpr int A_BYTES = BM * T_BK * 2;
    static constexpr int B_BYTES = BN * T_BK * 2;
    static constexpr int STAGE = A_BYTES + NB * B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int A_LOADS = A_BYTES / 16 / T_THREADS;  // 16-byte loads per thread
    static constexpr int B_LOADS = B_BYTES / 16 / T_THREADS;
    static constexpr int KB_ROWS = BN / 32;                   // KN: k rows per thread block (8 or 4)
    static_assert(WM * WN == 4, "four waves");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(BM % 32 == 0 && A_LOADS * T_THREADS * 16 == A_BYTES, "A loads");
    static_assert(B_NK || BN == 256 || BN == 128, "KN transpose blocks");
};

template <int BM, int BN, int WM, int WN, bool DUAL, bool B_NK>
__global__ __attribute__((amdgpu_flat_work_group_size(T_THREADS, T_THREADS), amdgpu_waves_per_eu(1, 1)))
void tile_kernel(Problem p) {
    using C = Cfg<BM, BN, WM, WN, DUAL, B_NK>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile selection (XCD-aware) ----
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (t / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- per-thread load assignment ----
    // A (and B^T when B_NK): thread -> 16-byte chunk tid%8 of rows tid/8 + 32 i
    const int a_chunk = tid & 7, a_row = tid >> 3;
    // B [K, N]: thread -> column block nb (8 columns) and KB_ROWS k rows starting kb * KB_ROWS
    const int b_nb = tid % (BN / 8), b_kb = tid / (BN / 8);

    const int nk = (p.K + T_BK - 1) / T_BK;
    const int64_t lda_b = p.lda * 2, ldb_b = p.ldb * 2;

    u32x4 ra[C::A_LOADS];
    u32x4 rb[C::NB][C::B_LOADS];

    auto load_stage = [&](int ks) {
        const int k0 = ks * T_BK;
        {
            const char *base = (const char *)p.A + ((int64_t)m0 * p.lda + k0) * 2;
            const int64_t rem = ((int64_t)(p.M - 1 - m0) * p.lda + (p.K - k0)) * 2;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(base, rem > 0 ? (uint32_t)rem : 0u);
            const bool kin = k0 + a_chunk * 8 < p.K;
#pragma unroll
            for (int i = 0; i < C::A_LOADS; ++i) {
                const uint32_t off = (uint32_t)((a_row + 32 * i) * lda_b) + a_chunk * 16;
                ra[i] = bload(r, kin ? off : OOB);
            }
        }
#pragma unroll
        for (int d = 0; d < C::NB; ++d) {
            const void *B = d == 0 ? p.B : p.B2;
            if constexpr (B_NK) {
                const char *base = (const char *)B + ((int64_t)n0 * p.ldb + k0) * 2;
                const int64_t rem = ((int64_t)(p.N - 1 - n0) * p.ldb + (p.K - k0)) * 2;
                const __amdgpu_buffer_rsrc_t r = make_rsrc(base, rem > 0 ? (uint32_t)rem : 0u);
                const bool kin = k0 + a_chunk * 8 < p.K;
#pragma unroll
                for (int i = 0; i < C::B_LOADS; ++i) {
                    const uint32_t off = (uint32_t)((a_row + 32 * i) * ldb_b) + a_chunk * 16;
                    rb[d][i] = bload(r, kin ? off : OOB);
                }
            } else {
                const char *base = (const char *)B + ((int64_t)k0 * p.ldb + n0) * 2;
                const int64_t rem = ((int64_t)(p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2;
                const __amdgpu_buffer_rsrc_t r = make_rsrc(base, rem > 0 ? (uint32_t)rem : 0u);
                const bool nin = n0 + b_nb * 8 < p.N;
#pragma unroll
                for (int i = 0; i < C::B_LOADS; ++i) {
                    const uint32_t off = (uint32_t)((b_kb * C::KB_ROWS + i) * ldb_b) + b_nb * 16;
                    rb[d][i] = bload(r, nin ? off : OOB);
                }
            }
        }
    };

    auto store_stage = [&](int buf) {
        char *sA = smem + buf * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) *(u32x4 *)(sA + swz(a_row + 32 * i, a_chunk)) = ra[i];
#pragma unroll
        for (int d = 0; d < C::NB; ++d) {
            char *sB = sA + C::A_BYTES + d * C::B_BYTES;
            if constexpr (B_NK) {
#pragma unroll
                for (int i = 0; i < C::B_LOADS; ++i) *(u32x4 *)(sB + swz(a_row + 32 * i, a_chunk)) = rb[d][i];
            } else if constexpr (C::KB_ROWS == 8) {
                // 8 k rows x 8 columns -> for each column, its 8 k values (one 16-byte chunk)
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    u32x4 lo, hi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        lo[q] = pack_lo(rb[d][2 * q][dw], rb[d][2 * q + 1][dw]);
                        hi[q] = pack_hi(rb[d][2 * q][dw], rb[d][2 * q + 1][dw]);
                    }
                    *(u32x4 *)(sB + swz(b_nb * 8 + 2 * dw, b_kb)) = lo;
                    *(u32x4 *)(sB + swz(b_nb * 8 + 2 * dw + 1, b_kb)) = hi;
                }
            } else {
                // 4 k rows x 8 columns -> for each column, 4 k values (half a chunk)
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    u32x2 lo, hi;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        lo[q] = pack_lo(rb[d][2 * q][dw], rb[d][2 * q + 1][dw]);
                        hi[q] = pack_hi(rb[d][2 * q][dw], rb[d][2 * q + 1][dw]);
                    }
                    const int half = (b_kb & 1) * 8;
                    *(u32x2 *)(sB + swz(b_nb * 8 + 2 * dw, b_kb >> 1) + half) = lo;
                    *(u32x2 *)(sB + swz(b_nb * 8 + 2 * dw + 1, b_kb >> 1) + half) = hi;
                }
            }
        }
    };

    f32x4 acc[C::NB][C::MT][C::NT];
#pragma unroll
    for (int d = 0; d < C::NB; ++d)
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) acc[d][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15, fchunk = lane >> 4;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) load_stage(ks + 1);
        const char *sA = smem + buf * C::STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 af[C::MT];
#pragma unroll
            for (int i = 0; i < C::MT; ++i)
                af[i] = *(const bf16x8 *)(sA + swz(wm * C::WTM + i * 16 + frow, kk * 4 + fchunk));
#pragma unroll
            for (int d = 0; d < C::NB; ++d) {
                const char *sB = sA + C::A_BYTES + d * C::B_BYTES;
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    const bf16x8 bfr = *(const bf16x8 *)(sB + swz(wn * C::WTN + j * 16 + frow, kk * 4 + fchunk));
#pragma unroll
                    for (int i = 0; i < C::MT; ++i) acc[d][i][j] = mfma_bf16(bfr, af[i], acc[d][i][j]);
                }
            }
        }
        if (ks + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows m, columns n..n+3 of each 16x16 tile ----
    const EpiArgs &e = p.epi;
    const int mbase = m0 + wm * C::WTM + frow;
    const int nbase = n0 + wn * C::WTN + fchunk * 4;
    if constexpr (DUAL) {
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) {
                const int m = mbase + i * 16, n = nbase + j * 16;
                if (m < p.M && n < p.N) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = activate<GE_ACT_SILU>(acc[0][i][j][r]) * acc[1][i][j][r];
                    store4(e.D, e.d_type, (int64_t)m * e.ldd + n, v);
                }
            }
    } else {
        with_act(e.act, [&](auto ACTC) {
            constexpr int ACT = decltype(ACTC)::value;
#pragma unroll
            for (int i = 0; i < C::MT; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    const int m = mbase + i * 16, n = nbase + j * 16;
                    if (m < p.M && n < p.N) {
                        float v[4] = {acc[0][i][j][0], acc[0][i][j][1], acc[0][i][j][2], acc[0][i][j][3]};
                        epi4<ACT>(e, v, m, n);
                    }
                }
        });
    }
}

template <int BM, int BN, int WM, int WN, bool DUAL, bool B_NK>
hipError_t launch_cfg(const Problem &p, hipStream_t s) {
    using C = Cfg<BM, BN, WM, WN, DUAL, B_NK>;
    auto k = tile_kernel<BM, BN, WM, WN, DUAL, B_NK>;
    static bool attr_set = false;  // benign race: every thread sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(k, dim3(tiles), dim3(T_THREADS), C::LDS, s, p);
    return hipGetLastError();
}

bool al16(const void *q) { return ((uintptr_t)q & 15) == 0; }

bool epi_ok(const Problem &p) {
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

}  // namespace

bool tile_supported(const Problem &p) {
    if (p.ab_type != GE_BF16 || p.mode == MODE_W4) return false;
    if (p.M < 128) return false;
    // buffer offsets are 31-bit: operands below 2 GiB
    const int64_t a_bytes = ((int64_t)(p.M - 1) * p.lda + p.K) * 2;
    const int64_t b_bytes = (p.b_layout == GE_LAYOUT_KN ? (int64_t)(p.K - 1) * p.ldb + p.N
                                                        : (int64_t)(p.N - 1) * p.ldb + p.K) * 2;
    if (a_bytes >= (1ll << 31) || b_bytes >= (1ll << 31)) return false;
    if ((p.K & 7) || (p.N & 7) || (p.lda & 7) || (p.ldb & 7)) return false;
    if (!al16(p.A) || !al16(p.B) || (p.mode == MODE_SWIGLU && !al16(p.B2))) return false;
    if (p.mode == MODE_SWIGLU && p.b_layout != GE_LAYOUT_KN) return false;
    return epi_ok(p);
}

const char *tile_kernel_name(const Problem &p) {
    if (p.mode == MODE_SWIGLU) return "tile_swiglu_256x128x64";
    return p.b_layout == GE_LAYOUT_NK ? "tile_nk_256x256x64" : "tile_kn_256x256x64";
}

hipError_t launch_tile(const Problem &p, int, hipStream_t s) {
    if (!tile_supported(p)) return hipErrorInvalidValue;
    if (p.mode == MODE_SWIGLU) return launch_cfg<256, 128, 2, 2, true, false>(p, s);
    if (p.b_layout == GE_LAYOUT_NK) return launch_cfg<256, 256, 2, 2, false, true>(p, s);
    return launch_cfg<256, 256, 2, 2, false, false>(p, s);
}

}  // namespace ge
