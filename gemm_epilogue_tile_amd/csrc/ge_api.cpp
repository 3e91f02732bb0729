// ge_api.cpp -- the C ABI: descriptor validation, planning (kernel choice),
// and the run entry points.  Host code only; kernels live in the .hip units.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "gemm_epi.h"
#include "ge_launch.hpp"

using namespace ge;

namespace {

thread_local std::string g_last_error;

ge_status fail(ge_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ge_status ok() {
    g_last_error.clear();
    return GE_OK;
}

ge_status hip_status(hipError_t e, const char *what) {
#ifdef GE_DEBUG_SYNC
    // race-guard build: every call completes on the device before it returns, so a kernel fault is
    // reported by the call that launched it
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipGetLastError();
#endif
    if (e == hipSuccess) return ok();
    return fail(GE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_float_type(int32_t t) { return t == GE_F32 || t == GE_BF16; }
size_t type_size(int32_t t) { return t == GE_F32 ? 4 : 2; }

}  // namespace

struct ge_plan {
    ge_desc d;
    int32_t kind;
    int device;
    int cu_count;
    int64_t lda, ldb, ldc, ldd, ldr, ld_s;
    int32_t group;
    const char *kernel;  // fused kernel chosen for aligned inputs
    int32_t split;       // K splits of the 8-bit streaming kernel (1: none)
    int32_t scratch_use; // what scratch holds: SCRATCH_NONE / SCRATCH_SPLIT / SCRATCH_SK / SCRATCH_TILE_SPLIT
    void *scratch;       // device scratch owned by the plan, or NULL
    size_t scratch_bytes;
};

namespace {

// GE_LOG=1 in the environment: each plan prints its kernel choice to stderr (read once)
bool log_enabled() {
    static const bool on = [] {
        const char *v = std::getenv("GE_LOG");
        return v && v[0] == '1';
    }();
    return on;
}

// plan scratch: the 8-bit kernel's split tiles and counters, or the stream-K decode kernel's tiles
// and counters
enum { SCRATCH_NONE = 0, SCRATCH_SPLIT = 1, SCRATCH_SK = 3, SCRATCH_TILE_SPLIT = 4, SCRATCH_SWIGLU = 5 };

int32_t wfmt_of(const ge_desc &d) {
    return d.b_type == GE_U8 ? WFMT_U8 : d.b_type == GE_FP8E4M3 ? WFMT_FP8 : WFMT_U4;
}

// Fill a Problem from a plan and the run's pointers.
Problem make_problem(const ge_plan *pl, const void *A, const void *B, const void *B2, const void *scales,
                     const void *C, const void *bias, const void *R, void *D) {
    const ge_desc &d = pl->d;
    Problem p{};
    p.M = d.M;
    p.N = d.N;
    p.K = d.K;
    p.mode = pl->kind == GE_KIND_SWIGLU ? MODE_SWIGLU : pl->kind == GE_KIND_W4 ? MODE_W4 : MODE_GENERIC;
    p.ab_type = d.a_type;
    p.b_layout = pl->kind == GE_KIND_GENERIC ? d.b_layout : GE_LAYOUT_KN;
    p.A = A;
    p.B = B;
    p.B2 = B2;
    p.scales = scales;
    p.lda = pl->lda;
    p.ldb = pl->ldb;
    p.ld_s = pl->ld_s;
    p.group = pl->group;
    p.zero_point = d.zero_point;
    p.lo_first = (d.flags & GE_FLAG_NIBBLE_LO_FIRST) ? 1 : 0;
    EpiArgs &e = p.epi;
    e.alpha = d.alpha;
    e.beta = d.beta;
    e.C = C;
    e.bias = bias;
    e.R = R;
    e.D = D;
    e.ldc = pl->ldc;
    e.ldr = pl->ldr;
    e.ldd = pl->ldd;
    e.c_type = d.c_type;
    e.bias_type = d.bias_type;
    e.r_type = d.r_type;
    e.d_type = d.d_type;
    e.act = pl->kind == GE_KIND_SWIGLU ? GE_ACT_NONE : d.act;
    uint32_t f = 0;
    p.w4_packed = (pl->kind == GE_KIND_W4 && (d.flags & GE_FLAG_W4_PREPACKED)) ? 1 : 0;
    p.b_packed = ((pl->kind == GE_KIND_GENERIC || pl->kind == GE_KIND_SWIGLU) && (d.flags & GE_FLAG_B_PREPACKED)) ? 1 : 0;
    p.wfmt = wfmt_of(d);
    // scratch goes only to the kernel it was made for (unfused chains run copies of a plan
    // with another kind)
    p.split = 1;
    const bool split_use = pl->scratch_use == SCRATCH_SPLIT && p.mode == MODE_W4;
    const bool tsplit_use = pl->scratch_use == SCRATCH_TILE_SPLIT && p.mode == MODE_W4;
    const bool sk_use = pl->scratch_use == SCRATCH_SK && p.mode == MODE_GENERIC;
    if (pl->scratch && pl->scratch_use == SCRATCH_SWIGLU && p.mode == MODE_SWIGLU) {
        // the gate / up tile pairs of the SwiGLU decode kernels, then one counter per column block
        const int64_t ncb = swiglu_pair_blocks(d.N, pl->cu_count, p.b_packed != 0);
        p.split = 2;
        p.split_ws = (float *)pl->scratch;
        p.split_cnt = (uint32_t *)((char *)pl->scratch + pl->scratch_bytes - ncb * 4);
    }
    if (pl->scratch && (split_use || tsplit_use || sk_use)) {
        p.split = pl->split;
        p.split_ws = (float *)pl->scratch;
        const size_t counters = split_use    ? (size_t)split_counters(p)
                                : tsplit_use ? (size_t)tile_w4_split_counters(p)
                                             : (size_t)((d.N + 127) / 128);
        p.split_cnt = (uint32_t *)((char *)pl->scratch + pl->scratch_bytes - counters * 4);
    }
    if (pl->kind != GE_KIND_SWIGLU) {
        if ((d.flags & GE_FLAG_C) && d.beta != 0.0f) f |= GE_FLAG_C;
        if (d.flags & GE_FLAG_BIAS) f |= GE_FLAG_BIAS;
        if (d.flags & GE_FLAG_RESIDUAL) f |= GE_FLAG_RESIDUAL;
    }
    e.flags = f;
    return p;
}

// Launch the fused kernel for p: the specialised kernels when their
// preconditions (shape, alignment) hold, the general kernel otherwise.
hipError_t launch_fused(const ge_plan *pl, const Problem &p, hipStream_t s) {
    if (skinny_supported(p)) return launch_skinny(p, pl->cu_count, s);
    if (tile_supported(p)) return launch_tile(p, pl->cu_count, s);
    if (p.w4_packed || p.b_packed) return hipErrorInvalidValue;  // only the specialised kernels read packed layouts
    return launch_general(p, pl->cu_count, s);
}

const char *fused_name(const Problem &p, int cu_count, bool scratch = true) {
    if (skinny_supported(p)) return skinny_kernel_name(p, cu_count, scratch);
    if (tile_supported(p)) return tile_kernel_name(p, cu_count);
    return general_kernel_name(p, cu_count);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ge_status check_device(const ge_plan *pl) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev != pl->device)
        return fail(GE_ERR_INVALID_ARG, "plan was made on device %d but device %d is current", pl->device, dev);
    return GE_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// D may alias C or R only exactly; A and B must not overlap D at all.
ge_status check_alias(const ge_plan *pl, const void *A, size_t nA, const void *B, size_t nB,
                      const void *C, const void *R, const void *D) {
    const ge_desc &d = pl->d;
    const size_t nD = ((size_t)(d.M - 1) * pl->ldd + d.N) * type_size(d.d_type);
    if (overlaps(A, nA, D, nD) || overlaps(B, nB, D, nD))
        return fail(GE_ERR_INVALID_ARG, "D overlaps an operand of the product");
    if (C && C != D && (d.flags & GE_FLAG_C) && d.beta != 0.0f) {
        const size_t nC = ((size_t)(d.M - 1) * pl->ldc + d.N) * type_size(d.c_type);
        if (overlaps(C, nC, D, nD)) return fail(GE_ERR_INVALID_ARG, "D partially overlaps C");
    }
    if (C && C == D && pl->ldc != pl->ldd) return fail(GE_ERR_INVALID_ARG, "D aliases C with another stride");
    if (R && R != D && (d.flags & GE_FLAG_RESIDUAL)) {
        const size_t nR = ((size_t)(d.M - 1) * pl->ldr + d.N) * type_size(d.r_type);
        if (overlaps(R, nR, D, nD)) return fail(GE_ERR_INVALID_ARG, "D partially overlaps R");
    }
    if (R && R == D && pl->ldr != pl->ldd) return fail(GE_ERR_INVALID_ARG, "D aliases R with another stride");
    return GE_OK;
}

ge_status check_epi_ptrs(const ge_plan *pl, const void *C, const void *bias, const void *R, const void *D) {
    const ge_desc &d = pl->d;
    if (!D) return fail(GE_ERR_INVALID_ARG, "D is NULL");
    if ((d.flags & GE_FLAG_C) && d.beta != 0.0f && !C) return fail(GE_ERR_INVALID_ARG, "C is NULL");
    if ((d.flags & GE_FLAG_BIAS) && !bias) return fail(GE_ERR_INVALID_ARG, "bias is NULL");
    if ((d.flags & GE_FLAG_RESIDUAL) && !R) return fail(GE_ERR_INVALID_ARG, "R is NULL");
    return GE_OK;
}


// One non-blocking stream per device, made on first use, for the library's own set-up work
// (zeroing plan scratch): waiting for it does not wait for the callers' streams.
constexpr int MAX_DEVICES = 64;
std::mutex g_init_mutex;
hipStream_t g_init_stream[MAX_DEVICES];

hipError_t init_stream(int dev, hipStream_t *out) {
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (!g_init_stream[dev]) {
        hipError_t e = hipStreamCreateWithFlags(&g_init_stream[dev], hipStreamNonBlocking);
        if (e != hipSuccess) {
            g_init_stream[dev] = nullptr;
            return e;
        }
    }
    *out = g_init_stream[dev];
    return hipSuccess;
}

}  // namespace

// Device scratch of gemm_epi_run_noalloc (for callers that cannot allocate): the stream-K decode
// kernel's per-column-block arrival counters (first NOALLOC_COUNTER_BYTES, which must start at zero;
// the kernel re-arms them) and its fp32 partial tiles (the rest).  Every GPU the library runs on
// holds one copy until the process ends; host code uses only the address hipGetSymbolAddress returns
// for the current device, never the array's name.
#define NOALLOC_COUNTER_BYTES (64u << 10)
#define NOALLOC_TILE_BYTES (8u << 20)
static __device__ __align__(256) unsigned char scratch[NOALLOC_COUNTER_BYTES + NOALLOC_TILE_BYTES];

namespace {

void *g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` per device (guarded by g_init_mutex)

__global__ void zero_words_kernel(uint32_t *p, uint32_t n) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Address of this device's scratch; on the first call on a device its counters are cleared by a
// kernel on the caller's stream (a kernel, not a memset, so that a graph capturing this call
// replays correctly).
ge_status noalloc_scratch(int dev, hipStream_t s, unsigned char **out) {
    if (dev < 0 || dev >= MAX_DEVICES) return fail(GE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(GE_ERR_HIP, "hipGetSymbolAddress of the static scratch: %s", hipGetErrorString(e));
        }
        hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, s, (uint32_t *)ptr, NOALLOC_COUNTER_BYTES / 4);
        if ((e = hipGetLastError()) != hipSuccess) return hip_status(e, "clearing the static scratch");
        g_scratch_ptr[dev] = ptr;
    }
    *out = (unsigned char *)g_scratch_ptr[dev];
    return GE_OK;
}

}  // namespace

extern "C" {

void ge_desc_init(ge_desc *d) {
    if (!d) return;
    std::memset(d, 0, sizeof *d);
    d->alpha = 1.0f;
    d->b_layout = GE_LAYOUT_KN;
    d->a_type = d->b_type = d->c_type = d->d_type = d->bias_type = d->r_type = GE_BF16;
    d->scale_type = GE_BF16;
    d->group_size = 128;
    d->zero_point = 8;
}

const char *ge_status_string(ge_status s) {
    switch (s) {
    case GE_OK: return "GE_OK";
    case GE_ERR_INVALID_ARG: return "GE_ERR_INVALID_ARG";
    case GE_ERR_UNSUPPORTED: return "GE_ERR_UNSUPPORTED";
    case GE_ERR_NO_DEVICE: return "GE_ERR_NO_DEVICE";
    case GE_ERR_HIP: return "GE_ERR_HIP";
    case GE_ERR_ALIGN: return "GE_ERR_ALIGN";
    default: return "GE_ERR_UNKNOWN";
    }
}

const char *ge_last_error(void) { return g_last_error.c_str(); }

const char *ge_version(void) { return "0.1.0"; }

ge_status gemm_epi_plan(const ge_desc *dp, int32_t kind, ge_plan **out) {
    if (!dp || !out) return fail(GE_ERR_INVALID_ARG, "descriptor or output pointer is NULL");
    *out = nullptr;
    const ge_desc d = *dp;
    if (kind != GE_KIND_GENERIC && kind != GE_KIND_SWIGLU && kind != GE_KIND_W4)
        return fail(GE_ERR_INVALID_ARG, "unknown kind %d", kind);
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return fail(GE_ERR_INVALID_ARG, "M, N, K must be positive");
    if ((int64_t)d.M * d.N >= (1ll << 31) || (int64_t)d.K * d.N >= (1ll << 31) ||
        (int64_t)d.M * d.K >= (1ll << 31))
        return fail(GE_ERR_UNSUPPORTED, "matrix with 2^31 or more elements");
    if (d.act < GE_ACT_NONE || d.act > GE_ACT_SILU) return fail(GE_ERR_INVALID_ARG, "unknown activation %d", d.act);
    if (d.flags & ~(GE_FLAG_BIAS | GE_FLAG_C | GE_FLAG_RESIDUAL | GE_FLAG_NIBBLE_LO_FIRST | GE_FLAG_W4_PREPACKED |
                    GE_FLAG_B_PREPACKED | GE_FLAG_NO_SCRATCH))
        return fail(GE_ERR_INVALID_ARG, "unknown flag bits 0x%x", d.flags);
    if ((d.flags & GE_FLAG_B_PREPACKED) && kind != GE_KIND_GENERIC && kind != GE_KIND_SWIGLU)
        return fail(GE_ERR_INVALID_ARG, "B_PREPACKED applies to generic and swiglu bf16 plans");
    if (d.b_layout != GE_LAYOUT_KN && d.b_layout != GE_LAYOUT_NK)
        return fail(GE_ERR_INVALID_ARG, "unknown b_layout %d", d.b_layout);
    if (!is_float_type(d.d_type)) return fail(GE_ERR_INVALID_ARG, "d_type must be F32 or BF16");
    if ((d.flags & GE_FLAG_C) && d.beta != 0.0f && !is_float_type(d.c_type))
        return fail(GE_ERR_INVALID_ARG, "c_type must be F32 or BF16");
    if ((d.flags & GE_FLAG_BIAS) && !is_float_type(d.bias_type))
        return fail(GE_ERR_INVALID_ARG, "bias_type must be F32 or BF16");
    if ((d.flags & GE_FLAG_RESIDUAL) && !is_float_type(d.r_type))
        return fail(GE_ERR_INVALID_ARG, "r_type must be F32 or BF16");

    ge_plan pl{};
    pl.d = d;
    pl.kind = kind;
    pl.group = d.group_size ? d.group_size : 128;
    pl.lda = d.lda ? d.lda : d.K;
    pl.ldc = d.ldc ? d.ldc : d.N;
    pl.ldd = d.ldd ? d.ldd : d.N;
    pl.ldr = d.ldr ? d.ldr : d.N;
    if (d.lda < 0 || d.ldb < 0 || d.ldc < 0 || d.ldd < 0 || d.ldr < 0)
        return fail(GE_ERR_INVALID_ARG, "negative leading dimension");
    if (pl.lda < d.K) return fail(GE_ERR_INVALID_ARG, "lda < K");
    if (pl.ldd < d.N) return fail(GE_ERR_INVALID_ARG, "ldd < N");
    if ((d.flags & GE_FLAG_C) && d.beta != 0.0f && pl.ldc < d.N) return fail(GE_ERR_INVALID_ARG, "ldc < N");
    if ((d.flags & GE_FLAG_RESIDUAL) && pl.ldr < d.N) return fail(GE_ERR_INVALID_ARG, "ldr < N");

    if (kind == GE_KIND_GENERIC) {
        if (d.a_type != d.b_type || !is_float_type(d.a_type))
            return fail(GE_ERR_UNSUPPORTED, "generic kind needs a_type == b_type in {F32, BF16}");
        if (d.flags & (GE_FLAG_NIBBLE_LO_FIRST | GE_FLAG_W4_PREPACKED))
            return fail(GE_ERR_INVALID_ARG, "int4 flag on a dense product");
        pl.ldb = d.ldb ? d.ldb : (d.b_layout == GE_LAYOUT_KN ? d.N : d.K);
        if (pl.ldb < (d.b_layout == GE_LAYOUT_KN ? d.N : d.K)) return fail(GE_ERR_INVALID_ARG, "ldb too small");
        if ((d.flags & GE_FLAG_B_PREPACKED) &&
            (d.a_type != GE_BF16 || d.b_layout != GE_LAYOUT_KN || d.M > 32 || d.N % 128 || d.K % 32))
            return fail(GE_ERR_UNSUPPORTED, "prepacked bf16 weights need bf16 KN operands, M <= 32, N %% 128 == 0 "
                                            "and K %% 32 == 0");
    } else if (kind == GE_KIND_SWIGLU) {
        if (d.a_type != GE_BF16 || d.b_type != GE_BF16 || d.d_type != GE_BF16)
            return fail(GE_ERR_UNSUPPORTED, "swiglu needs bf16 X, W and D");
        if (d.b_layout != GE_LAYOUT_KN) return fail(GE_ERR_UNSUPPORTED, "swiglu needs KN weights");
        if (d.act != GE_ACT_NONE || (d.flags & ~(GE_FLAG_B_PREPACKED | GE_FLAG_NO_SCRATCH)) || d.alpha != 1.0f)
            return fail(GE_ERR_UNSUPPORTED, "swiglu takes no extra epilogue");
        if ((d.flags & GE_FLAG_B_PREPACKED) && (d.flags & GE_FLAG_NO_SCRATCH))
            return fail(GE_ERR_UNSUPPORTED, "prepacked swiglu needs the plan's scratch");
        pl.ldb = d.ldb ? d.ldb : d.N;
        if (pl.ldb < d.N) return fail(GE_ERR_INVALID_ARG, "ldb < N");
        if ((d.flags & GE_FLAG_B_PREPACKED) && (d.M > 32 || d.N % 128 || d.K % 32 || pl.ldb != d.N))
            return fail(GE_ERR_UNSUPPORTED, "prepacked swiglu weights need M <= 32, N %% 128 == 0, K %% 32 == 0 and "
                                            "dense weights");
    } else if (d.b_type == GE_U8 || d.b_type == GE_FP8E4M3) {
        if (d.a_type != GE_BF16 || d.scale_type != GE_BF16)
            return fail(GE_ERR_UNSUPPORTED, "8-bit weights need bf16 X and bf16 scales");
        if (d.b_layout != GE_LAYOUT_KN) return fail(GE_ERR_UNSUPPORTED, "8-bit weights are [K, N]");
        if (d.flags & GE_FLAG_NIBBLE_LO_FIRST) return fail(GE_ERR_INVALID_ARG, "nibble order applies to int4 weights only");
        if ((d.flags & GE_FLAG_W4_PREPACKED) && (d.M > 16 || d.N % 128 || d.K % 32))
            return fail(GE_ERR_UNSUPPORTED, "prepacked 8-bit weights need M <= 16, N %% 128 == 0 and K %% 32 == 0");
        if (pl.group != 32 && pl.group != 64 && pl.group != 128 && pl.group != 256)
            return fail(GE_ERR_UNSUPPORTED, "group size %d not in {32, 64, 128, 256}", pl.group);
        if (d.K % pl.group) return fail(GE_ERR_INVALID_ARG, "K %% group != 0");
        if (d.b_type == GE_U8 ? (d.zero_point < 0 || d.zero_point > 255) : d.zero_point != 0)
            return fail(GE_ERR_INVALID_ARG, "zero_point must be in [0, 255] for u8 weights and 0 for fp8");
        pl.ldb = d.ldb ? d.ldb : d.N;
        if (pl.ldb < d.N) return fail(GE_ERR_INVALID_ARG, "ldb < N bytes");
        pl.ld_s = d.N;
    } else {
        if (d.a_type != GE_BF16 || d.b_type != GE_U4X2 || d.scale_type != GE_BF16)
            return fail(GE_ERR_UNSUPPORTED, "w4 needs bf16 X, U4X2 / U8 / FP8E4M3 weights and bf16 scales");
        if (d.b_layout != GE_LAYOUT_KN) return fail(GE_ERR_UNSUPPORTED, "w4 weights are [K, N/2]");
        if (d.N % 2) return fail(GE_ERR_INVALID_ARG, "w4 needs an even N");
        if (pl.group != 32 && pl.group != 64 && pl.group != 128 && pl.group != 256)
            return fail(GE_ERR_UNSUPPORTED, "group size %d not in {32, 64, 128, 256}", pl.group);
        if (d.K % pl.group) return fail(GE_ERR_INVALID_ARG, "K %% group != 0");
        if (d.zero_point < 0 || d.zero_point > 15) return fail(GE_ERR_INVALID_ARG, "zero_point outside [0, 15]");
        pl.ldb = d.ldb ? d.ldb : d.N / 2;
        if (pl.ldb < d.N / 2) return fail(GE_ERR_INVALID_ARG, "ldb < N/2 bytes");
        pl.ld_s = d.N;
        if (d.flags & GE_FLAG_W4_PREPACKED) {
            if (d.N % (d.M <= 32 ? 16 : 128) || d.K % 128 || pl.group > 128 || (d.M > 32 && pl.group != 128))
                return fail(GE_ERR_UNSUPPORTED,
                            "prepacked int4 weights need K %% 128 == 0 and either M <= 32, N %% 16 == 0, group <= 128 "
                            "or N %% 128 == 0, group == 128");
        }
    }

    // device
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        return fail(GE_ERR_NO_DEVICE, "no HIP device visible");
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GE_ERR_NO_DEVICE, "hipGetDevice failed");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(GE_ERR_NO_DEVICE, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(GE_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
    pl.device = dev;
    pl.cu_count = prop.multiProcessorCount;

    // name of the fused kernel for aligned pointers
    Problem p = make_problem(&pl, (const void *)256, (const void *)256, (const void *)256, (const void *)256,
                             (const void *)256, (const void *)256, (const void *)256, (void *)256);
    pl.kernel = fused_name(p, pl.cu_count);

    // device scratch: the 8-bit, the int4 and the bf16 streaming kernels split K over
    // workgroups when the column blocks alone do not fill the GPU
    pl.split = 1;
    pl.scratch_use = SCRATCH_NONE;
    pl.scratch = nullptr;
    pl.scratch_bytes = 0;
    int64_t bytes = 0;
    int32_t use = SCRATCH_NONE;
    if (kind == GE_KIND_W4 && skinny_supported(p)) {
        const int split = w8_split(p, pl.cu_count);
        if (split > 1) {
            bytes = w8_split_scratch_bytes(p, split);
            use = SCRATCH_SPLIT;
            pl.split = split;
        }
    } else if (kind == GE_KIND_W4 && tile_supported(p)) {
        const int split = tile_w4_split(p, pl.cu_count);
        if (split > 1) {
            bytes = tile_w4_split_scratch_bytes(p, split);
            use = SCRATCH_TILE_SPLIT;
            pl.split = split;
        }
    } else if (kind == GE_KIND_GENERIC && skinny_supported(p)) {
        const int slots = bf16_sk_slots(p, pl.cu_count);
        if (slots > 0) {
            bytes = bf16_sk_scratch_bytes(p, slots);
            use = SCRATCH_SK;
            pl.split = slots;
        }
    } else if (kind == GE_KIND_SWIGLU && (d.flags & GE_FLAG_B_PREPACKED)) {
        bytes = swiglu_prepacked_scratch_bytes(d.M, d.N, pl.cu_count);
        use = SCRATCH_SWIGLU;
        pl.split = 2;
        pl.kernel = swiglu_prepacked_name(d.N, pl.cu_count);
    } else if (kind == GE_KIND_SWIGLU && !(d.flags & GE_FLAG_NO_SCRATCH) && swiglu_raw_supported(p)) {
        // decode sizes on raw weights: the gate / up workgroup pairs over the raw layout
        bytes = swiglu_raw_scratch_bytes(d.M, d.N, pl.cu_count);
        use = SCRATCH_SWIGLU;
        pl.split = 2;
        pl.kernel = swiglu_raw_name(d.N, pl.cu_count);
    }
    if (bytes > 0 && (d.flags & GE_FLAG_NO_SCRATCH)) {
        // no device memory: the variant of the kernel that needs none
        pl.kernel = fused_name(p, pl.cu_count, false);
        bytes = 0;
    }
    if (bytes > 0) {
        hipError_t e = hipMalloc(&pl.scratch, (size_t)bytes);
        if (e != hipSuccess) {
            pl.scratch = nullptr;
            (void)hipGetLastError();
            return fail(GE_ERR_HIP,
                        "allocating the plan's %lld bytes of device scratch failed (%s); plans that own scratch "
                        "must be made outside graph capture",
                        (long long)bytes, hipGetErrorString(e));
        }
        // zeroed on a stream of the library's own, waiting for that stream alone (the callers'
        // streams keep running)
        hipStream_t zs = nullptr;
        e = init_stream(dev, &zs);
        if (e == hipSuccess) e = hipMemsetAsync(pl.scratch, 0, (size_t)bytes, zs);
        if (e == hipSuccess) e = hipStreamSynchronize(zs);
        if (e != hipSuccess) {
            (void)hipFree(pl.scratch);
            return hip_status(e, "zeroing the plan's device scratch");
        }
        pl.scratch_use = use;
        pl.scratch_bytes = (size_t)bytes;
        if (use == SCRATCH_TILE_SPLIT) {  // the split kernel's name
            Problem q = p;
            q.split = pl.split;
            pl.kernel = fused_name(q, pl.cu_count);
        }
    } else {
        pl.split = 1;
    }

    ge_plan *h = new (std::nothrow) ge_plan(pl);
    if (!h) {
        if (pl.scratch) (void)hipFree(pl.scratch);
        return fail(GE_ERR_INVALID_ARG, "out of host memory");
    }
    *out = h;
    if (log_enabled()) {
        static const char *kinds[] = {"generic", "swiglu", "w4"};
        std::fprintf(stderr,
                     "ge: plan kind=%s M=%d N=%d K=%d a=%d b=%d d=%d act=%d flags=0x%x group=%d -> kernel=%s "
                     "split=%d scratch=%zu\n",
                     kinds[kind], d.M, d.N, d.K, d.a_type, d.b_type, d.d_type, d.act, (unsigned)d.flags, pl.group,
                     pl.kernel, pl.split, pl.scratch_bytes);
    }
    return ok();
}

ge_status gemm_epi_plan_destroy(ge_plan *plan) {
    if (plan && plan->scratch) {
        int cur = -1;
        const bool have = hipGetDevice(&cur) == hipSuccess;
        if (have && cur != plan->device) (void)hipSetDevice(plan->device);
        (void)hipFree(plan->scratch);
        if (have && cur != plan->device) (void)hipSetDevice(cur);
    }
    delete plan;
    return ok();
}

const char *gemm_epi_plan_kernel(const ge_plan *plan) { return plan ? plan->kernel : ""; }

size_t gemm_epi_plan_scratch_bytes(const ge_plan *plan) { return plan ? plan->scratch_bytes : 0; }

ge_status gemm_epi_run(const ge_plan *pl, const void *A, const void *B, const void *C, const void *bias,
                       const void *R, void *D, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_GENERIC) return fail(GE_ERR_INVALID_ARG, "plan is not a generic plan");
    if (!A || !B) return fail(GE_ERR_INVALID_ARG, "A or B is NULL");
    ge_status st = check_epi_ptrs(pl, C, bias, R, D);
    if (st) return st;
    const ge_desc &d = pl->d;
    const size_t es = type_size(d.a_type);
    const size_t nA = ((size_t)(d.M - 1) * pl->lda + d.K) * es;
    const size_t nB = (d.flags & GE_FLAG_B_PREPACKED) ? (size_t)d.K * d.N * es
                      : (d.b_layout == GE_LAYOUT_KN ? (size_t)(d.K - 1) * pl->ldb + d.N
                                                    : (size_t)(d.N - 1) * pl->ldb + d.K) * es;
    if ((st = check_alias(pl, A, nA, B, nB, C, R, D))) return st;
    if ((st = check_device(pl))) return st;
    const Problem p = make_problem(pl, A, B, nullptr, nullptr, C, bias, R, D);
    if (p.b_packed && !skinny_supported(p))
        return fail(GE_ERR_ALIGN, "prepacked bf16 path needs 16-byte aligned A and B and an lda that is a multiple of 8");
    return hip_status(launch_fused(pl, p, (hipStream_t)stream), "gemm_epi_run launch");
}

ge_status gemm_epi_run_noalloc(const ge_plan *pl, const void *A, const void *B, const void *C, const void *bias,
                               const void *R, void *D, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_GENERIC) return fail(GE_ERR_INVALID_ARG, "plan is not a generic plan");
    if (!A || !B) return fail(GE_ERR_INVALID_ARG, "A or B is NULL");
    ge_status st = check_epi_ptrs(pl, C, bias, R, D);
    if (st) return st;
    const ge_desc &d = pl->d;
    const size_t es = type_size(d.a_type);
    const size_t nA = ((size_t)(d.M - 1) * pl->lda + d.K) * es;
    const size_t nB = (d.flags & GE_FLAG_B_PREPACKED) ? (size_t)d.K * d.N * es
                      : (d.b_layout == GE_LAYOUT_KN ? (size_t)(d.K - 1) * pl->ldb + d.N
                                                    : (size_t)(d.N - 1) * pl->ldb + d.K) * es;
    if ((st = check_alias(pl, A, nA, B, nB, C, R, D))) return st;
    if ((st = check_device(pl))) return st;
    hipStream_t s = (hipStream_t)stream;
    Problem p = make_problem(pl, A, B, nullptr, nullptr, C, bias, R, D);
    p.split = 1;
    p.split_ws = nullptr;
    p.split_cnt = nullptr;
    if (p.b_packed && !skinny_supported(p))
        return fail(GE_ERR_ALIGN, "prepacked bf16 path needs 16-byte aligned A and B and an lda that is a multiple of 8");
    // the kernel a plan with scratch would launch, its tiles and counters in the static scratch
    const int slots = skinny_supported(p) ? bf16_sk_slots(p, pl->cu_count) : 0;
    if (slots > 0) {
        const int64_t ncb = (d.N + 127) / 128;
        const int64_t tiles = bf16_sk_scratch_bytes(p, slots) - ncb * 4;
        if (ncb * 4 > (int64_t)NOALLOC_COUNTER_BYTES || tiles > (int64_t)NOALLOC_TILE_BYTES)
            return fail(GE_ERR_UNSUPPORTED,
                        "this shape needs %lld bytes of partial tiles and %lld counters; the static scratch holds "
                        "%u bytes and %u counters",
                        (long long)tiles, (long long)ncb, NOALLOC_TILE_BYTES, NOALLOC_COUNTER_BYTES / 4);
        unsigned char *base = nullptr;
        if ((st = noalloc_scratch(pl->device, s, &base))) return st;
        p.split = slots;
        p.split_cnt = (uint32_t *)base;
        p.split_ws = (float *)(base + NOALLOC_COUNTER_BYTES);
    }
    return hip_status(launch_fused(pl, p, s), "gemm_epi_run_noalloc launch");
}

ge_status gemm_swiglu_run(const ge_plan *pl, const void *X, const void *Wg, const void *Wu, void *D,
                          void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_SWIGLU) return fail(GE_ERR_INVALID_ARG, "plan is not a swiglu plan");
    if (!X || !Wg || !Wu || !D) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    const ge_desc &d = pl->d;
    const size_t nX = ((size_t)(d.M - 1) * pl->lda + d.K) * 2;
    const size_t nW = ((size_t)(d.K - 1) * pl->ldb + d.N) * 2;
    const size_t nD = ((size_t)(d.M - 1) * pl->ldd + d.N) * 2;
    if (overlaps(X, nX, D, nD) || overlaps(Wg, nW, D, nD) || overlaps(Wu, nW, D, nD))
        return fail(GE_ERR_INVALID_ARG, "D overlaps an input");
    ge_status st;
    if ((st = check_device(pl))) return st;
    if (d.flags & GE_FLAG_B_PREPACKED) {
        if (!pl->scratch || pl->scratch_use != SCRATCH_SWIGLU)
            return fail(GE_ERR_INVALID_ARG, "prepacked swiglu plan has no scratch");
        if (((uintptr_t)X & 15) || (pl->lda & 7) || ((uintptr_t)Wg & 15) || ((uintptr_t)Wu & 15))
            return fail(GE_ERR_ALIGN, "prepacked swiglu needs 16-byte aligned X, Wg and Wu and an lda that is a multiple of 8");
        if (nX >= (1ull << 31) || (int64_t)d.K * 256 >= (1ll << 31))
            return fail(GE_ERR_UNSUPPORTED, "prepacked swiglu addresses X and each weight block with 32-bit offsets");
        const Problem p = make_problem(pl, X, Wg, Wu, nullptr, nullptr, nullptr, nullptr, D);
        return hip_status(launch_swiglu_prepacked(p, pl->cu_count, (hipStream_t)stream), "gemm_swiglu_run launch (prepacked)");
    }
    Problem p = make_problem(pl, X, Wg, Wu, nullptr, nullptr, nullptr, nullptr, D);
    if (pl->scratch_use == SCRATCH_SWIGLU && swiglu_raw_supported(p))
        return hip_status(launch_swiglu_raw(p, pl->cu_count, (hipStream_t)stream), "gemm_swiglu_run launch (pairs)");
    // the tile or general kernel (also when these pointers do not suit the pairs)
    p.split = 1;
    p.split_ws = nullptr;
    p.split_cnt = nullptr;
    return hip_status(launch_fused(pl, p, (hipStream_t)stream), "gemm_swiglu_run launch");
}

ge_status gemm_w4_run(const ge_plan *pl, const void *X, const uint8_t *Wq, const void *scales, const void *C,
                      const void *bias, const void *R, void *D, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_W4) return fail(GE_ERR_INVALID_ARG, "plan is not a w4 plan");
    if (!X || !Wq || !scales) return fail(GE_ERR_INVALID_ARG, "X, Wq or scales is NULL");
    ge_status st = check_epi_ptrs(pl, C, bias, R, D);
    if (st) return st;
    const ge_desc &d = pl->d;
    const size_t nX = ((size_t)(d.M - 1) * pl->lda + d.K) * 2;
    const size_t nW = (size_t)(d.K - 1) * pl->ldb + (d.b_type == GE_U4X2 ? d.N / 2 : d.N);
    if ((st = check_alias(pl, X, nX, Wq, nW, C, R, D))) return st;
    const size_t nS = (size_t)(d.K / pl->group) * d.N * 2;
    const size_t nD = ((size_t)(d.M - 1) * pl->ldd + d.N) * type_size(d.d_type);
    if (overlaps(scales, nS, D, nD)) return fail(GE_ERR_INVALID_ARG, "D overlaps the scales");
    if ((st = check_device(pl))) return st;
    const Problem p = make_problem(pl, X, Wq, nullptr, scales, C, bias, R, D);
    if (p.w4_packed && !skinny_supported(p) && !tile_supported(p))
        return fail(GE_ERR_ALIGN, "prepacked int4 path needs 16-byte aligned X, Wq, D, bias, C, R and "
                                  "leading dimensions that are multiples of 8");
    return hip_status(launch_fused(pl, p, (hipStream_t)stream), "gemm_w4_run launch");
}

// ---------------------------------------------------------------------------
// unfused chains
// ---------------------------------------------------------------------------

ge_status gemm_epi_unfused_workspace_bytes(const ge_plan *pl, size_t *bytes) {
    if (!pl || !bytes) return fail(GE_ERR_INVALID_ARG, "NULL argument");
    const ge_desc &d = pl->d;
    const size_t mn = (size_t)d.M * d.N;
    size_t b = 0;
    if (pl->kind == GE_KIND_SWIGLU) {
        b = 3 * align256(mn * 2);
    } else {
        b = 2 * align256(mn * type_size(d.d_type));
        if (pl->kind == GE_KIND_W4) b += align256((size_t)d.K * d.N * 2);
    }
    *bytes = b;
    return ok();
}

namespace {

// The epilogue of a generic / w4 plan as separate kernels.  T0 holds the plain
// product (d_type, dense); each step reads its input buffer and writes the
// next one; the last step writes D.
hipError_t run_epilogue_chain(const ge_plan *pl, const void *C, const void *bias, const void *R, void *D,
                              void *T0, void *T1, hipStream_t s) {
    const ge_desc &d = pl->d;
    const int32_t t = d.d_type;
    const bool use_scale = d.alpha != 1.0f;
    const bool use_c = (d.flags & GE_FLAG_C) && d.beta != 0.0f;
    const bool use_bias = (d.flags & GE_FLAG_BIAS) != 0;
    const bool use_act = d.act != GE_ACT_NONE;
    const bool use_r = (d.flags & GE_FLAG_RESIDUAL) != 0;
    const int steps = use_scale + use_c + use_bias + use_act + use_r;
    void *bufs[2] = {T0, T1};
    int cur = 0, done = 0;
    auto dst = [&]() -> void * { return ++done == steps ? D : bufs[cur ^ 1]; };
    hipError_t e = hipSuccess;
    if (steps == 0) return launch_ew_copy(d.M, d.N, T0, t, D, t, d.N, s);
    if (use_scale) {
        void *y = dst();
        e = launch_ew_axpby(d.M, d.N, d.alpha, bufs[cur], t, 0.0f, nullptr, t, 0, y, t, s);
        cur ^= 1;
        if (e) return e;
    }
    if (use_c) {
        void *y = dst();
        e = launch_ew_axpby(d.M, d.N, 1.0f, bufs[cur], t, d.beta, C, d.c_type, pl->ldc, y, t, s);
        cur ^= 1;
        if (e) return e;
    }
    if (use_bias) {
        void *y = dst();
        e = launch_ew_bias(d.M, d.N, bufs[cur], t, bias, d.bias_type, y, t, s);
        cur ^= 1;
        if (e) return e;
    }
    if (use_act) {
        void *y = dst();
        e = launch_ew_act(d.M, d.N, d.act, bufs[cur], t, y, t, s);
        cur ^= 1;
        if (e) return e;
    }
    if (use_r) {
        void *y = dst();
        e = launch_ew_add(d.M, d.N, bufs[cur], t, R, d.r_type, pl->ldr, y, t, d.N, s);
        cur ^= 1;
    }
    return e;
}

// plain product into a dense buffer of the output type
Problem plain_problem(const ge_plan *pl, const void *A, const void *B, const void *B2, const void *scales,
                      void *out, int32_t out_type) {
    Problem p = make_problem(pl, A, B, B2, scales, nullptr, nullptr, nullptr, out);
    p.epi.alpha = 1.0f;
    p.epi.beta = 0.0f;
    p.epi.flags = 0;
    p.epi.act = GE_ACT_NONE;
    p.epi.ldd = pl->d.N;
    p.epi.d_type = out_type;
    return p;
}

ge_status check_ws(const ge_plan *pl, void *ws) {
    if (!ws) return fail(GE_ERR_INVALID_ARG, "workspace is NULL");
    if ((uintptr_t)ws & 255) return fail(GE_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (pl->ldd != pl->d.N) return fail(GE_ERR_UNSUPPORTED, "unfused chains write a dense D (ldd == N)");
    return GE_OK;
}

}  // namespace

ge_status gemm_epi_run_unfused(const ge_plan *pl, const void *A, const void *B, const void *C,
                               const void *bias, const void *R, void *D, void *ws, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_GENERIC) return fail(GE_ERR_INVALID_ARG, "plan is not a generic plan");
    if (pl->d.flags & GE_FLAG_B_PREPACKED) return fail(GE_ERR_UNSUPPORTED, "this entry point takes raw weights");
    if (!A || !B) return fail(GE_ERR_INVALID_ARG, "A or B is NULL");
    ge_status st = check_epi_ptrs(pl, C, bias, R, D);
    if (st || (st = check_ws(pl, ws)) || (st = check_device(pl))) return st;
    const ge_desc &d = pl->d;
    const size_t mnb = align256((size_t)d.M * d.N * type_size(d.d_type));
    void *T0 = ws, *T1 = (char *)ws + mnb;
    hipStream_t s = (hipStream_t)stream;
    Problem p = plain_problem(pl, A, B, nullptr, nullptr, T0, d.d_type);
    hipError_t e = launch_fused(pl, p, s);
    if (e == hipSuccess) e = run_epilogue_chain(pl, C, bias, R, D, T0, T1, s);
    return hip_status(e, "gemm_epi_run_unfused");
}

ge_status gemm_swiglu_run_unfused(const ge_plan *pl, const void *X, const void *Wg, const void *Wu, void *D,
                                  void *ws, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_SWIGLU) return fail(GE_ERR_INVALID_ARG, "plan is not a swiglu plan");
    if (!X || !Wg || !Wu || !D) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    if (pl->d.flags & GE_FLAG_B_PREPACKED)
        return fail(GE_ERR_UNSUPPORTED, "the unfused swiglu chain reads the raw [K, N] weights");
    ge_status st;
    if ((st = check_ws(pl, ws)) || (st = check_device(pl))) return st;
    const ge_desc &d = pl->d;
    const int64_t mn = (int64_t)d.M * d.N;
    const size_t mnb = align256((size_t)mn * 2);
    void *G = ws, *U = (char *)ws + mnb, *S = (char *)ws + 2 * mnb;
    hipStream_t s = (hipStream_t)stream;
    // gate and up products as two plain GEMMs (generic kind, bf16 out)
    ge_plan gp = *pl;
    gp.kind = GE_KIND_GENERIC;
    gp.d.b_layout = GE_LAYOUT_KN;
    Problem pg = plain_problem(&gp, X, Wg, nullptr, nullptr, G, GE_BF16);
    Problem pu = plain_problem(&gp, X, Wu, nullptr, nullptr, U, GE_BF16);
    hipError_t e = launch_fused(&gp, pg, s);
    if (!e) e = launch_fused(&gp, pu, s);
    if (!e) e = launch_ew_sigmoid(mn, G, S, s);   // s = sigmoid(g)
    if (!e) e = launch_ew_mul(mn, G, S, S, s);    // h = g * s  (silu)
    if (!e) e = launch_ew_mul(mn, S, U, D, s);    // out = h * u
    return hip_status(e, "gemm_swiglu_run_unfused");
}

ge_status gemm_w4_run_unfused(const ge_plan *pl, const void *X, const uint8_t *Wq, const void *scales,
                              const void *C, const void *bias, const void *R, void *D, void *ws, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_W4) return fail(GE_ERR_INVALID_ARG, "plan is not a w4 plan");
    if (pl->d.flags & GE_FLAG_W4_PREPACKED) return fail(GE_ERR_UNSUPPORTED, "this entry point takes raw (not prepacked) weights");
    if (!X || !Wq || !scales) return fail(GE_ERR_INVALID_ARG, "X, Wq or scales is NULL");
    ge_status st = check_epi_ptrs(pl, C, bias, R, D);
    if (st || (st = check_ws(pl, ws)) || (st = check_device(pl))) return st;
    const ge_desc &d = pl->d;
    const size_t mnb = align256((size_t)d.M * d.N * type_size(d.d_type));
    void *W = ws;
    void *T0 = (char *)ws + align256((size_t)d.K * d.N * 2);
    void *T1 = (char *)T0 + mnb;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_w4_dequant(d.K, d.N, Wq, pl->ldb, scales, pl->ld_s, pl->group, d.zero_point,
                                     (d.flags & GE_FLAG_NIBBLE_LO_FIRST) ? 1 : 0, W, s, wfmt_of(d));
    if (!e) {
        ge_plan gp = *pl;
        gp.kind = GE_KIND_GENERIC;
        gp.d.b_type = GE_BF16;
        gp.d.b_layout = GE_LAYOUT_KN;
        gp.ldb = d.N;
        Problem p = plain_problem(&gp, X, W, nullptr, nullptr, T0, d.d_type);
        e = launch_fused(&gp, p, s);
    }
    if (!e) e = run_epilogue_chain(pl, C, bias, R, D, T0, T1, s);
    return hip_status(e, "gemm_w4_run_unfused");
}

ge_status gemm_w4_dequant_run(const ge_plan *pl, const uint8_t *Wq, const void *scales, void *W, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_W4) return fail(GE_ERR_INVALID_ARG, "plan is not a w4 plan");
    if (pl->d.flags & GE_FLAG_W4_PREPACKED) return fail(GE_ERR_UNSUPPORTED, "this entry point takes raw (not prepacked) weights");
    if (!Wq || !scales || !W) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    ge_status st;
    if ((st = check_device(pl))) return st;
    const ge_desc &d = pl->d;
    return hip_status(launch_w4_dequant(d.K, d.N, Wq, pl->ldb, scales, pl->ld_s, pl->group, d.zero_point,
                                        (d.flags & GE_FLAG_NIBBLE_LO_FIRST) ? 1 : 0, W, (hipStream_t)stream,
                                        wfmt_of(d)),
                      "gemm_w4_dequant_run");
}

ge_status gemm_w4_prepack(const ge_plan *pl, const uint8_t *Wq, uint8_t *Wp, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_W4) return fail(GE_ERR_INVALID_ARG, "plan is not a w4 plan");
    if (!Wq || !Wp) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    const ge_desc &d = pl->d;
    if (d.b_type == GE_U8 || d.b_type == GE_FP8E4M3) {
        if (d.N % 128 || d.K % 32) return fail(GE_ERR_UNSUPPORTED, "8-bit prepack needs N %% 128 == 0 and K %% 32 == 0");
        if (((uintptr_t)Wp & 15) || ((uintptr_t)Wq & 7) || (pl->ldb & 7))
            return fail(GE_ERR_ALIGN, "8-bit prepack needs an 8-byte aligned Wq and ldb and a 16-byte aligned Wp");
        const size_t nq8 = (size_t)(d.K - 1) * pl->ldb + d.N, np8 = (size_t)d.K * d.N;
        if (overlaps(Wq, nq8, Wp, np8)) return fail(GE_ERR_INVALID_ARG, "Wp overlaps Wq");
        ge_status st8;
        if ((st8 = check_device(pl))) return st8;
        return hip_status(launch_w8_prepack(d.K, d.N, Wq, pl->ldb, Wp, (hipStream_t)stream), "gemm_w4_prepack");
    }
    if (d.b_type != GE_U4X2) return fail(GE_ERR_UNSUPPORTED, "prepacking applies to int4 and 8-bit weights");
    if (d.N % 16 || d.K % 128) return fail(GE_ERR_UNSUPPORTED, "prepack needs N %% 16 == 0 and K %% 128 == 0");
    if ((uintptr_t)Wp & 15) return fail(GE_ERR_ALIGN, "Wp must be 16-byte aligned");
    const size_t nq = (size_t)(d.K - 1) * pl->ldb + d.N / 2, np = (size_t)d.K * d.N / 2;
    if (overlaps(Wq, nq, Wp, np)) return fail(GE_ERR_INVALID_ARG, "Wp overlaps Wq");
    ge_status st;
    if ((st = check_device(pl))) return st;
    return hip_status(launch_w4_prepack(d.K, d.N, Wq, pl->ldb, (d.flags & GE_FLAG_NIBBLE_LO_FIRST) ? 1 : 0, Wp,
                                        (hipStream_t)stream),
                      "gemm_w4_prepack");
}

ge_status gemm_b_prepack(const ge_plan *pl, const void *B, void *Bp, void *stream) {
    if (!pl) return fail(GE_ERR_INVALID_ARG, "plan is NULL");
    if (pl->kind != GE_KIND_GENERIC && pl->kind != GE_KIND_SWIGLU)
        return fail(GE_ERR_INVALID_ARG, "plan is not a generic or swiglu plan");
    if (!B || !Bp) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    const ge_desc &d = pl->d;
    if (d.b_type != GE_BF16 || d.b_layout != GE_LAYOUT_KN)
        return fail(GE_ERR_UNSUPPORTED, "prepacking applies to bf16 [K, N] weights");
    if (d.N % 128 || d.K % 32) return fail(GE_ERR_UNSUPPORTED, "prepack needs N %% 128 == 0 and K %% 32 == 0");
    if (((uintptr_t)Bp & 15) || ((uintptr_t)B & 1)) return fail(GE_ERR_ALIGN, "B must be 2-byte and Bp 16-byte aligned");
    const size_t nb = ((size_t)(d.K - 1) * pl->ldb + d.N) * 2, np = (size_t)d.K * d.N * 2;
    if (overlaps(B, nb, Bp, np)) return fail(GE_ERR_INVALID_ARG, "Bp overlaps B");
    ge_status st;
    if ((st = check_device(pl))) return st;
    return hip_status(
        launch_b_prepack(d.K, d.N, (const uint16_t *)B, pl->ldb, (uint16_t *)Bp, pl->cu_count, (hipStream_t)stream,
                         pl->kind == GE_KIND_SWIGLU ? swiglu_block_tiles(d.N, pl->cu_count) : 0),
        "gemm_b_prepack");
}

namespace {
ge_status rope_common(int32_t batch, int32_t D, const float *cosT, const float *sinT, int32_t n_pos) {
    if (batch <= 0 || batch > 65535) return fail(GE_ERR_INVALID_ARG, "batch must be in [1, 65535]");
    if (D != 64 && D != 128) return fail(GE_ERR_UNSUPPORTED, "head dimension %d not in {64, 128}", D);
    if (!cosT || !sinT) return fail(GE_ERR_INVALID_ARG, "cos or sin is NULL");
    if (((uintptr_t)cosT & 15) || ((uintptr_t)sinT & 15)) return fail(GE_ERR_ALIGN, "cos and sin must be 16-byte aligned");
    if (n_pos <= 0) return fail(GE_ERR_INVALID_ARG, "n_pos must be positive");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        return fail(GE_ERR_NO_DEVICE, "no HIP device visible");
    }
    return GE_OK;
}
}  // namespace

ge_status ge_rope_qk_run(int32_t batch, int32_t Sq, int32_t Sk, int32_t D, const void *Q, const void *K,
                         const float *cos_t, const float *sin_t, int32_t n_pos, int32_t q_pos0, int32_t k_pos0,
                         int32_t flags, float alpha, int32_t s_type, void *S, void *stream) {
    if (Sq <= 0 || Sk <= 0) return fail(GE_ERR_INVALID_ARG, "Sq and Sk must be positive");
    if (flags & ~(GE_ROPE_INTERLEAVED | GE_ROPE_EXACT)) return fail(GE_ERR_INVALID_ARG, "unknown rope flag bits");
    if (!Q || !K || !S) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    if (s_type != GE_F32 && s_type != GE_BF16) return fail(GE_ERR_INVALID_ARG, "s_type must be F32 or BF16");
    if (((uintptr_t)Q & 15) || ((uintptr_t)K & 15)) return fail(GE_ERR_ALIGN, "Q and K must be 16-byte aligned");
    const bool rot = cos_t || sin_t;
    ge_status st;
    if (rot) {
        if ((st = rope_common(batch, D, cos_t, sin_t, n_pos))) return st;
        if (q_pos0 < 0 || k_pos0 < 0 || (int64_t)q_pos0 + Sq > n_pos || (int64_t)k_pos0 + Sk > n_pos)
            return fail(GE_ERR_INVALID_ARG, "positions outside the cos / sin tables");
    } else {
        if (batch <= 0 || batch > 65535) return fail(GE_ERR_INVALID_ARG, "batch must be in [1, 65535]");
        if (D != 64 && D != 128) return fail(GE_ERR_UNSUPPORTED, "head dimension %d not in {64, 128}", D);
    }
    const size_t nq = (size_t)batch * Sq * D * 2, nk = (size_t)batch * Sk * D * 2;
    const size_t ns = (size_t)batch * Sq * Sk * (s_type == GE_F32 ? 4 : 2);
    if (overlaps(S, ns, Q, nq) || overlaps(S, ns, K, nk)) return fail(GE_ERR_INVALID_ARG, "S overlaps Q or K");
    RopeArgs a{};
    a.batch = batch;
    a.Sq = Sq;
    a.Sk = Sk;
    a.D = D;
    a.q_pos0 = q_pos0;
    a.k_pos0 = k_pos0;
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.cos = rot ? cos_t : nullptr;
    a.sin = rot ? sin_t : nullptr;
    a.alpha = alpha;
    a.S = S;
    return hip_status(launch_rope_qk(a, (flags & GE_ROPE_INTERLEAVED) != 0, s_type == GE_F32, (flags & GE_ROPE_EXACT) != 0,
                                     (hipStream_t)stream),
                      "ge_rope_qk_run");
}

ge_status ge_rope_run(int32_t batch, int32_t S, int32_t D, const void *X, const float *cos_t, const float *sin_t,
                      int32_t n_pos, int32_t pos0, int32_t flags, void *Y, void *stream) {
    if (S <= 0) return fail(GE_ERR_INVALID_ARG, "S must be positive");
    if (flags & ~(GE_ROPE_INTERLEAVED | GE_ROPE_EXACT)) return fail(GE_ERR_INVALID_ARG, "unknown rope flag bits");
    if (!X || !Y) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    if (((uintptr_t)X & 15) || ((uintptr_t)Y & 15)) return fail(GE_ERR_ALIGN, "X and Y must be 16-byte aligned");
    ge_status st;
    if ((st = rope_common(batch, D, cos_t, sin_t, n_pos))) return st;
    if (pos0 < 0 || (int64_t)pos0 + S > n_pos) return fail(GE_ERR_INVALID_ARG, "positions outside the cos / sin tables");
    const size_t nb = (size_t)batch * S * D * 2;
    if (overlaps(X, nb, Y, nb)) return fail(GE_ERR_INVALID_ARG, "Y overlaps X");
    return hip_status(launch_rope(batch, S, D, (const uint16_t *)X, cos_t, sin_t, pos0, (flags & GE_ROPE_INTERLEAVED) != 0,
                                  (flags & GE_ROPE_EXACT) != 0, (uint16_t *)Y, (hipStream_t)stream),
                      "ge_rope_run");
}

static ge_status add_rmsnorm_common(bool fused, int32_t M, int32_t N, const void *a, const void *x, const void *w,
                                    float eps, void *resid, void *out, void *stream) {
    if (M <= 0 || N <= 0) return fail(GE_ERR_INVALID_ARG, "M and N must be positive");
    if (N > 16384) return fail(GE_ERR_UNSUPPORTED, "rows longer than 16384 elements");
    if (!a || !x || !w || !resid || !out) return fail(GE_ERR_INVALID_ARG, "NULL pointer");
    if (!(eps >= 0.0f)) return fail(GE_ERR_INVALID_ARG, "eps must be >= 0");
    const size_t nb = (size_t)M * N * 2;
    if (overlaps(out, nb, a, nb) || overlaps(out, nb, x, nb) || overlaps(out, nb, resid, nb))
        return fail(GE_ERR_INVALID_ARG, "out overlaps an input or resid");
    if ((resid != a && overlaps(resid, nb, a, nb)) || (resid != x && overlaps(resid, nb, x, nb)))
        return fail(GE_ERR_INVALID_ARG, "resid partially overlaps an input");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        return fail(GE_ERR_NO_DEVICE, "no HIP device visible");
    }
    if (fused)
        return hip_status(launch_add_rmsnorm(M, N, a, x, w, eps, resid, out, (hipStream_t)stream),
                          "ge_add_rmsnorm_run");
    return hip_status(launch_add_rmsnorm_unfused(M, N, a, x, w, eps, resid, out, (hipStream_t)stream),
                      "ge_add_rmsnorm_run_unfused");
}

ge_status ge_add_rmsnorm_run(int32_t M, int32_t N, const void *a, const void *x, const void *w, float eps,
                             void *resid, void *out, void *stream) {
    return add_rmsnorm_common(true, M, N, a, x, w, eps, resid, out, stream);
}

ge_status ge_add_rmsnorm_run_unfused(int32_t M, int32_t N, const void *a, const void *x, const void *w, float eps,
                                     void *resid, void *out, void *stream) {
    return add_rmsnorm_common(false, M, N, a, x, w, eps, resid, out, stream);
}

}  // extern "C"
