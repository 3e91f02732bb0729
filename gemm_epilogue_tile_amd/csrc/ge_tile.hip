// ge_tile.hip -- large-tile bf16 MFMA kernel with the epilogue in the store path.
//
// One 256-thread workgroup (four waves, 2 x 2) owns a BM x BN output tile and
// its whole K reduction, so the epilogue needs nothing from other workgroups
// (page "kernel fusion" wiki: the activation is applied to each output tile
// before it leaves the compute unit; page "Fusion and Epilogues": the ending
// is applied to the accumulators on the way to their single store).
//
// Data path, per 32-deep K stage:
//   memory -> LDS   buffer_load ... lds (16 bytes per lane, straight into LDS,
//                   no registers); lanes past the end of a matrix read zeros.
//                   Four LDS stages: the loads of stage s+4 are issued while
//                   stage s is multiplied, three stages ahead of their use.
//   A in LDS        [BM][32] bf16, 16-byte chunk c of row r at c ^ ((r>>1)&3):
//                   conflict-free 128-bit fragment reads.
//   B in LDS        KN layout: [32][BN] as stored in memory, 16-byte chunk c of
//                   row k at c ^ ((k&3)<<1) ^ (((k>>3)&1)<<3); fragments come from the gfx950
//                   transposing read ds_read_b64_tr_b16, which turns four
//                   rows x sixteen columns into one k-vector per column.
//                   NK layout: [BN][32] like A.
//   LDS -> MFMA     v_mfma_f32_16x16x32_bf16, fp32 accumulators (AGPRs).  B is
//                   the first operand, so each lane ends up holding four
//                   consecutive output columns of one row.  The fragments of
//                   stage s+1 are read while the MFMAs of stage s run.
//   One barrier per stage.
//
// Epilogue: alpha*acc + beta*C + bias -> activation -> + R (or silu(g)*u for
// the dual product), 4 consecutive columns per lane, one rounding to the
// output type, one store.
//
// Workgroup -> tile map: consecutive workgroup ids land on different XCDs
// (round-robin dispatch), so ids are first regrouped so that each XCD owns a
// contiguous run of tiles, then runs are laid out in bands of GROUP_M (dual: 2 GROUP_M) tile
// rows: the tiles one XCD works on at a time share A rows and B columns in
// that XCD's L2.

#include "ge_launch.hpp"

namespace ge {
namespace {

#include "ge_tile_common.hpp"


template <int BM, int BN, int WM, int WN, bool DUAL, bool B_NK>
struct Cfg {
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int MT = WTM / 16, NT = WTN / 16;   // 16x16 MFMA tiles per wave
    static constexpr int NB = DUAL ? 2 : 1;
    static constexpr int A_STAGE = BM * T_BK * 2;        // bytes of one stage
    static constexpr int A_PAIR = 2 * A_STAGE;           // A is staged two stages at a time: [BM][64]
    static constexpr int B_STAGE = BN * T_BK * 2;
    static constexpr int B_BASE = T_NS * A_STAGE;        // LDS: the two A pair buffers, then all B stages
    static constexpr int LDS = T_NS * (A_STAGE + NB * B_STAGE);
    static constexpr int AP_INSTR = A_PAIR / 1024 / 4;   // 1 KB direct loads per wave per A pair
    static constexpr int B_INSTR = B_STAGE / 1024 / 4;   // ... per wave per B stage
    static constexpr int NBI = NB * B_INSTR;
    static constexpr int B_PAIR = 2 * B_STAGE;           // NK: B staged two stages at a time, like A
    static constexpr int BP_INSTR = B_PAIR / 1024 / 4;
    static constexpr int LOADS = AP_INSTR + (B_NK ? BP_INSTR : NBI);  // most loads a wave issues in one stage
    static constexpr int B_ROWS_PER_INSTR = 1024 / (BN * 2);  // KN: k rows one load instruction fills
    static_assert(WM * WN == 4, "four waves");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(T_NS == 4, "two A pairs: four stages");
    static_assert(AP_INSTR >= 1 && B_INSTR >= 1 && AP_INSTR * 4096 == A_PAIR && B_INSTR * 4096 == B_STAGE, "loads");
    static_assert(B_NK || BN == 256 || BN == 128 || BN == 512, "KN row width");
    static_assert(A_PAIR + (MT - 1) * 2048 + 128 < 65536, "A fragment offsets fit the ds offset field");
    static_assert((NB * T_NS - 1) * B_STAGE < 65536, "B stage offsets fit the ds offset field");
    static_assert(!B_NK || (NB == 1 && B_PAIR + (NT - 1) * 2048 + 128 < 65536), "NK B fragment offsets");
};

template <int BM, int BN, int WM, int WN, bool DUAL, bool B_NK>
__global__ __attribute__((amdgpu_flat_work_group_size(T_THREADS, T_THREADS), amdgpu_waves_per_eu(1, 1)))
void tile_kernel(Problem p) {
    using C = Cfg<BM, BN, WM, WN, DUAL, B_NK>;
    // LDS: the T_NS A stages, then the T_NS B stages (then the B2 stages).  Every
    // fragment address is a per-lane base plus a compile-time offset below 64 KiB.
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(AS3 void *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile selection (XCD-aware) ----
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    // bands of GM tile rows: 4 for plain products; 8 for the dual product, whose 128-column tiles
    // make a band of 4 rows twice as wide (2048 x 14336 SwiGLU: 344 -> 336 us; 4096^3 with 8: 97.4
    // -> 98.8 us)
    constexpr int GM = DUAL ? 2 * GROUP_M : GROUP_M;
    const int per_group = GM * tiles_n;
    const int first_m = (t / per_group) * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- direct-load lane offsets (constant across stages; k advances in the resource base) ----
    // A pair (stages 2t, 2t + 1): [BM][64] with 128-byte rows, so that every load fetches whole
    // 128-byte lines (8 rows x 8 chunks per 1 KB instruction; 64-byte rows took two line requests
    // per 128 bytes); lane -> row 8 i + lane/8 of instruction i, LDS slot lane%8, which holds
    // logical chunk (lane%8) ^ ((row>>1)&7) (stage 2t: chunks 0-3, stage 2t + 1: chunks 4-7).  Bit
    // 2 of that swizzle is the parity of i (AP_INSTR is even), so a lane's chunk takes two values.
    const int arow_l = lane >> 3;
    int achunk[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) achunk[e] = (lane & 7) ^ ((arow_l >> 1) & 7) ^ (4 * e);
    static_assert(C::AP_INSTR % 2 == 0, "instruction parity");
    uint32_t a_off[C::AP_INSTR];
#pragma unroll
    for (int q = 0; q < C::AP_INSTR; ++q) {
        const int row = (wave * C::AP_INSTR + q) * 8 + arow_l;
        a_off[q] = (uint32_t)(row * p.lda * 2) + ((lane & 7) ^ ((row >> 1) & 7)) * 16;
    }
    // B: KN -> one stage [32][BN] at a time, an instruction fills B_ROWS_PER_INSTR k rows; NK -> B^T
    // is staged in pairs exactly like A ([BN][64], the same lane mapping and swizzle).
    uint32_t b_off[B_NK ? C::BP_INSTR : C::B_INSTR];
    if constexpr (B_NK) {
#pragma unroll
        for (int q = 0; q < C::BP_INSTR; ++q) {
            const int row = (wave * C::BP_INSTR + q) * 8 + arow_l;
            b_off[q] = (uint32_t)(row * p.ldb * 2) + ((lane & 7) ^ ((row >> 1) & 7)) * 16;
        }
    } else {
        constexpr int CPR = BN / 8;  // 16-byte chunks per k row
        const int krow_l = lane / CPR;
        const int slot = lane % CPR;
#pragma unroll
        for (int q = 0; q < C::B_INSTR; ++q) {
            const int k = (wave * C::B_INSTR + q) * C::B_ROWS_PER_INSTR + krow_l;
            const int chunk = slot ^ swz_b_key(k);
            // columns past N read zeros (fixed per lane, so folded in once)
            b_off[q] = n0 + chunk * 8 < p.N ? (uint32_t)(k * p.ldb * 2) + chunk * 16 : OOB;
        }
    }

    // Direct loads: B stage s (K offset 32 s) into B buffer s % T_NS; A pair t (K offset 64 t, the
    // stages 2t and 2t + 1) into A pair buffer t % 2.  Both are loaded in order, and the buffer
    // resources of the next B stage and the next A pair are kept in scalar registers and advanced
    // one step at a time: the base moves by the step, the range shrinks by as much and stays at 0
    // once it is empty (a step beyond 2^31 - 1 bytes empties it at once: every operand is below
    // 2 GiB).  No 64-bit multiply is left in the loop.
    struct BLoads {
        i32x4 rb[C::NB];
        uint32_t bdst[C::NB];
        bool bkin[2];  // NK: by instruction parity
    };
    struct ALoads {
        i32x4 ra;
        uint32_t adst;
        bool akin[2];  // by instruction parity
    };
    auto rsrc_at = [](uint64_t a, int32_t range) {
        i32x4 r;
        r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
        r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
        r[2] = __builtin_amdgcn_readfirstlane(range);
        r[3] = 0x00020000;
        return r;
    };
    constexpr int32_t A_STEP = 2 * T_BK * 2;  // one pair
    const int64_t b_step64 = B_NK ? (int64_t)2 * T_BK * 2 : (int64_t)T_BK * p.ldb * 2;  // NK: one pair
    const int32_t b_step = b_step64 < 0x7fffffffll ? (int32_t)b_step64 : 0x7fffffff;
    uint64_t a_ptr = (uint64_t)(uintptr_t)p.A + (uint64_t)((int64_t)m0 * p.lda * 2);
    int32_t a_rng = (int32_t)(((int64_t)(p.M - 1 - m0) * p.lda + p.K) * 2);
    uint64_t b_ptr[C::NB];
#pragma unroll
    for (int d = 0; d < C::NB; ++d)
        b_ptr[d] = (uint64_t)(uintptr_t)(d == 0 ? p.B : p.B2) + (uint64_t)(B_NK ? (int64_t)n0 * p.ldb * 2 : (int64_t)n0 * 2);
    int32_t b_rng = (int32_t)(B_NK ? ((int64_t)(p.N - 1 - n0) * p.ldb + p.K) * 2
                                   : ((int64_t)(p.K - 1) * p.ldb + (p.N - n0)) * 2);
    int kb_next = 0, ka_next = 0;  // K offsets of the next B stage and the next A pair to load
    auto b_loads = [&](int s) {  // s: the next B stage (NK: pair) in load order
        BLoads L;
        const int buf = s & (T_NS - 1);
        if constexpr (B_NK) {
            L.bkin[0] = kb_next + achunk[0] * 8 < p.K;
            L.bkin[1] = kb_next + achunk[1] * 8 < p.K;
            L.bdst[0] = lds0 + C::B_BASE + (s & 1) * C::B_PAIR + wave * C::BP_INSTR * 1024;
            L.rb[0] = rsrc_at(b_ptr[0], b_rng);
            b_ptr[0] += (uint64_t)b_step64;
            kb_next += 2 * T_BK;
        } else {
#pragma unroll
            for (int d = 0; d < C::NB; ++d) {
                L.bdst[d] = lds0 + C::B_BASE + d * T_NS * C::B_STAGE + buf * C::B_STAGE + wave * C::B_INSTR * 1024;
                L.rb[d] = rsrc_at(b_ptr[d], b_rng);
                b_ptr[d] += (uint64_t)b_step64;
            }
            kb_next += T_BK;
        }
        b_rng = b_rng > b_step ? b_rng - b_step : 0;
        return L;
    };
    auto a_loads = [&](int t) {  // t: the next A pair in load order
        ALoads L;
        L.ra = rsrc_at(a_ptr, a_rng);
        L.akin[0] = ka_next + achunk[0] * 8 < p.K;
        L.akin[1] = ka_next + achunk[1] * 8 < p.K;
        L.adst = lds0 + (t & 1) * C::A_PAIR + wave * C::AP_INSTR * 1024;
        a_ptr += A_STEP;
        a_rng = a_rng > A_STEP ? a_rng - A_STEP : 0;
        ka_next += 2 * T_BK;
        return L;
    };
    auto issue_a = [&](const ALoads &L, int q) { load_lds16(L.ra, L.adst + q * 1024, L.akin[q & 1] ? a_off[q] : OOB); };
    auto issue_b = [&](const BLoads &L, int q) {
        if constexpr (B_NK) {
            load_lds16(L.rb[0], L.bdst[0] + q * 1024, L.bkin[q & 1] ? b_off[q] : OOB);
        } else {
            const int d = q / C::B_INSTR, qq = q % C::B_INSTR;
            load_lds16(L.rb[d], L.bdst[d] + qq * 1024, b_off[qq]);
        }
    };
    auto load_a_pair = [&](int t) {
        const ALoads L = a_loads(t);
#pragma unroll
        for (int q = 0; q < C::AP_INSTR; ++q) issue_a(L, q);
    };
    constexpr int NBL = B_NK ? C::BP_INSTR : C::NBI;  // B loads per load step (NK: per pair)
    auto load_b_stage = [&](int s) {
        const BLoads L = b_loads(s);
#pragma unroll
        for (int q = 0; q < NBL; ++q) issue_b(L, q);
    };

    // ---- fragment addresses (stage 0; other stages add a compile-time offset) ----
    const int frow = lane & 15, fgrp = lane >> 4;
    // A fragment i of stage 2t + h: rows wm*WTM + 16 i + frow of pair buffer t % 2, logical chunk
    // 4 h + fgrp (k = 8 fgrp .. 8 fgrp + 7 of the stage); rows 16 apart share the swizzle
    int a_frag[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = wm * C::WTM + frow;
        a_frag[h] = row * 128 + (((4 * h + fgrp) ^ ((row >> 1) & 7)) << 4);
    }
    // B fragment j:
    //   NK: like A;
    //   KN: two transposing reads r = 0, 1: lane (g, jj) points at k = 8 g + 4 r + jj/4 and
    //       columns 16 j + 4 (jj % 4) .. + 3; the read hands lane jj the k-vector of column jj.
    int b_frag[C::NT][2];
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        if constexpr (B_NK) {
            // like A: row wn*WTN + 16 j + frow of the pair buffer, logical chunk 4 h + fgrp (h: the
            // stage's half, 0 / 1 in b_frag[j][h])
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = wn * C::WTN + j * 16 + frow;
                b_frag[j][h] = C::B_BASE + row * 128 + (((4 * h + fgrp) ^ ((row >> 1) & 7)) << 4);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int k = 8 * fgrp + 4 * r + (frow >> 2);
                const int n = wn * C::WTN + j * 16 + 4 * (frow & 3);
                b_frag[j][r] = C::B_BASE + swz_b<BN>(k, n >> 3) + ((n >> 2) & 1) * 8;
            }
        }
    }

    bf16x8 fa[2][C::MT], fb[2][C::NB][C::NT];
    const AS3 char *s3 = (const AS3 char *)smem;
    auto read_a = [&](int buf, int i, bf16x8 &a) {
        a = *(const AS3 bf16x8 *)(s3 + a_frag[buf & 1] + (buf >> 1) * C::A_PAIR + i * 2048);
    };
    auto read_b = [&](int buf, int d, int j, bf16x8 &b) {
        const int off = d * T_NS * C::B_STAGE + buf * C::B_STAGE;
        if constexpr (B_NK) {
            b = *(const AS3 bf16x8 *)(s3 + b_frag[j][buf & 1] + (buf >> 1) * C::B_PAIR);
        } else {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 i16x4 *)(s3 + b_frag[j][0] + off));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 i16x4 *)(s3 + b_frag[j][1] + off));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            b = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        }
    };
    // fragment read r of a stage: A fragments and B fragments alternate
    constexpr int NRD = C::MT + C::NB * C::NT;
    // read r < NRD: A and B fragments interleave in proportion to their counts
    constexpr int NBT = C::NB * C::NT;
    auto read_frag = [&](int buf, int r, bf16x8 (&a)[C::MT], bf16x8 (&b)[C::NB][C::NT]) {
        // read r is an A read when ceil((r + 1) * MT / NRD) > ceil(r * MT / NRD) (read 0 is A)
        const int a_before = (r * C::MT + NRD - 1) / NRD, a_after = ((r + 1) * C::MT + NRD - 1) / NRD;
        if (a_after > a_before) {
            read_a(buf, a_before, a[a_before]);
        } else {
            const int bi = r - a_before;
            read_b(buf, bi / C::NT, bi % C::NT, b[bi / C::NT][bi % C::NT]);
        }
    };
    auto read_frags = [&](int buf, bf16x8 (&a)[C::MT], bf16x8 (&b)[C::NB][C::NT]) {
#pragma unroll
        for (int r = 0; r < NRD; ++r) read_frag(buf, r, a, b);
    };

    f32x4 acc[C::NB][C::MT][C::NT];
#pragma unroll
    for (int d = 0; d < C::NB; ++d)
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) acc[d][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS-only barrier: orders this workgroup's LDS traffic without waiting for prefetches
    auto lds_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // One stage: the 64 MFMAs of stage s, with the next stage's fragment reads and the direct
    // loads issued in this stage (odd s: A pair (s + 3) / 2; every s: B stage s + T_NS) spread
    // between them so the matrix pipe never waits on a burst of LDS or memory instructions.
    // Reads go after MFMAs 0, 3, 6, ..., loads after 1, 4, 7, ...; an empty asm with a memory
    // clobber pins each one to its slot.
    constexpr int NMF = C::NB * C::NT * C::MT;
    // side-op spacing: reads after MFMAs 0, SP, 2 SP, ..., loads after 1, SP + 1, ...
    constexpr int SP = (3 * (NRD - 1) < NMF && 3 * (C::LOADS - 1) + 1 < NMF) ? 3 : 2;
    static_assert(SP * (NRD - 1) < NMF && SP * (C::LOADS - 1) + 1 < NMF, "side-op slots");
    // (NK: odd stages issue the A pair and the B pair, even stages nothing)
    auto stage = [&](bool with_a, const ALoads &LA, const BLoads &LB, int nbuf, const bf16x8 (&a)[C::MT],
                     const bf16x8 (&b)[C::NB][C::NT], bf16x8 (&na)[C::MT], bf16x8 (&nb)[C::NB][C::NT]) {
        const int nload = with_a ? C::LOADS : (B_NK ? 0 : C::NBI);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            const int d = q / (C::NT * C::MT), j = (q / C::MT) % C::NT, i = q % C::MT;
            mfma_bf16_acc(acc[d][i][j], b[d][j], a[i]);
            if (q % SP == 0 && q / SP < NRD) {
                asm volatile("" ::: "memory");
                read_frag(nbuf, q / SP, na, nb);
                asm volatile("" ::: "memory");
            } else if (q % SP == 1 && q / SP < nload) {
                const int l = q / SP;  // A pair loads first, then the B stage's
                if (with_a && l < C::AP_INSTR)
                    issue_a(LA, l);
                else
                    issue_b(LB, with_a ? l - C::AP_INSTR : l);
            }
        }
    };

    // wait until at most n of this wave's direct loads are outstanding
    // (vmcnt counts them in issue order; lgkm / exp counters left at their maximum)
#define GE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x70 | 0xF00)

    const int nk = (p.K + T_BK - 1) / T_BK;
    const int nsteps = (nk + T_NS - 1) / T_NS * T_NS;  // whole rounds of T_NS stages (extra stages read zeros)

    // Load order: stage s issues (odd s) A pair (s + 3) / 2, then B stage s + 4 (NK: odd s only, the
    // B pair (s + 3) / 2).  The prologue issues what stages -4 .. -1 would have (B 0, A pair 0, B 1,
    // B 2, A pair 1, B 3; NK: A pair 0, B pair 0, A pair 1, B pair 1), waits for stage 0's loads and
    // reads its fragments.
    if constexpr (B_NK) {
        load_a_pair(0);
        load_b_stage(0);
        load_a_pair(1);
        load_b_stage(1);
        GE_WAIT_VM(C::AP_INSTR + C::BP_INSTR);
    } else {
        load_b_stage(0);
        load_a_pair(0);
        load_b_stage(1);
        load_b_stage(2);
        load_a_pair(1);
        load_b_stage(3);
        GE_WAIT_VM(3 * C::NBI + C::AP_INSTR);
    }
    lds_barrier();
    read_frags(0, fa[0], fb[0]);

    for (int s0 = 0; s0 < nsteps; s0 += T_NS) {
#pragma unroll
        for (int b = 0; b < T_NS; ++b) {
            const int s = s0 + b;
            // stage s+1 landed (own loads), visible to all; every wave is done reading stage s.  Still
            // in flight may be what stages s-2 and s-1 issued after stage s+1's loads: the B stages
            // s+2 and s+3 and, for even s, the A pair of stages s+2 and s+3 (issued by stage s-1).
            // NK: for even s the A and B pairs of stages s+2 and s+3, for odd s nothing.
            if constexpr (B_NK) {
                if (b & 1)
                    GE_WAIT_VM(0);
                else
                    GE_WAIT_VM(C::AP_INSTR + C::BP_INSTR);
            } else {
                if (b & 1)
                    GE_WAIT_VM(2 * C::NBI);
                else
                    GE_WAIT_VM(2 * C::NBI + C::AP_INSTR);
            }
            lds_barrier();
            GE_DEBUG_BARRIER();
            // odd s: A pair (s + 3) / 2 into the pair buffer of stages s - 1, s (read by now); NK: the
            // B pair as well
            ALoads LA{};
            BLoads LB{};
            if (b & 1) LA = a_loads((s + 3) >> 1);
            if constexpr (B_NK) {
                if (b & 1) LB = b_loads((s + 3) >> 1);
            } else {
                LB = b_loads(s + T_NS);  // into buffer b, three stages ahead
            }
            stage((b & 1) != 0, LA, LB, (b + 1) & (T_NS - 1), fa[b & 1], fb[b & 1], fa[(b + 1) & 1], fb[(b + 1) & 1]);
        }
    }
#undef GE_WAIT_VM
    // drain the (zero-reading) prefetches past the end before the workgroup can exit,
    // and let the last MFMAs retire before their accumulators are read
    __builtin_amdgcn_s_waitcnt(0);
    mfma_drain();
    // tie every accumulator to the drain so no read of it is scheduled above the wait
#pragma unroll
    for (int d = 0; d < C::NB; ++d)
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) asm volatile("" : "+a"(acc[d][i][j]));

    // ---- epilogue: lane holds row m, columns n..n+3 of each 16x16 tile ----
    const EpiArgs &e = p.epi;
    const int mbase = m0 + wm * C::WTM + frow;
    const int nbase = n0 + wn * C::WTN + fgrp * 4;
    auto small = [&](int64_t ld) { return ((int64_t)(p.M + 15) * ld + p.N) * 2 < (1ll << 31); };
    const bool all_bf16 = e.d_type == GE_BF16 && small(e.ldd) &&
                          (!(e.flags & GE_FLAG_C) || (e.c_type == GE_BF16 && small(e.ldc))) &&
                          (!(e.flags & GE_FLAG_RESIDUAL) || (e.r_type == GE_BF16 && small(e.ldr))) &&
                          (!(e.flags & GE_FLAG_BIAS) || e.bias_type == GE_BF16);
    if constexpr (DUAL) {
        // SwiGLU outputs are bf16 (checked at plan time)
        epilogue_swiglu(e, acc[0], acc[1], p.M, p.N, mbase, n0 + wn * C::WTN + fgrp * 8);
    } else if (all_bf16) {
        with_act(e.act, [&](auto ACTC) {
            constexpr int ACT = decltype(ACTC)::value;
            if (e.flags & GE_FLAG_C)
                epilogue_bf16<ACT, true>(e, acc[0], p.M, p.N, mbase, n0 + wn * C::WTN + fgrp * 8);
            else
                epilogue_bf16<ACT, false>(e, acc[0], p.M, p.N, mbase, n0 + wn * C::WTN + fgrp * 8);
        });
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
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(k, dim3(tiles), dim3(T_THREADS), C::LDS, s, p);
    return hipGetLastError();
}

}  // namespace

bool tile_supported(const Problem &p) {
    if (p.mode == MODE_W4) return tile_w4_supported(p);
    if (p.ab_type != GE_BF16) return false;
    // the streaming kernels take plain products of M <= 32; SwiGLU has no streaming kernel
    if (p.M <= 32 && p.mode != MODE_SWIGLU) return false;
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

// SwiGLU tiles are 256 x 128.  When their count leaves the last round of workgroups
// partly empty (2048 x 14336: 896 tiles = 3.5 rounds of 256 CUs), the columns of the
// partial round are peeled off and run as 128 x 128 tiles, one full round of half-size
// tiles: returns the 128-column blocks that stay in 256 x 128 tiles (all of them when
// nothing is peeled).
int swiglu_big_blocks(const Problem &p, int cu_count) {
    const int tiles_m = (p.M + 255) / 256, ncb = (p.N + 127) / 128;
    const int64_t total = (int64_t)tiles_m * ncb;
    if (cu_count <= 0 || total <= cu_count || total % cu_count == 0) return ncb;
    const int64_t full = total / cu_count * cu_count;
    if (full % tiles_m) return ncb;
    const int nb = (int)(full / tiles_m);
    const int64_t small = (int64_t)((p.M + 127) / 128) * (ncb - nb);
    return small <= cu_count ? nb : ncb;
}

// Plain products use 128 x 128 tiles when those fit in one round over the CUs (a few rows, or
// few columns: 33..128 x 28672 and 512 x 8192 take 0.6-0.8x the time of 256 x 256 tiles, which
// would leave half the CUs or more idle), and 256 x 256 tiles otherwise.
static bool small_tiles(const Problem &p, int cu_count) {
    const int64_t n128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
    return n128 <= (cu_count > 0 ? cu_count : 256);
}

const char *tile_kernel_name(const Problem &p, int cu_count) {
    if (p.mode == MODE_W4) return tile_w4_kernel_name(p, cu_count);
    if (p.mode == MODE_SWIGLU)
        return swiglu_big_blocks(p, cu_count) * 128 < p.N ? "tile_swiglu_256x128x32+128x128x32"
                                                           : "tile_swiglu_256x128x32";
    if (small_tiles(p, cu_count)) return p.b_layout == GE_LAYOUT_NK ? "tile_nk_128x128x32" : "tile_kn_128x128x32";
    return p.b_layout == GE_LAYOUT_NK ? "tile_nk_256x256x32" : "tile_kn_256x256x32";
}

hipError_t launch_tile(const Problem &p, int cu_count, hipStream_t s) {
    if (!tile_supported(p)) return hipErrorInvalidValue;
    if (p.mode == MODE_W4) return launch_tile_w4(p, cu_count, s);
    if (p.mode == MODE_SWIGLU) {
        const int nb = swiglu_big_blocks(p, cu_count);
        if (nb * 128 >= p.N) return launch_cfg<256, 128, 2, 2, true, false>(p, s);
        // columns [0, 128 nb) in 256 x 128 tiles, the rest in 128 x 128 tiles
        const int64_t off = (int64_t)nb * 128;
        Problem big = p, rest = p;
        big.N = (int32_t)off;
        rest.N = p.N - (int32_t)off;
        rest.B = (const uint16_t *)p.B + off;
        rest.B2 = (const uint16_t *)p.B2 + off;
        rest.epi.D = (uint16_t *)p.epi.D + off;
        hipError_t e = launch_cfg<256, 128, 2, 2, true, false>(big, s);
        if (e == hipSuccess) e = launch_cfg<128, 128, 2, 2, true, false>(rest, s);
        return e;
    }
    if (small_tiles(p, cu_count)) {
        if (p.b_layout == GE_LAYOUT_NK) return launch_cfg<128, 128, 2, 2, false, true>(p, s);
        return launch_cfg<128, 128, 2, 2, false, false>(p, s);
    }
    if (p.b_layout == GE_LAYOUT_NK) return launch_cfg<256, 256, 2, 2, false, true>(p, s);
    return launch_cfg<256, 256, 2, 2, false, false>(p, s);
}

}  // namespace ge
