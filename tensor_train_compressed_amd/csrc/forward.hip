// Forward pass of the TT-EmbeddingBag library.
//
// Every chunk of a prefix group shares the partial product of the first two
// cores, P = G1[i1] x G2[i2] (n1*n2 x R), which is kept on chip and reused for
// every lookup of the chunk; only the last contraction, P x G3[i3], is done per
// lookup, and its row goes straight into the pooled output. This is the
// flow-reuse idea of the FlowTT pages (summary card, key innovations: prefix
// grouping and flow-aligned on-chip execution; problem statement: the shared
// part of the chain is otherwise recomputed and intermediates round-trip
// through off-chip memory).
#include "tt_device.h"

namespace tt {

// Generic shapes: one workgroup per chunk. P lives in LDS; each thread forms
// output elements of the chunk's lookups and adds them to the bag's row.
__global__ __launch_bounds__(256) void k_fwd_generic(
    const TabDev* __restrict__ desc, int32_t T, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ group_key, const int32_t* __restrict__ chunk_group,
    const int32_t* __restrict__ chunk_begin, const int32_t* __restrict__ chunk_end,
    const int32_t* __restrict__ sorted_i3, const int32_t* __restrict__ sorted_bag,
    const float* __restrict__ g1, const float* __restrict__ g2, const float* __restrict__ g3,
    float* __restrict__ out, int32_t D) {
    extern __shared__ float P[];  // [n1*n2][R]
    const int32_t c = blockIdx.x;
    if (c >= ctrl[CTRL_NUM_CHUNKS]) return;
    const int32_t g = chunk_group[c];
    const int32_t key = group_key[g];
    const TabDev d = desc[find_table(desc, T, key)];
    const int32_t local = key - d.key_base;
    const int32_t i2 = local / d.m1, i1 = local % d.m1;
    const int32_t R = d.R, n2 = d.n2, n3 = d.n3;
    const int32_t np = d.n1 * n2;
    const float* A = g1 + d.o1 + (int64_t)i1 * d.n1 * R;
    const float* Bc = g2 + d.o2 + (int64_t)i2 * R * n2 * R;
    for (int e = threadIdx.x; e < np * R; e += blockDim.x) {
        const int p = e / R, r2 = e % R;
        const int j1 = p / n2, j2 = p % n2;
        float s = 0.f;
        for (int r1 = 0; r1 < R; ++r1) s = fmaf(A[j1 * R + r1], Bc[(r1 * n2 + j2) * R + r2], s);
        P[e] = s;
    }
    __syncthreads();
    const int32_t b = chunk_begin[c], e_end = chunk_end[c];
    const int64_t work = (int64_t)(e_end - b) * D;
    const float* C0 = g3 + d.o3;
    for (int64_t w = threadIdx.x; w < work; w += blockDim.x) {
        const int32_t s = b + (int32_t)(w / D);
        const int32_t dd = (int32_t)(w % D);
        const int p = dd / n3, j3 = dd % n3;
        const float* Cs = C0 + (int64_t)sorted_i3[s] * R * n3;
        float v = 0.f;
        for (int r2 = 0; r2 < R; ++r2) v = fmaf(P[p * R + r2], Cs[r2 * n3 + j3], v);
        atomicAdd(&out[(int64_t)sorted_bag[s] * D + dd], v);
    }
}


// ---------------------------------------------------------------------------
// Matrix-core path for the shapes the library is built for (every table of
// the plan with the same n1, n2, n3 and R).
//
// One workgroup (4 waves) per batch of up to kFwdBatch prefix groups of one
// (table, i2) slice: groups that share a G2 slice are adjacent in key order.
// The workgroup reads the G2 slice into LDS once and forms the batch's prefixes
// P_g = G1[i1(g)] x G2[i2] together, as one (4*batch) x (n2*R) x R product on
// the matrix cores (v_mfma_f32_16x16x4_f32), keeping all of them in LDS.
// Inside a group the planner has put repeats of one table row next to each
// other, so a group is a list of runs, one per distinct row; the last contraction P_g x G3[i3] is done once per run, in tiles
// of 16 output columns = 4 runs x 4 columns of G3. Each run's row is written
// once to the stage buffer at its run id; k_pool then sums every bag's rows in
// input order and writes the bag's output row: no atomics, and the same bits
// on every run.

// Every table's G3 slices transposed to [n3][R] (g3t, same packing as G3),
// so that a tile lane's suffix operand, eight consecutive r2 of one j3, is two
// 16-byte loads instead of eight 4-byte loads 16 bytes apart. One thread per
// G3 element the tables use (tables sharing a G3 write the same values).
__global__ __launch_bounds__(256) void k_g3t(const TabDev* __restrict__ desc, int32_t T, int64_t n,
                                             const float* __restrict__ g3, float* __restrict__ g3t) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    int lo = 0, hi = T;   // last table with g3_base <= e
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (desc[mid].g3_base <= e) lo = mid; else hi = mid;
    }
    const TabDev d = desc[lo];
    const int64_t cn = (int64_t)d.R * d.n3, local = e - d.g3_base;
    const int64_t slice = d.o3 + (local / cn) * cn;
    const int64_t w = local % cn;          // destination: [j3][r2]
    const int64_t j3 = w / d.R, r2 = w % d.R;
    g3t[slice + w] = g3[slice + r2 * d.n3 + j3];
}

struct FwdArgs {
    const BatchRec* recs;
    const int32_t* run_i3;
    const float* g1;
    const float* g2;
    const float* g3t;      // G3 with each slice transposed to [n3][R]
    float* stage;
    int64_t L;             // first spare stage row
    float* pbuf;           // when set, each group's P is also kept here (for the backward)
    int32_t* claims;       // [kFwdCounters][32]: batch claim counters (zero at the launch)
};

// The runs of one batch: tiles of LK = 16/n3 runs of one group. The suffix
// product of a tile is E^T = G3[i3]^T P^T: rows (run, j3), columns p, K = r2.
// Lane (col, q) feeds G3 of run col/n3 (its column j3 = col%n3) as the A
// operand and P row 16mt + col as the B operand, and receives rows 4q..4q+3
// of the tile's E^T at p = 16mt + col: with n3 >= 4, four consecutive j3 of
// one run (one 16-byte store); with n3 = 2, two j3 of each of two runs; with
// n3 = 1, one value of each of four runs.
// Wave w takes a contiguous range of tiles (consecutive tiles mostly share a
// group, so P is reloaded once per group). Every wave forms the batch's tile
// prefix itself, in registers (lane g: first tile of group g), so begin() can
// issue the G3 loads of the wave's first tile straight after the prologue,
// before the next batch's loads and with no barrier: most batches have one
// tile per wave, whose operand latency would otherwise be exposed. In run(),
// a tile's G3 operand is loaded one tile ahead, before the current tile's
// stores: loads and stores share one in-order completion counter, so a load
// can only be waited for alone if every memory access issued after it is
// certain to have been issued. The loop body therefore holds no conditional
// access (lanes past the group's last run store to spare rows, the
// look-ahead tile is clamped to the last one, run i3 values come from LDS),
// it is unrolled by two with ping-pong operand sets, and no register that a
// load is still filling is ever copied.
template <int N1, int N2, int R, int N3>
struct FwdTiles {
    using B = PrefixBatch<N1, N2, R>;
    static constexpr int NP = B::NP, D = NP * N3, KS = B::KS, AS = B::AS, WAVES = B::WAVES;
    static constexpr int MT = NP / 16, LK = 16 / N3;
    static constexpr int RPL = N3 >= 4 ? 1 : 4 / N3;   // runs of a lane's four results
    static constexpr int VPR = 4 / RPL;                // results per run (consecutive j3)
    static_assert(16 % N3 == 0 && LK <= kStageSpare, "suffix tile shape");
    struct Ids {
        int g;
        int32_t r[RPL];    // stage rows of the lane's result runs (spare rows past the group's end)
        int32_t i3;        // i3 of the lane's operand run col/n3 (the tile's first run's past the end)
    };
    struct Ops {
        int g;
        int32_t r[RPL];
        floatx4 bv[KS / 4];   // G3[i3 of run col/n3][j3 = col%n3][r2 = KS*q + 4h + u], K = r2
    };
    int32_t tpl;           // lane g <= ng: the batch's first tile of group g (lane ng: the tile count)
    int t0, n, gs;
    Ids IA, IB;
    Ops OA, OB;

    __device__ __forceinline__ int tp(int g) const { return __builtin_amdgcn_readlane(tpl, g); }

    __device__ __forceinline__ void ids_of(const FwdArgs& a, const BatchCtx& c, const int32_t* sRb,
                                           const int32_t* sI3, int k, Ids& o) {
        const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4, lk = col / N3;
        const int tt = t0 + k;
        while (tp(gs + 1) <= tt) ++gs;
        o.g = gs;
        const int32_t rb = sRb[gs] + LK * (tt - tp(gs)), re = sRb[gs + 1];   // relative to rb0
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
            const int lr = (4 * q) / N3 + u;
            o.r[u] = rb + lr < re ? c.rb0 + rb + lr : (int32_t)a.L + lr;
        }
        o.i3 = sI3[rb + lk < re ? rb + lk : rb];
    }
    __device__ __forceinline__ void load_ops(const FwdArgs& a, const BatchCtx& c, const Ids& o, Ops& x) {
        const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4, j3 = col % N3;
        x.g = o.g;
#pragma unroll
        for (int u = 0; u < RPL; ++u) x.r[u] = o.r[u];
        const floatx4* gb = reinterpret_cast<const floatx4*>(a.g3t + c.o3 + (int64_t)o.i3 * R * N3 + j3 * R + KS * q);
#pragma unroll
        for (int h = 0; h < KS / 4; ++h) x.bv[h] = gb[h];
    }

    // After the prologue (sRb, sI3 and P in LDS, visible to every wave): the
    // wave's tile range and the loads of its first tile.
    __device__ __forceinline__ void begin(const FwdArgs& a, const BatchCtx& c, const int32_t* sRb,
                                          const int32_t* sI3) {
        const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int gl = min(lane, c.ng - 1);   // c.ng >= 1 here; sRb has kFwdBatch + 1 entries
        const int32_t cnt = lane < c.ng ? (sRb[gl + 1] - sRb[gl] + LK - 1) / LK : 0;
        int32_t inc = cnt;
#pragma unroll
        for (int o = 1; o <= kFwdBatch; o <<= 1) {
            const int32_t y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        tpl = inc - cnt;
        const int ntile = tp(c.ng);
        const int per = (ntile + WAVES - 1) / WAVES;
        t0 = min(ntile, w * per);
        n = min(ntile, t0 + per) - t0;
        gs = 0;
        if (n > 0) {
            ids_of(a, c, sRb, sI3, 0, IA);
            load_ops(a, c, IA, OA);
            ids_of(a, c, sRb, sI3, min(1, n - 1), IB);
        }
    }

    __device__ __forceinline__ void run(const FwdArgs& a, const BatchCtx& c, const float* sP, const int32_t* sRb,
                                        const int32_t* sI3) {
        if (n <= 0) return;
        const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4;
        const int jb = N3 >= 4 ? (4 * q) % N3 : 0;   // first j3 of the lane's results
        int cur = -1;
        float bp[MT][KS];      // P[16mt + col][KS*q + s2]
        auto step = [&](int k, Ops& C, Ops& Nx, Ids& Inew, const Ids& Inext) {
            ids_of(a, c, sRb, sI3, min(k + 2, n - 1), Inew);
            load_ops(a, c, Inext, Nx);
            if (C.g != cur) {
                cur = C.g;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) bp[mt][s2] = sP[(cur * NP + 16 * mt + col) * AS + KS * q + s2];
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                floatx4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2)
                    e = __builtin_amdgcn_mfma_f32_16x16x4f32(C.bv[s2 / 4][s2 % 4], bp[mt][s2], e, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < RPL; ++u) {
                    float* dst = a.stage + (int64_t)C.r[u] * D + (16 * mt + col) * N3 + jb;
                    if constexpr (VPR == 4) {
                        *reinterpret_cast<floatx4*>(dst) = e;
                    } else if constexpr (VPR == 2) {
                        typedef float floatx2 __attribute__((ext_vector_type(2)));
                        *reinterpret_cast<floatx2*>(dst) = floatx2{e[2 * u], e[2 * u + 1]};
                    } else {
                        *dst = e[u];
                    }
                }
            }
        };
        int k = 0;
        for (; k + 1 < n; k += 2) {
            step(k, OA, OB, IA, IB);
            step(k + 1, OB, OA, IB, IA);
        }
        if (k < n) step(k, OA, OB, IA, IB);
    }
};

// Persistent workgroups (a few per CU) claim their batches from the planner's
// batch list, each in the part of its XCD class (batch_walk, batch_claims):
// the list holds only batches with groups and each part starts with its
// heaviest, so the claims hand out the heaviest batches first and the last
// ones to finish are light. Thread 0 claims two batches ahead; while a
// workgroup runs the tiles of one batch, the loads of its next batch (G2
// slice, G1 rows, run i3 list) are in flight and the record of the one after
// is in registers, so a batch's prologue costs no exposed memory round trip.
// A fixed walk of the list left the last workgroup ending about 20% after
// the median one; the claims, spread over kFwdCounters addresses, cost a few
// hundred serialised atomics per counter.
template <int N1, int N2, int R, int N3, bool KEEP>
__global__ __launch_bounds__(256, 3) void k_fwd_batch(FwdArgs a, int64_t cap, const int32_t* __restrict__ ctrl) {
    using B = PrefixBatch<N1, N2, R>;
    constexpr int SG = B::SG;
    static_assert(B::NP % 16 == 0 && 64 * B::WAVES == 256, "shape");
    __shared__ __attribute__((aligned(16))) float sU[B::U_FLOATS];   // prologue, then P
    __shared__ int32_t sRb[SG + 1];
    __shared__ int32_t sClaim[2];
    extern __shared__ int32_t sI3[];   // the batch's run i3 list

    const BatchClaims bc = batch_claims(batch_walk(ctrl), a.claims);
    if (threadIdx.x == 0) {
        sClaim[0] = atomicAdd(bc.ctr, 1);
        sClaim[1] = atomicAdd(bc.ctr, 1);
    }
    __syncthreads();
    int64_t pA = bc.pos(sClaim[0]), pB = bc.pos(sClaim[1]);
    int32_t rwA = rec_word(a.recs, pA, cap, bc.end);
    int32_t rwB = rec_word(a.recs, pB, cap, bc.end);
    BatchPf<N1, N2, R> f;
    batch_fetch<N1, N2, R>(rwA, a.run_i3, a.g1, a.g2, f);
    FwdTiles<N1, N2, R, N3> tl;
    while (pA < bc.end) {
        int32_t cc = 0;
        if (threadIdx.x == 0) cc = atomicAdd(bc.ctr, 1);   // read at the batch's end
        BatchCtx c;
        const bool live = rec_field(rwA, RW_NG) > 0;
        if (live) {
            batch_prefix<N1, N2, R>(rwA, a.run_i3, f, sU, sRb, sI3, c);
            tl.begin(a, c, sRb, sI3);   // the first tile's G3 loads go out before the next batch's
        }
        batch_fetch<N1, N2, R>(rwB, a.run_i3, a.g1, a.g2, f);
        if (live) {
            if (KEEP) store_prefix_lanes<N1, N2, R, 256>(sU, c.g0, c.ng, a.pbuf);
            tl.run(a, c, sU, sRb, sI3);
        }
        if (threadIdx.x == 0) sClaim[0] = cc;
        __syncthreads();   // sU is the next prologue's; the claim is every wave's
        const int64_t pC = bc.pos(__builtin_amdgcn_readfirstlane(sClaim[0]));
        const int32_t rwC = rec_word(a.recs, pC, cap, bc.end);
        pA = pB;
        pB = pC;
        rwA = rwB;
        rwB = rwC;
    }
}

// Bags of at most this many lookups on average take the several-bags-per-wave
// pooling kernel.
constexpr int64_t kShortBag = 16;

// One wave per bag: sum the rows of the bag's lookups (in input order) from
// the stage buffer (one row per run id) and write the bag's output row. Empty
// bags get zeros. With a hot-row cache, a hot row's lookups carry -(slot + 1)
// in place of a run id and take the row from `hot`. Rows are read as 16-byte vectors, LPR = D/4 lanes per row,
// so one load instruction covers RPI = 64/LPR rows; lane group h takes rows
// h, h + RPI, ... of the bag and the RPI partial sums are added at the end.
template <int D>
__global__ __launch_bounds__(256) void k_pool(const int32_t* __restrict__ bag_start, int64_t TB,
                                              const int32_t* __restrict__ run_of,
                                              const float* __restrict__ stage,
                                              float* __restrict__ out, int32_t* ctrl,
                                              int32_t* __restrict__ fwd_claims,
                                              const float* __restrict__ hot) {
    // the batch kernel has finished: its claim counters start from zero at
    // the next forward call
    if (blockIdx.x == 0 && threadIdx.x < kFwdCounters) fwd_claims[threadIdx.x * 32] = 0;
    constexpr int LPR = D / 4, RPI = 64 / LPR, U = 8;   // U loads in flight
    static_assert(D % 4 == 0 && 64 % LPR == 0, "row shape");
    // wave-uniform bag: its loops are scalar control flow
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int h = lane / LPR, c4 = 4 * (lane % LPR);
    const int64_t q = (int64_t)blockIdx.x * 4 + w;
    if (q >= TB) return;
    const int32_t b0 = bag_start[q];
    const int32_t b1 = max(b0, bag_start[q + 1]);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int32_t base = b0; base < b1; base += 64) {
        const int n = min(64, b1 - base);
        const int32_t rv = (lane < n) ? run_of[base + lane] : 0;
        for (int j0 = 0; j0 < n; j0 += RPI * U) {
            floatx4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + RPI * u + h;
                const int32_t slot = __shfl(rv, min(j, n - 1));
                const float* src = slot >= 0 ? stage + (int64_t)slot * D : hot + (int64_t)(-1 - slot) * D;
                v[u] = *reinterpret_cast<const floatx4*>(src + c4);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j0 + RPI * u + h < n) acc += v[u];
        }
    }
#pragma unroll
    for (int m = LPR; m < 64; m *= 2) {
        floatx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __shfl_xor(acc[e], m);
        acc += o;
    }
    if (h == 0) *reinterpret_cast<floatx4*>(out + q * D + c4) = acc;
}

// Short bags (a few lookups each): one wave takes BPW = 64/LPR bags, lane
// group h (LPR lanes, a row's 16-byte pieces) owning bag BPW*wave + h and
// summing its rows in input order. A wave pays its bag-bounds, run-id and
// row round trips once for BPW bags, where the one-bag-per-wave kernel is
// bound by those round trips when bags are short. Rows the group's bag does
// not have are loaded (clamped) and not added.
template <int D>
__global__ __launch_bounds__(256) void k_pool_short(const int32_t* __restrict__ bag_start, int64_t TB,
                                                    const int32_t* __restrict__ run_of,
                                                    const float* __restrict__ stage,
                                                    float* __restrict__ out, int32_t* ctrl,
                                                    int32_t* __restrict__ fwd_claims,
                                                    const float* __restrict__ hot) {
    if (blockIdx.x == 0 && threadIdx.x < kFwdCounters) fwd_claims[threadIdx.x * 32] = 0;
    constexpr int LPR = D / 4, BPW = 64 / LPR, U = 8;
    static_assert(D % 4 == 0 && 64 % LPR == 0, "row shape");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int h = lane / LPR, i = lane % LPR, c4 = 4 * i;
    const int64_t q = ((int64_t)blockIdx.x * 4 + w) * BPW + h;   // this lane group's bag
    const bool qv = q < TB;
    const int32_t b0 = qv ? bag_start[q] : 0;
    const int32_t b1 = qv ? max(b0, bag_start[q + 1]) : b0;
    const int32_t n = b1 - b0;
    int32_t nmax = n;   // the wave's longest bag (wave-uniform)
#pragma unroll
    for (int m = LPR; m < 64; m *= 2) nmax = max(nmax, __shfl_xor(nmax, m));
    nmax = __builtin_amdgcn_readfirstlane(nmax);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int32_t base = 0; base < nmax; base += LPR) {
        // lane i of the group: the run id of its bag's lookup base + i
        const int32_t rv = base + i < n ? run_of[b0 + base + i] : 0;
        const int jn = min(LPR, nmax - base);
        for (int j0 = 0; j0 < jn; j0 += U) {
            floatx4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t slot = __shfl(rv, h * LPR + min(j0 + u, LPR - 1));
                const float* src = slot >= 0 ? stage + (int64_t)slot * D : hot + (int64_t)(-1 - slot) * D;
                v[u] = *reinterpret_cast<const floatx4*>(src + c4);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j0 + u < jn && base + j0 + u < n) acc += v[u];
        }
    }
    if (qv) *reinterpret_cast<floatx4*>(out + q * D + c4) = acc;
}

template <int N1, int N2, int R, int N3, bool BW>
static tt_status launch_fwd_mfma(const tt_emb_plan_s* p, const float* g1, const float* g2,
                                 const float* g3, float* out, bool keep, hipStream_t s, const float* hot) {
    int32_t* fwd_claims = p->at<int32_t>(p->lay.claims) + 32 * kRunCounters;
    float* g3t = p->at<float>(p->lay.g3t);
    FwdArgs a{p->at<BatchRec>(p->lay.batch), p->at<int32_t>(p->lay.run_i3), g1, g2, g3t,
              p->at<float>(p->lay.stage), p->L, keep ? p->at<float>(p->lay.pbuf) : nullptr, fwd_claims};
    if (p->L > 0 && p->n_fb > 0) {
        TT_LAUNCH(p, "k_g3t", s, k_g3t, dim3(grid_for(p->g3_total, 256)), dim3(256), 0, s, p->desc(), p->T,
                  p->g3_total, g3, g3t);
        TT_LAUNCH_CHECK();
        const size_t lds = sizeof(int32_t) * (size_t)kFwdBatch * (size_t)p->M3;
        const int64_t grid = batch_grid(p->n_fb, kFwdPersistBlocks);
        bool kept = false;
        if constexpr (BW) {
            if (keep) {
                TT_LAUNCH(p, "k_fwd_batch_keep", s, (k_fwd_batch<N1, N2, R, N3, true>), dim3((unsigned)grid),
                          dim3(64 * PrefixBatch<N1, N2, R>::WAVES), lds, s, a, p->n_fb, p->ctrl());
                kept = true;
            }
        }
        if (!kept)
            TT_LAUNCH(p, "k_fwd_batch", s, (k_fwd_batch<N1, N2, R, N3, false>), dim3((unsigned)grid),
                      dim3(64 * PrefixBatch<N1, N2, R>::WAVES), lds, s, a, p->n_fb, p->ctrl());
        TT_LAUNCH_CHECK();
    }
    if (p->TB > 0) {
        constexpr int D = N1 * N2 * N3, BPW = 64 / (D / 4);
        if (BPW > 1 && p->L <= kShortBag * p->TB)   // short bags: several per wave
            TT_LAUNCH(p, "k_pool", s, k_pool_short<D>, dim3(grid_for(p->TB, 4 * BPW)), dim3(256), 0, s,
                      p->at<int32_t>(p->lay.bag_start), p->TB, p->at<int32_t>(p->lay.run_of),
                      p->at<float>(p->lay.stage), out, p->ctrl(), fwd_claims, hot);
        else
            TT_LAUNCH(p, "k_pool", s, k_pool<D>, dim3(grid_for(p->TB, 4)), dim3(256), 0, s,
                      p->at<int32_t>(p->lay.bag_start), p->TB, p->at<int32_t>(p->lay.run_of),
                      p->at<float>(p->lay.stage), out, p->ctrl(), fwd_claims, hot);
        TT_LAUNCH_CHECK();
    }
    return TT_OK;
}

bool mfma_shape(int n1, int n2, int n3, int R, bool backward) {
#define TT_SHAPE_IS(a, b, c, d, bw) \
    if (n1 == a && n2 == b && n3 == c && R == d) return bw || !backward;
    TT_MFMA_SHAPES(TT_SHAPE_IS)
#undef TT_SHAPE_IS
    return false;
}

// The plan's shape and the cores' alignment admit the matrix-core kernels.
bool fwd_mfma_ok(const tt_emb_plan_s* p, const float* g1, const float* g2) {
    // the prologue reads G1 rows and the G2 slice as 16-byte vectors
    if (!p->uniform || !p->off4 || ((uintptr_t)g1 & 15) != 0 || ((uintptr_t)g2 & 15) != 0) return false;
    // the batch's run i3 list is staged in LDS
    if ((int64_t)sizeof(int32_t) * kFwdBatch * p->M3 > kMaxBatchI3Bytes) return false;
    return mfma_shape(p->n1, p->n2, p->n3, p->R, false);
}

static tt_status launch_fwd(const tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3,
                            float* out, bool keep, hipStream_t s, const float* hot) {
    const int n1 = p->n1, n2 = p->n2, n3 = p->n3, R = p->R;
#define TT_FWD_CASE(a, b, c, d, bw) \
    if (n1 == a && n2 == b && n3 == c && R == d) return launch_fwd_mfma<a, b, d, c, bw>(p, g1, g2, g3, out, keep, s, hot);
    TT_MFMA_SHAPES(TT_FWD_CASE)
#undef TT_FWD_CASE
    return TT_ERR_UNSUPPORTED;
}

}  // namespace tt

using namespace tt;

tt_status tt::forward_run(tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3, float* out,
                          bool keep, uint64_t* token, hipStream_t s, const float* hot_w) {
    if (token) *token = 0;
    if (!p || !g1 || !g2 || !g3 || (!out && p->TB > 0)) return TT_ERR_INVALID_ARG;
    if (p->cached) {
        // hot rows take the matrix-core path in both directions
        if (!hot_w && p->n_hot > 0) return TT_ERR_INVALID_ARG;
        if (!fwd_mfma_ok(p, g1, g2) || !bwd_mfma_ok(p, g1, g2)) return TT_ERR_UNSUPPORTED;
    }
    if (fwd_mfma_ok(p, g1, g2)) {
        // P is kept only where the backward's matrix-core path will read it
        const bool k = keep && !p->fwd_only && bwd_mfma_ok(p, g1, g2) && p->L > 0;
        if (k) p->kept_token = 0;   // pbuf is being rewritten
        const tt_status st = launch_fwd(p, g1, g2, g3, out, k, s, hot_w);
        if (k && st == TT_OK) {
            p->kept_token = ++p->next_token;
            p->kept_g1 = g1;
            p->kept_g2 = g2;
            if (token) *token = p->kept_token;
        }
        return st;
    }
    tt_status st = fill32(p, out, 0u, p->TB * p->D, s);
    if (st != TT_OK) return st;
    if (p->lay.Cmax == 0) return TT_OK;
    int maxp = 0;
    for (int32_t t = 0; t < p->T; ++t) maxp = std::max(maxp, p->tables[t].n[0] * p->tables[t].n[1] * p->tables[t].rank);
    const size_t lds = sizeof(float) * (size_t)maxp;
    TT_LAUNCH(p, "k_fwd_generic", s, k_fwd_generic, dim3((unsigned)p->lay.Cmax), dim3(256), lds, s, p->desc(),
                       p->T, p->ctrl(), p->at<int32_t>(p->lay.group_key),
                       p->at<int32_t>(p->lay.chunk_group), p->at<int32_t>(p->lay.chunk_begin),
                       p->at<int32_t>(p->lay.chunk_end), p->at<int32_t>(p->lay.sorted_i3),
                       p->at<int32_t>(p->lay.sorted_bag), g1, g2, g3, out, p->D);
    TT_LAUNCH_CHECK();
    return TT_OK;
}

extern "C" tt_status tt_emb_forward(tt_emb_plan_t p, const float* g1, const float* g2,
                                    const float* g3, float* out, void* stream) {
    if (p && p->cached) return TT_ERR_CACHE;
    return forward_run(p, g1, g2, g3, out, false, nullptr, (hipStream_t)stream);
}

extern "C" tt_status tt_emb_forward_train(tt_emb_plan_t p, const float* g1, const float* g2,
                                          const float* g3, float* out, uint64_t* kept_token,
                                          void* stream) {
    if (kept_token) *kept_token = 0;
    if (p && p->cached) return TT_ERR_CACHE;
    return forward_run(p, g1, g2, g3, out, true, kept_token, (hipStream_t)stream);
}

extern "C" tt_status tt_emb_forward_cached(tt_emb_plan_t p, const float* g1, const float* g2,
                                           const float* g3, const float* hot_w, float* out,
                                           uint64_t* kept_token, void* stream) {
    if (kept_token) *kept_token = 0;
    if (p && !p->cached) return TT_ERR_CACHE;
    return forward_run(p, g1, g2, g3, out, kept_token != nullptr, kept_token, (hipStream_t)stream, hot_w);
}
