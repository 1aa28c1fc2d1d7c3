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
// Matrix-core path for the common shapes (all tables share n1, n2, n3, R).
//
// One wave per chunk. The prefix P = G1[i1] x G2[i2] is formed once per chunk
// (VALU, into LDS) and held in registers as the A operand of
// v_mfma_f32_16x16x4_f32 for the whole chunk. Inside a group the planner has
// put repeats of one table row next to each other, so the chunk is a list of
// runs, one per distinct row; the last contraction P x G3[i3] is done once per
// run. A tile is 16 output columns = (16/n3 runs) x (n3 columns of G3), so a
// chunk wastes at most 16/n3 - 1 run slots. Each run's row leaves the matrix
// cores through LDS and is written once, as a whole row, to the stage buffer
// at the run's first sorted position; every lookup records that position in
// row_of. k_pool then sums each bag's rows in input order and writes the
// bag's output row: no atomics, and the same bits on every run.

struct FwdArgs {
    const TabDev* desc;
    int32_t T;
    int32_t* ctrl;
    const int32_t* task_start;
    const int32_t* group_key;
    const int32_t* chunk_group;
    const int32_t* chunk_begin;
    const int32_t* chunk_end;
    const int32_t* sorted_i3;
    const int32_t* perm;
    const uint8_t* run_head;
    const float* g1;
    const float* g2;
    const float* g3;
    float* stage;
    int32_t* row_of;
};

template <int N1, int N2, int R, int N3>
struct FwdShape {
    static constexpr int NP = N1 * N2;      // rows of P
    static constexpr int D = NP * N3;       // output width
    static constexpr int KS = R / 4;        // k-steps of 16x16x4 per tile
    static constexpr int MT = NP / 16;      // 16-row blocks of P
    static constexpr int LK = 16 / N3;      // runs per tile
    static constexpr int TPB = 4;           // tiles per batch
    static constexpr int BL = LK * TPB;     // runs per batch
    static constexpr int RS = D + 4;        // LDS row stride (floats)
    static constexpr int HG = 64 / R;       // lane groups sharing an r2 in the P build
    static constexpr int PE = NP * R / 64;  // P elements per lane
    static constexpr int DL = D / 64;       // output floats per lane
    static_assert(NP % 16 == 0 && R % 4 == 0 && 16 % N3 == 0 && D % 64 == 0, "shape");
    static_assert(64 % R == 0 && N2 % HG == 0 && DL <= 4 && BL <= 64, "shape");
};

template <int N1, int N2, int R, int N3>
__global__ __launch_bounds__(256) void k_fwd_mfma(FwdArgs a) {
    using S = FwdShape<N1, N2, R, N3>;
    constexpr int NP = S::NP, D = S::D, KS = S::KS, MT = S::MT, LK = S::LK, TPB = S::TPB;
    constexpr int BL = S::BL, RS = S::RS, DL = S::DL;
    __shared__ __attribute__((aligned(16))) float sP[4][NP * R];
    __shared__ float sRow[4][BL * RS];
    __shared__ float sG1[4][N1 * R];
    __shared__ int32_t sHead[4][64];
    __shared__ int32_t sHeadI3[4][64];

    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, q = lane >> 4;
    const int lk = col / N3, j3 = col % N3;
    const uint64_t below_eq = (lane == 63) ? ~0ull : ((2ull << lane) - 1);
    int32_t cur_key = -1;
    TabDev d{};
    float afr[MT][KS];

    {
        const int32_t c = span_chunk(a.ctrl[CTRL_NUM_CHUNKS], w);
        if (c >= 0) {
            const int32_t key = a.group_key[a.chunk_group[c]];
            if (key != cur_key) {
                // new group: rebuild P and reload the A operand
                cur_key = key;
                d = a.desc[find_table(a.desc, a.T, key)];
                const int32_t local = key - d.key_base;
                const int32_t i2 = local / d.m1, i1 = local % d.m1;
                build_prefix<N1, N2, R>(a.g1 + d.o1 + (int64_t)i1 * N1 * R,
                                        a.g2 + d.o2 + (int64_t)i2 * R * N2 * R, sG1[w], sP[w], lane);
                // A operand: lane (i = lane%16, q) holds P[16*mt + i][KS*q + s]
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) afr[mt][s2] = sP[w][(16 * mt + col) * R + KS * q + s2];
            }
            const int32_t s0 = a.chunk_begin[c], s1 = a.chunk_end[c];
            const float* G3 = a.g3 + d.o3;
            int32_t carried = s0;   // head of the run that continues into the next batch
            for (int32_t sb = s0; sb < s1; sb += 64) {
                const int32_t sl = sb + lane;
                const bool valid = sl < s1;
                const bool head = valid && (a.run_head[sl] != 0);
                const uint64_t m = __ballot(head);
                // every lookup records its run head
                if (valid) {
                    const uint64_t le = m & below_eq;
                    const int32_t hp = le ? sb + 63 - __builtin_clzll(le) : carried;
                    a.row_of[a.perm[sl]] = hp;
                }
                if (head) {
                    const int rk = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    sHead[w][rk] = sl;
                    sHeadI3[w][rk] = a.sorted_i3[sl];
                }
                if (m) carried = sb + 63 - __builtin_clzll(m);
                wave_lds_sync();
                const int nh = __popcll(m);
                for (int r0 = 0; r0 < nh; r0 += BL) {
                    const int nr = min(BL, nh - r0);
#pragma unroll
                    for (int tt = 0; tt < TPB; ++tt) {
                        const int ri = r0 + tt * LK + lk;
                        const int32_t i3 = (ri < nh) ? sHeadI3[w][ri] : 0;
                        const float* gb = G3 + (int64_t)i3 * R * N3 + j3 + KS * q * N3;
                        float bv[KS];
#pragma unroll
                        for (int s2 = 0; s2 < KS; ++s2) bv[s2] = gb[s2 * N3];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s2 = 0; s2 < KS; ++s2)
                                cacc = __builtin_amdgcn_mfma_f32_16x16x4f32(afr[mt][s2], bv[s2], cacc, 0, 0, 0);
                            // C[i][j]: lane holds rows 4q+v of column col -> p = 16mt + 4q + v
                            const int rr = tt * LK + lk;
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                sRow[w][rr * RS + (16 * mt + 4 * q + v) * N3 + j3] = cacc[v];
                        }
                    }
                    wave_lds_sync();
                    for (int r = 0; r < nr; ++r) {
                        const int32_t hs = sHead[w][r0 + r];
                        float* dst = a.stage + (int64_t)hs * D + lane * DL;
#pragma unroll
                        for (int k = 0; k < DL; ++k) dst[k] = sRow[w][r * RS + lane * DL + k];
                    }
                    wave_lds_sync();
                }
            }
        }
    }
}

// One wave per bag: sum the rows of the bag's lookups (in input order) from
// the stage buffer and write the bag's output row. Empty bags get zeros.
template <int DL>
__global__ __launch_bounds__(256) void k_pool(const int32_t* __restrict__ bag_start, int64_t TB,
                                              const int32_t* __restrict__ row_of,
                                              const float* __restrict__ stage,
                                              float* __restrict__ out, int32_t* ctrl) {
    constexpr int D = 64 * DL;
    reset_queues(ctrl, 0);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t q = (int64_t)blockIdx.x * 4 + w;
    if (q >= TB) return;
    const int32_t b0 = bag_start[q];
    const int32_t b1 = max(b0, bag_start[q + 1]);
    float acc[DL];
#pragma unroll
    for (int k = 0; k < DL; ++k) acc[k] = 0.f;
    for (int32_t base = b0; base < b1; base += 64) {
        const int n = min(64, b1 - base);
        const int32_t rv = (lane < n) ? row_of[base + lane] : row_of[b0];
        // 8 rows in flight; rows past n re-read a valid row and are not added
        for (int j0 = 0; j0 < n; j0 += 8) {
            float v[8][DL];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int32_t slot = __builtin_amdgcn_readlane(rv, min(j0 + u, 63));
                const float* src = stage + (int64_t)slot * D + lane * DL;
#pragma unroll
                for (int k = 0; k < DL; ++k) v[u][k] = src[k];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u < n)
#pragma unroll
                    for (int k = 0; k < DL; ++k) acc[k] += v[u][k];
        }
    }
    float* dst = out + q * D + lane * DL;
#pragma unroll
    for (int k = 0; k < DL; ++k) dst[k] = acc[k];
}

template <int N1, int N2, int R, int N3>
static tt_status launch_fwd_mfma(const tt_emb_plan_s* p, const float* g1, const float* g2,
                                 const float* g3, float* out, hipStream_t s) {
    FwdArgs a{p->desc(), p->T, p->ctrl(), p->at<int32_t>(p->lay.task_start),
              p->at<int32_t>(p->lay.group_key),
              p->at<int32_t>(p->lay.chunk_group), p->at<int32_t>(p->lay.chunk_begin),
              p->at<int32_t>(p->lay.chunk_end), p->at<int32_t>(p->lay.sorted_i3),
              p->at<int32_t>(p->lay.perm), p->at<uint8_t>(p->lay.run_head), g1, g2, g3,
              p->at<float>(p->lay.stage), p->at<int32_t>(p->lay.row_of)};
    if (p->lay.Cmax > 0) {
        hipLaunchKernelGGL((k_fwd_mfma<N1, N2, R, N3>), dim3(span_grid(p->lay.Cmax)), dim3(256), 0, s, a);
        TT_LAUNCH_CHECK();
    }
    constexpr int DL = FwdShape<N1, N2, R, N3>::DL;
    if (p->TB > 0) {
        hipLaunchKernelGGL(k_pool<DL>, dim3(grid_for(p->TB, 4)), dim3(256), 0, s,
                           p->at<int32_t>(p->lay.bag_start), p->TB, p->at<int32_t>(p->lay.row_of),
                           p->at<float>(p->lay.stage), out, p->ctrl());
        TT_LAUNCH_CHECK();
    }
    return TT_OK;
}

// Returns true (and launches) when the plan's shape has a matrix-core kernel.
static bool try_fwd_mfma(const tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3,
                         float* out, hipStream_t s, tt_status* st) {
    // the prefix build reads G2 rows as float4
    if (!p->uniform || !p->off4 || ((uintptr_t)g2 & 15) != 0) return false;
    const int n1 = p->n1, n2 = p->n2, n3 = p->n3, R = p->R;
    if (n1 == 4 && n2 == 8 && n3 == 4 && R == 32) { *st = launch_fwd_mfma<4, 8, 32, 4>(p, g1, g2, g3, out, s); return true; }
    if (n1 == 4 && n2 == 4 && n3 == 4 && R == 32) { *st = launch_fwd_mfma<4, 4, 32, 4>(p, g1, g2, g3, out, s); return true; }
    if (n1 == 4 && n2 == 4 && n3 == 4 && R == 16) { *st = launch_fwd_mfma<4, 4, 16, 4>(p, g1, g2, g3, out, s); return true; }
    return false;
}

}  // namespace tt

using namespace tt;

extern "C" tt_status tt_emb_forward(tt_emb_plan_t p, const float* g1, const float* g2,
                                    const float* g3, float* out, void* stream) {
    if (!p || !g1 || !g2 || !g3 || (!out && p->TB > 0)) return TT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    tt_status st = TT_OK;
    if (try_fwd_mfma(p, g1, g2, g3, out, s, &st)) return st;
    st = fill32(out, 0u, p->TB * p->D, s);
    if (st != TT_OK) return st;
    if (p->lay.Cmax == 0) return TT_OK;
    int maxp = 0;
    for (const auto& x : p->tables) maxp = std::max(maxp, x.n[0] * x.n[1] * x.rank);
    const size_t lds = sizeof(float) * (size_t)maxp;
    hipLaunchKernelGGL(k_fwd_generic, dim3((unsigned)p->lay.Cmax), dim3(256), lds, s, p->desc(),
                       p->T, p->ctrl(), p->at<int32_t>(p->lay.group_key),
                       p->at<int32_t>(p->lay.chunk_group), p->at<int32_t>(p->lay.chunk_begin),
                       p->at<int32_t>(p->lay.chunk_end), p->at<int32_t>(p->lay.sorted_i3),
                       p->at<int32_t>(p->lay.sorted_bag), g1, g2, g3, out, p->D);
    TT_LAUNCH_CHECK();
    return TT_OK;
}
