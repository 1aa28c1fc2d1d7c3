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
// Matrix-core path for the common shapes (n1 = 4, n3 = 4, shared n2 and R).
//
// One workgroup (8 waves) per batch of up to kFwdBatch prefix groups of one
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

struct FwdArgs {
    const TabDev* desc;
    int32_t T;
    const int32_t* ctrl;
    int64_t K;
    const uint64_t* key_scan;
    const int32_t* group_key;
    const int32_t* group_rbase;
    const int32_t* run_i3;
    const float* g1;
    const float* g2;
    const float* g3;
    float* stage;
};

template <int N1, int N2, int R, int N3>
struct FwdShape {
    static constexpr int NP = N1 * N2;      // rows of P
    static constexpr int N2R = N2 * R;      // columns of a G2 slice row
    static constexpr int D = NP * N3;       // output width
    static constexpr int SG = kFwdBatch;    // groups per batch
    static constexpr int MR = SG * N1;      // rows of the batched prefix product
    static constexpr int MTP = MR / 16;     // row tiles of the prefix product
    static constexpr int NT2 = N2R / 16;    // column tiles of the prefix product
    static constexpr int KS = R / 4;        // k-steps over r
    static constexpr int MT = NP / 16;      // row tiles of P
    static constexpr int LK = 16 / N3;      // runs per suffix tile
    static constexpr int GS = N2R + 16;     // LDS row stride of G2
    static constexpr int AS = R + 4;        // LDS row stride of P rows
    static constexpr int WAVES = 8;
    static constexpr int NTW = NT2 * MTP / WAVES;   // prefix tiles per wave
    static_assert(N1 == 4 && N3 == 4 && NP % 16 == 0 && N2R % 32 == 0 && R % 4 == 0, "shape");
    static_assert(WAVES % MTP == 0 && (NT2 * MTP) % WAVES == 0, "wave split");
};

template <int N1, int N2, int R, int N3>
__global__ __launch_bounds__(512) void k_fwd_batch(FwdArgs a) {
    using S = FwdShape<N1, N2, R, N3>;
    constexpr int NP = S::NP, N2R = S::N2R, D = S::D, SG = S::SG, MTP = S::MTP, NTW = S::NTW;
    constexpr int KS = S::KS, MT = S::MT, LK = S::LK, GS = S::GS, AS = S::AS, WAVES = S::WAVES;
    __shared__ __attribute__((aligned(16))) float sG2[R * GS];
    __shared__ float sP[SG * NP * AS];
    __shared__ int32_t sRb[SG + 1];
    __shared__ int32_t sTp[SG + 1];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, col = lane & 15, q = lane >> 4;
    // batch -> table, slice, group range
    const int32_t b = blockIdx.x;
    int t = 0;
    {
        int lo = 0, hi = a.T;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.desc[mid].fb_base <= b) lo = mid; else hi = mid;
        }
        t = lo;
    }
    const TabDev* dp = a.desc + t;
    const int32_t m1 = dp->m1, fb = dp->fb_base;
    const int64_t o1 = dp->o1, o2 = dp->o2, o3 = dp->o3;
    const int32_t nb = (m1 + SG - 1) / SG;
    const int32_t i2 = (b - fb) / nb, jb = (b - fb) % nb;
    const int64_t kb = (int64_t)dp->key_base + (int64_t)i2 * m1;
    const int64_t ke = kb + m1;
    const int32_t gs0 = (int32_t)(a.key_scan[kb] >> 32);
    const int32_t gs1 = ke < a.K ? (int32_t)(a.key_scan[ke] >> 32) : a.ctrl[CTRL_NUM_GROUPS];
    const int32_t g0 = gs0 + SG * jb;
    if (g0 >= gs1) return;
    const int ng = min(SG, gs1 - g0);

    // ---- G2 slice into LDS; prefix A operand (G1 rows) straight into registers
    {
        const float4* G2s = reinterpret_cast<const float4*>(a.g2 + o2 + (int64_t)i2 * R * N2R);
        constexpr int NQ = R * N2R / 4, NV = (NQ + 64 * WAVES - 1) / (64 * WAVES);
        float4 v[NV];
        constexpr bool even = NQ % (64 * WAVES) == 0;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int e4 = tid + 64 * WAVES * k;
            v[k] = (even || e4 < NQ) ? G2s[even ? e4 : min(e4, NQ - 1)] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int e4 = tid + 64 * WAVES * k;
            if (even || e4 < NQ) *reinterpret_cast<float4*>(sG2 + ((4 * e4) / N2R) * GS + (4 * e4) % N2R) = v[k];
        }
        if (tid <= ng) sRb[tid] = a.group_rbase[g0 + tid];
    }
    const int mtp = w % MTP;                  // prefix row tile: groups 4*mtp .. 4*mtp+3
    const int gA = 4 * mtp + col / N1;        // group of this lane's A row (col = 4*(g%4) + j1)
    float af[KS];
    {
        const bool live = gA < ng;
        const int32_t i1 = live ? (int32_t)(a.group_key[g0 + gA] - kb) : 0;
        const float* G1r = a.g1 + o1 + (int64_t)i1 * N1 * R + (col % N1) * R;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) af[s2] = live ? G1r[4 * s2 + q] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        sTp[0] = 0;
        for (int gi = 0; gi < ng; ++gi) {
            acc += (sRb[gi + 1] - sRb[gi] + LK - 1) / LK;
            sTp[gi + 1] = acc;
        }
    }

    // ---- batched prefix: rows (g, j1) of the G1 stack x G2 slice -> P_g[(j1, j2)][r2]
    if (4 * mtp < ng) {
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
            const int nt = w / MTP + (WAVES / MTP) * k;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[s2], sG2[(4 * s2 + q) * GS + 16 * nt + col],
                                                           acc, 0, 0, 0);
            // C row 4q+v = (group 4*mtp+q, j1 v); column c = 16nt + col = (j2, r2)
            const int gi = 4 * mtp + q, c = 16 * nt + col;
#pragma unroll
            for (int v = 0; v < 4; ++v) sP[(gi * NP + v * N2 + c / R) * AS + c % R] = acc[v];
        }
    }
    __syncthreads();

    // ---- runs: tiles of LK runs of one group, spread over the waves; the
    // next tile's run index and G3 operand are fetched before this tile's math
    const int ntile = sTp[ng];
    const int lk = col / N3, j3 = col % N3;
    const float* G3 = a.g3 + o3 + j3 + KS * q * N3;
    int cur = -1, gnext = 0;
    float afr[MT][KS];
    int tau = w;
    int32_t r = 0;
    bool valid = false;
    float bv[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) bv[s2] = 0.f;
    if (tau < ntile) {
        while (sTp[gnext + 1] <= tau) ++gnext;
        r = sRb[gnext] + LK * (tau - sTp[gnext]) + lk;
        valid = r < sRb[gnext + 1];
        const float* gb = G3 + (int64_t)(valid ? a.run_i3[r] : 0) * R * N3;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) bv[s2] = gb[s2 * N3];
    }
    for (; tau < ntile; tau += WAVES) {
        const int gi = gnext;
        if (gi != cur) {
            cur = gi;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) afr[mt][s2] = sP[(gi * NP + 16 * mt + col) * AS + KS * q + s2];
        }
        // prefetch the next tile
        const int tn = tau + WAVES;
        int32_t rn = 0;
        bool vn = false;
        float bn[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) bn[s2] = 0.f;
        if (tn < ntile) {
            while (sTp[gnext + 1] <= tn) ++gnext;
            rn = sRb[gnext] + LK * (tn - sTp[gnext]) + lk;
            vn = rn < sRb[gnext + 1];
            const float* gb = G3 + (int64_t)(vn ? a.run_i3[rn] : 0) * R * N3;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) bn[s2] = gb[s2 * N3];
        }
        float* dst = a.stage + (int64_t)r * D + j3;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                cacc = __builtin_amdgcn_mfma_f32_16x16x4f32(afr[mt][s2], bv[s2], cacc, 0, 0, 0);
            // C[i][j]: lane holds rows 4q+v of column col -> p = 16mt + 4q + v
            if (valid) {
#pragma unroll
                for (int v = 0; v < 4; ++v) dst[(16 * mt + 4 * q + v) * N3] = cacc[v];
            }
        }
        r = rn;
        valid = vn;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) bv[s2] = bn[s2];
    }
}

// One wave per bag: sum the rows of the bag's lookups (in input order) from
// the stage buffer (one row per run id) and write the bag's output row. Empty
// bags get zeros.
template <int DL>
__global__ __launch_bounds__(256) void k_pool(const int32_t* __restrict__ bag_start, int64_t TB,
                                              const int32_t* __restrict__ run_of,
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
        const int32_t rv = (lane < n) ? run_of[base + lane] : run_of[b0];
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
    FwdArgs a{p->desc(), p->T, p->ctrl(), p->K, p->at<uint64_t>(p->lay.key_scan),
              p->at<int32_t>(p->lay.group_key), p->at<int32_t>(p->lay.group_rbase),
              p->at<int32_t>(p->lay.run_i3), g1, g2, g3, p->at<float>(p->lay.stage)};
    if (p->L > 0 && p->n_fb > 0) {
        hipLaunchKernelGGL((k_fwd_batch<N1, N2, R, N3>), dim3((unsigned)p->n_fb), dim3(512), 0, s, a);
        TT_LAUNCH_CHECK();
    }
    constexpr int DL = FwdShape<N1, N2, R, N3>::D / 64;
    if (p->TB > 0) {
        hipLaunchKernelGGL(k_pool<DL>, dim3(grid_for(p->TB, 4)), dim3(256), 0, s,
                           p->at<int32_t>(p->lay.bag_start), p->TB, p->at<int32_t>(p->lay.run_of),
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
