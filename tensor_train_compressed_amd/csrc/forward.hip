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
#include "tt_internal.h"

namespace tt {

__device__ __forceinline__ int find_table(const TabDev* __restrict__ desc, int32_t T, int32_t key) {
    int lo = 0, hi = T;  // last t with key_base <= key
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (desc[mid].key_base <= key) lo = mid; else hi = mid;
    }
    return lo;
}

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

}  // namespace tt

using namespace tt;

extern "C" tt_status tt_emb_forward(tt_emb_plan_t p, const float* g1, const float* g2,
                                    const float* g3, float* out, void* stream) {
    if (!p || !g1 || !g2 || !g3 || (!out && p->TB > 0)) return TT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    tt_status st = fill32(out, 0u, p->TB * p->D, s);
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
