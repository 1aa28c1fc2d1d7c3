// Backward pass and SGD update of the TT-EmbeddingBag library.
//
// The pages evaluate training through the TT lookup (FlowTT abstract: training
// latency at batch 32,768) but give no formulas; the gradients here are those
// of the loss <grad_out, out> with respect to each core, by multilinear
// calculus on the TT chain. Per chunk, the shared prefix P = G1[i1] x G2[i2]
// is recomputed on chip; each lookup adds to dP (kept in LDS for the whole
// chunk) and to its dG3 slice; the chunk then turns dP into its dG1 and dG2
// contributions.
#include "tt_internal.h"

namespace tt {

__device__ __forceinline__ int find_table_b(const TabDev* __restrict__ desc, int32_t T, int32_t key) {
    int lo = 0, hi = T;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (desc[mid].key_base <= key) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_bwd_generic(
    const TabDev* __restrict__ desc, int32_t T, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ group_key, const int32_t* __restrict__ chunk_group,
    const int32_t* __restrict__ chunk_begin, const int32_t* __restrict__ chunk_end,
    const int32_t* __restrict__ sorted_i3, const int32_t* __restrict__ sorted_bag,
    const float* __restrict__ g1, const float* __restrict__ g2, const float* __restrict__ g3,
    const float* __restrict__ gout, float* __restrict__ dg1, float* __restrict__ dg2,
    float* __restrict__ dg3, int32_t D) {
    extern __shared__ float sm[];
    const int32_t c = blockIdx.x;
    if (c >= ctrl[CTRL_NUM_CHUNKS]) return;
    const int32_t g = chunk_group[c];
    const int32_t key = group_key[g];
    const TabDev d = desc[find_table_b(desc, T, key)];
    const int32_t local = key - d.key_base;
    const int32_t i2 = local / d.m1, i1 = local % d.m1;
    const int32_t R = d.R, n1 = d.n1, n2 = d.n2, n3 = d.n3;
    const int32_t np = n1 * n2;
    float* P = sm;            // [np][R]
    float* dP = sm + np * R;  // [np][R]
    const float* A = g1 + d.o1 + (int64_t)i1 * n1 * R;
    const float* Bc = g2 + d.o2 + (int64_t)i2 * R * n2 * R;
    const float* C0 = g3 + d.o3;
    for (int e = threadIdx.x; e < np * R; e += blockDim.x) {
        const int p = e / R, r2 = e % R;
        const int j1 = p / n2, j2 = p % n2;
        float s = 0.f;
        for (int r1 = 0; r1 < R; ++r1) s = fmaf(A[j1 * R + r1], Bc[(r1 * n2 + j2) * R + r2], s);
        P[e] = s;
    }
    __syncthreads();
    const int32_t b = chunk_begin[c], e_end = chunk_end[c];
    // dP[p][r2] = sum over the chunk's lookups of sum_j3 g[p*n3+j3] G3[i3][r2][j3]
    for (int e = threadIdx.x; e < np * R; e += blockDim.x) {
        const int p = e / R, r2 = e % R;
        float s = 0.f;
        for (int32_t l = b; l < e_end; ++l) {
            const float* gr = gout + (int64_t)sorted_bag[l] * D + p * n3;
            const float* Cs = C0 + (int64_t)sorted_i3[l] * R * n3 + r2 * n3;
            for (int j3 = 0; j3 < n3; ++j3) s = fmaf(gr[j3], Cs[j3], s);
        }
        dP[e] = s;
    }
    // dG3[i3][r2][j3] += sum_p P[p][r2] g[p*n3+j3], per lookup
    const int64_t work3 = (int64_t)(e_end - b) * R * n3;
    for (int64_t w = threadIdx.x; w < work3; w += blockDim.x) {
        const int32_t l = b + (int32_t)(w / (R * n3));
        const int32_t rem = (int32_t)(w % (R * n3));
        const int r2 = rem / n3, j3 = rem % n3;
        const float* gr = gout + (int64_t)sorted_bag[l] * D;
        float s = 0.f;
        for (int p = 0; p < np; ++p) s = fmaf(P[p * R + r2], gr[p * n3 + j3], s);
        atomicAdd(&dg3[d.o3 + (int64_t)sorted_i3[l] * R * n3 + r2 * n3 + j3], s);
    }
    __syncthreads();
    // dG1[i1][j1][r1] += sum_{j2,r2} dP[j1*n2+j2][r2] G2[i2][r1][j2][r2]
    for (int e = threadIdx.x; e < n1 * R; e += blockDim.x) {
        const int j1 = e / R, r1 = e % R;
        float s = 0.f;
        for (int j2 = 0; j2 < n2; ++j2)
            for (int r2 = 0; r2 < R; ++r2)
                s = fmaf(dP[(j1 * n2 + j2) * R + r2], Bc[(r1 * n2 + j2) * R + r2], s);
        atomicAdd(&dg1[d.o1 + (int64_t)i1 * n1 * R + e], s);
    }
    // dG2[i2][r1][j2][r2] += sum_j1 G1[i1][j1][r1] dP[j1*n2+j2][r2]
    for (int e = threadIdx.x; e < R * n2 * R; e += blockDim.x) {
        const int r1 = e / (n2 * R);
        const int rem = e % (n2 * R);
        const int j2 = rem / R, r2 = rem % R;
        float s = 0.f;
        for (int j1 = 0; j1 < n1; ++j1) s = fmaf(A[j1 * R + r1], dP[(j1 * n2 + j2) * R + r2], s);
        atomicAdd(&dg2[d.o2 + (int64_t)i2 * R * n2 * R + e], s);
    }
}

__global__ __launch_bounds__(256) void k_sgd(float* __restrict__ g, const float* __restrict__ dg,
                                             float lr, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) g[i] = fmaf(-lr, dg[i], g[i]);
}

}  // namespace tt

using namespace tt;

extern "C" tt_status tt_emb_backward(tt_emb_plan_t p, const float* g1, const float* g2,
                                     const float* g3, const float* grad_out, float* dg1,
                                     float* dg2, float* dg3, void* stream) {
    if (!p || !g1 || !g2 || !g3 || !dg1 || !dg2 || !dg3 || (!grad_out && p->TB > 0))
        return TT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    tt_status st;
    if ((st = fill32(dg1, 0u, p->extent[0], s)) != TT_OK) return st;
    if ((st = fill32(dg2, 0u, p->extent[1], s)) != TT_OK) return st;
    if ((st = fill32(dg3, 0u, p->extent[2], s)) != TT_OK) return st;
    if (p->lay.Cmax == 0) return TT_OK;
    int maxp = 0;
    for (const auto& x : p->tables) maxp = std::max(maxp, x.n[0] * x.n[1] * x.rank);
    const size_t lds = 2 * sizeof(float) * (size_t)maxp;
    hipLaunchKernelGGL(k_bwd_generic, dim3((unsigned)p->lay.Cmax), dim3(256), lds, s, p->desc(),
                       p->T, p->ctrl(), p->at<int32_t>(p->lay.group_key),
                       p->at<int32_t>(p->lay.chunk_group), p->at<int32_t>(p->lay.chunk_begin),
                       p->at<int32_t>(p->lay.chunk_end), p->at<int32_t>(p->lay.sorted_i3),
                       p->at<int32_t>(p->lay.sorted_bag), g1, g2, g3, grad_out, dg1, dg2, dg3,
                       p->D);
    TT_LAUNCH_CHECK();
    return TT_OK;
}

extern "C" tt_status tt_emb_sgd(tt_emb_plan_t p, float* g1, float* g2, float* g3,
                                const float* dg1, const float* dg2, const float* dg3, float lr,
                                void* stream) {
    if (!p || !g1 || !g2 || !g3 || !dg1 || !dg2 || !dg3) return TT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    float* gs[3] = {g1, g2, g3};
    const float* ds[3] = {dg1, dg2, dg3};
    for (int k = 0; k < 3; ++k) {
        const int64_t n = p->extent[k];
        if (n <= 0) continue;
        hipLaunchKernelGGL(k_sgd, dim3(std::min<unsigned>(grid_for(n, 256), 8192u)), dim3(256), 0,
                           s, gs[k], ds[k], lr, n);
        TT_LAUNCH_CHECK();
    }
    return TT_OK;
}
