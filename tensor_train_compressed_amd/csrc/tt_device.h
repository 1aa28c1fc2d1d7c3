// Device helpers shared by the forward and backward kernels (gfx950, wave64).
#pragma once

#include "tt_internal.h"

namespace tt {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int find_table(const TabDev* __restrict__ desc, int32_t T, int32_t key) {
    int lo = 0, hi = T;  // last t with key_base <= key
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (desc[mid].key_base <= key) lo = mid; else hi = mid;
    }
    return lo;
}

// Orders this wave's LDS writes before its later LDS reads (LDS executes a
// wave's operations in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// P[p][r2] = sum_r1 G1[i1][j1][r1] G2[i2][r1][j2][r2] (p = j1*N2 + j2) into
// sP, one wave, VALU. Lane owns r2 = lane % R and rows p = h + HG*k.
template <int N1, int N2, int R>
__device__ __forceinline__ void build_prefix(const float* __restrict__ A, const float* __restrict__ Bc,
                                             float* sG1, float* sP, int lane) {
    constexpr int NP = N1 * N2, HG = 64 / R, PE = NP * R / 64, J2N = N2 / HG;
    for (int e = lane; e < N1 * R; e += 64) sG1[e] = A[e];
    wave_lds_sync();
    const int r2 = lane % R, h = lane / R;
    float acc[PE];
#pragma unroll
    for (int k = 0; k < PE; ++k) acc[k] = 0.f;
#pragma unroll 4
    for (int r1 = 0; r1 < R; ++r1) {
        float b2[J2N];
#pragma unroll
        for (int jj = 0; jj < J2N; ++jj) b2[jj] = Bc[(r1 * N2 + h + HG * jj) * R + r2];
#pragma unroll
        for (int k = 0; k < PE; ++k)  // p = h + HG*k: j2 = h + HG*(k % J2N), j1 = k / J2N
            acc[k] = fmaf(sG1[(k / J2N) * R + r1], b2[k % J2N], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < PE; ++k) sP[(h + HG * k) * R + r2] = acc[k];
    wave_lds_sync();
}

}  // namespace tt
