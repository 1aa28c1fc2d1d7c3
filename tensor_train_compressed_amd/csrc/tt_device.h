// Device helpers shared by the forward and backward kernels (gfx950, wave64).
#pragma once

#include "tt_internal.h"

#include <cstddef>

namespace tt {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

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

// Persistent grid: blocks per CU times the CU count.
inline unsigned persistent_grid(int blocks_per_cu) { return (unsigned)(256 * blocks_per_cu); }

// ---------------------------------------------------------------------------
// Prefix batches: up to kFwdBatch groups of one (table, i2) slice, one
// workgroup, described by the planner's BatchRec. batch_begin reads the record,
// then issues every load the batch needs at once (G2 slice and G1 rows as
// coalesced 16-byte loads, the run i3 list), so the prologue costs two
// dependent round trips. The G2 slice and the G1 rows go to LDS; every group's
// P = G1[i1] x G2[i2] is then formed as one (n1*batch) x (n2*R) x R product on
// the matrix cores, and P is written over the same LDS (sP[g][p][AS]).

struct BatchCtx {
    int32_t g0, ng, rb0, nr;
    int64_t o3;
};

template <int N1, int N2, int R>
struct PrefixBatch {
    static constexpr int NP = N1 * N2, N2R = N2 * R, SG = kFwdBatch;
    static constexpr int MR = SG * N1, MTP = MR / 16, NT2 = N2R / 16, KS = R / 4;
    static constexpr int GS = N2R + 16;      // LDS row stride of the G2 slice
    static constexpr int AS = R + 4;         // LDS row stride of G1 rows and of P rows
    static constexpr int WAVES = 4;
    static constexpr int NTW = (NT2 + WAVES - 1) / WAVES;   // column tiles per wave
    static constexpr int G2_FLOATS = R * GS;
    static constexpr int G1_FLOATS = MR * AS;
    static constexpr int P_FLOATS = SG * NP * AS;
    // LDS of the prologue: G2 slice then G1 rows; P is written over them
    static constexpr int U_FLOATS = (G2_FLOATS + G1_FLOATS) > P_FLOATS ? (G2_FLOATS + G1_FLOATS) : P_FLOATS;
    static_assert(16 % N1 == 0 && MR % 16 == 0 && N2R % 16 == 0 && R % 16 == 0, "prefix batch shape");
};

// The record of batch b of the list as one word per lane (lane k holds word k
// of the BatchRec; lanes past it hold word 0); all zero (ng = 0) for b >= nl,
// the list's length. The address depends only on b and the list's capacity,
// so the load need not wait for nl (a zero record reads slice 0 only).
constexpr int kRecWords = (int)(sizeof(BatchRec) / 4);
static_assert(kRecWords <= 64, "BatchRec fits one wave");
__device__ __forceinline__ int32_t rec_word(const BatchRec* __restrict__ recs, int64_t b, int64_t cap, int64_t nl) {
    const int lane = threadIdx.x & 63;
    const int32_t* w = reinterpret_cast<const int32_t*>(recs + (b < cap ? b : 0));
    const int32_t x = w[lane < kRecWords ? lane : 0];
    return b < nl ? x : 0;
}

// The batch of round r of workgroup w among G persistent workgroups: a snake
// over the list (r*G + w on even rounds, r*G + G-1-w on odd ones), so that the
// workgroups given the list's first, heaviest batches get its lighter ones
// next.
__device__ __forceinline__ int64_t snake(int64_t r, int64_t w, int64_t G) {
    return r * G + ((r & 1) ? G - 1 - w : w);
}

// The part of the batch list a persistent workgroup walks, and its place
// among the workgroups walking it. When the list's XCD-class parts are about
// equal (and the grid is a multiple of kXcds), workgroup w walks the part of
// its own class, w mod kXcds (it runs on that XCD, whose L2 then holds that
// class's G2 slices), in a snake over that class's workgroups; otherwise (a
// few slices hold most batches) the whole list, in a snake over all.
struct BatchWalk {
    int64_t base, n, wi, G;
    bool classed;
    __device__ __forceinline__ int64_t at(int64_t r) const { return base + snake(r, wi, G); }
    __device__ __forceinline__ bool has(int64_t r) const { return snake(r, wi, G) < n; }
};
__device__ __forceinline__ BatchWalk batch_walk(const int32_t* __restrict__ ctrl) {
    const int64_t G = gridDim.x, w = blockIdx.x;
    int32_t cb[kXcds + 1];
#pragma unroll
    for (int c = 0; c <= kXcds; ++c) cb[c] = ctrl[CTRL_CLASS_BASE + c];
    const int64_t nl = cb[kXcds];
    int64_t mx = 0;
#pragma unroll
    for (int c = 0; c < kXcds; ++c) mx = max(mx, (int64_t)(cb[c + 1] - cb[c]));
    BatchWalk bw{0, nl, w, G, false};
    if (G % kXcds == 0 && mx * kXcds <= nl + nl / 4 + 4 * kXcds) {
        const int c = (int)(w % kXcds);
        bw.base = cb[c];
        bw.n = cb[c + 1] - cb[c];
        bw.wi = w / kXcds;
        bw.G = G / kXcds;
        bw.classed = true;
    }
    return bw;
}

// Claimed batches: workgroup b claims from counter cidx = b mod kFwdCounters;
// claim j of that counter is batch base + j*stride + off of the walked part
// (classed: the kFwdCounters/kXcds counters of the part's class interleave
// over it; otherwise all kFwdCounters over the whole list), so each counter
// hands out its share in list order, heaviest first.
struct BatchClaims {
    int64_t base, end, stride, off;
    int32_t* ctr;
    __device__ __forceinline__ int64_t pos(int32_t j) const { return base + (int64_t)j * stride + off; }
};
__device__ __forceinline__ BatchClaims batch_claims(const BatchWalk& bw, int32_t* __restrict__ counters) {
    const int cidx = (int)(blockIdx.x % kFwdCounters);
    BatchClaims c;
    c.base = bw.base;
    c.end = bw.base + bw.n;
    c.stride = bw.classed ? kFwdCounters / kXcds : kFwdCounters;
    c.off = bw.classed ? cidx / kXcds : cidx;
    c.ctr = counters + cidx * 32;
    return c;
}

// Persistent grid of a batch kernel: a multiple of kFwdCounters (so every
// counter, and every class, has its workgroups), at most `cap`.
inline unsigned batch_grid(int64_t slots, int64_t cap) {
    static_assert(kFwdPersistBlocks % kFwdCounters == 0, "grid of whole counter sets");
    const int64_t g = std::min<int64_t>(cap, (slots + kFwdCounters - 1) / kFwdCounters * kFwdCounters);
    return (unsigned)std::max<int64_t>(g, kFwdCounters);
}
__device__ __forceinline__ int32_t rec_field(int32_t rw, int k) { return __builtin_amdgcn_readlane(rw, k); }
__device__ __forceinline__ int64_t rec_field64(int32_t rw, int k) {
    return (int64_t)(uint32_t)__builtin_amdgcn_readlane(rw, k) |
           ((int64_t)__builtin_amdgcn_readlane(rw, k + 1) << 32);
}
// word offsets of the BatchRec fields
enum RecWord : int { RW_NG = 0, RW_G0 = 1, RW_I2 = 2, RW_RB0 = 3, RW_NR = 4, RW_O1 = 8, RW_O2 = 10,
                     RW_O3 = 12, RW_I1 = 16, RW_RBASE = 24 };
static_assert(offsetof(BatchRec, o1) == 4 * RW_O1 && offsetof(BatchRec, o3) == 4 * RW_O3 &&
              offsetof(BatchRec, i1) == 4 * RW_I1 && offsetof(BatchRec, rbase) == 4 * RW_RBASE &&
              offsetof(BatchRec, nr) == 4 * RW_NR, "BatchRec words");

// Registers that carry one batch's operands from their loads to LDS.
template <int N1, int N2, int R>
struct BatchPf {
    using B = PrefixBatch<N1, N2, R>;
    static constexpr int NT = 64 * B::WAVES;
    static constexpr int NQ = R * B::N2R / 4, NV = (NQ + NT - 1) / NT;          // G2 slice, float4
    static constexpr int Q1 = N1 * R / 4, NQ1 = kFwdBatch * Q1, NV1 = (NQ1 + NT - 1) / NT;   // G1 rows
    static constexpr int NI = 4;                                                // run i3 values
    floatx4 v[NV];
    floatx4 u[NV1];
    int32_t i3[NI];
};

// Issues the loads of batch `rw` (all threads; nothing when ng = 0). Groups
// past ng read G1[0] (the record's i1 is 0 there); their P rows are written
// but never read.
template <int N1, int N2, int R>
__device__ __forceinline__ void batch_fetch(int32_t rw, const int32_t* __restrict__ run_i3,
                                            const float* __restrict__ g1, const float* __restrict__ g2,
                                            BatchPf<N1, N2, R>& f) {
    using F = BatchPf<N1, N2, R>;
    constexpr int N2R = N2 * R, NT = F::NT;
    const int tid = threadIdx.x, lane = tid & 63;
    const floatx4* G2s = reinterpret_cast<const floatx4*>(g2 + rec_field64(rw, RW_O2) +
                                                        (int64_t)rec_field(rw, RW_I2) * R * N2R);
#pragma unroll
    for (int k = 0; k < F::NV; ++k) f.v[k] = G2s[min(tid + NT * k, F::NQ - 1)];
    const float* G1b = g1 + rec_field64(rw, RW_O1);
#pragma unroll
    for (int k = 0; k < F::NV1; ++k) {
        const int e = min(tid + NT * k, F::NQ1 - 1);
        const int32_t i1 = __shfl(rw, RW_I1 + e / F::Q1);
        f.u[k] = reinterpret_cast<const floatx4*>(G1b + (int64_t)i1 * N1 * R)[e % F::Q1];
    }
    const int32_t rb0 = rec_field(rw, RW_RB0), nr = rec_field(rw, RW_NR);
#pragma unroll
    for (int j = 0; j < F::NI; ++j) {
        const int e = tid + NT * j;
        f.i3[j] = run_i3[rb0 + max(0, min(e, nr - 1))];
    }
    (void)lane;
}

// Moves a fetched batch into LDS and forms its prefixes. All WAVES waves call
// it (only for ng > 0); it ends with the block synchronised, sU holding P (row
// g*NP + p at stride AS), sRb[0..kFwdBatch] the groups' first row runs relative
// to rb0 and sI3[0..nr) the batch's run i3 values.
template <int N1, int N2, int R>
__device__ __forceinline__ void batch_prefix(int32_t rw, const int32_t* __restrict__ run_i3,
                                             const BatchPf<N1, N2, R>& f, float* sU, int32_t* sRb,
                                             int32_t* sI3, BatchCtx& c) {
    using B = PrefixBatch<N1, N2, R>;
    using F = BatchPf<N1, N2, R>;
    constexpr int NP = B::NP, N2R = B::N2R, MTP = B::MTP, KS = B::KS, GS = B::GS, AS = B::AS;
    constexpr int WAVES = B::WAVES, NT2 = B::NT2, NTW = B::NTW, NT = F::NT;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 15,
              q = lane >> 4;   // w wave-uniform: branches and loops on it are scalar
    c.ng = rec_field(rw, RW_NG); c.g0 = rec_field(rw, RW_G0);
    c.rb0 = rec_field(rw, RW_RB0); c.nr = rec_field(rw, RW_NR); c.o3 = rec_field64(rw, RW_O3);
    float* sG2 = sU;
    float* sG1 = sU + B::G2_FLOATS;
#pragma unroll
    for (int k = 0; k < F::NV; ++k) {
        const int e4 = tid + NT * k;
        if (e4 < F::NQ) *reinterpret_cast<floatx4*>(sG2 + ((4 * e4) / N2R) * GS + (4 * e4) % N2R) = f.v[k];
    }
#pragma unroll
    for (int k = 0; k < F::NV1; ++k) {
        const int e = tid + NT * k;   // group e / Q1, element 4*(e % Q1) = (j1, r1)
        if (e < F::NQ1) {
            const int x = 4 * (e % F::Q1);
            *reinterpret_cast<floatx4*>(sG1 + ((e / F::Q1) * N1 + x / R) * AS + x % R) = f.u[k];
        }
    }
#pragma unroll
    for (int j = 0; j < F::NI; ++j) {
        const int e = tid + NT * j;
        if (e < c.nr) sI3[e] = f.i3[j];
    }
    for (int e = tid + NT * F::NI; e < c.nr; e += NT) sI3[e] = run_i3[c.rb0 + e];
    const int32_t rbw = __shfl(rw, RW_RBASE + min(lane, kFwdBatch));
    if (tid <= kFwdBatch) sRb[tid] = rbw;
    __syncthreads();
    // wave w: column tiles nt = w + WAVES*k, every row tile mt (row 16mt + i =
    // group (16mt + i)/N1, j1 = (16mt + i)%N1); K = r1
    floatx4 acc[NTW][MTP];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        const int nt = min(w + WAVES * k, NT2 - 1);
        float bf[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) bf[s2] = sG2[(4 * s2 + q) * GS + 16 * nt + col];
#pragma unroll
        for (int mt = 0; mt < MTP; ++mt) {
            acc[k][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                acc[k][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sG1[(16 * mt + col) * AS + 4 * s2 + q], bf[s2],
                                                                  acc[k][mt], 0, 0, 0);
        }
    }
    __syncthreads();
    float* sP = sU;
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        const int nt = w + WAVES * k;
        if (nt < NT2) {
#pragma unroll
            for (int mt = 0; mt < MTP; ++mt) {
                // C row 4q+v2 of tile mt = (group, j1) of row 16mt + 4q + v2;
                // column cc = 16nt + col = (j2, r2)
                const int cc = 16 * nt + col;
#pragma unroll
                for (int v2 = 0; v2 < 4; ++v2) {
                    const int rho = 16 * mt + 4 * q + v2, gi = rho / N1, j1 = rho % N1;
                    sP[(gi * NP + j1 * N2 + cc / R) * AS + cc % R] = acc[k][mt][v2];
                }
            }
        }
    }
    __syncthreads();
}

// Stores the batch's P (in LDS, row gi*NP + p at stride AS) to pbuf in the
// lane order of the backward run kernel's matrix-core operand: float4 number
// x = ((rt*KQ + h)*4 + q)*16 + col of a group holds P[4*(4h + u) + q][16*rt +
// col], u = 0..3 (KQ = n1*n2/16), so that lane (col, q) reads its whole
// operand as RT*KQ float4. All NT threads of the workgroup call it.
template <int N1, int N2, int R, int NT>
__device__ __forceinline__ void store_prefix_lanes(const float* sP, int32_t g0, int ng, float* __restrict__ pbuf) {
    using B = PrefixBatch<N1, N2, R>;
    constexpr int NP = B::NP, AS = B::AS, KQ = NP / 16, PF4 = NP * R / 4;
    static_assert(NP % 16 == 0 && R % 16 == 0, "shape");
    for (int e4 = threadIdx.x; e4 < ng * PF4; e4 += NT) {
        const int gi = e4 / PF4, x = e4 % PF4;
        const int col = x & 15, q = (x >> 4) & 3, h = (x >> 6) % KQ, rt = (x >> 6) / KQ;
        const float* src = sP + (gi * NP + 16 * h + q) * AS + 16 * rt + col;
        const floatx4 v = {src[0], src[4 * AS], src[8 * AS], src[12 * AS]};
        *reinterpret_cast<floatx4*>(pbuf + ((int64_t)(g0 + gi) * PF4 + x) * 4) = v;
    }
}

}  // namespace tt
