// Backward pass and SGD update of the TT-EmbeddingBag library.
//
// The pages evaluate training through the TT lookup (FlowTT abstract: training
// latency at batch 32,768) but give no formulas; the gradients here are those
// of the loss <grad_out, out> with respect to each core, by multilinear
// calculus on the TT chain. The generic kernel below works per chunk with
// fp32 atomics; the matrix-core kernels further down work per row run and per
// group, with fp64 sums where long cancelling sequences meet.
#include "tt_device.h"

namespace tt {

__global__ __launch_bounds__(256) void k_bwd_generic(
    const TabDev* __restrict__ desc, int32_t T, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ group_key, const int32_t* __restrict__ chunk_group,
    const int32_t* __restrict__ chunk_begin, const int32_t* __restrict__ chunk_end,
    const int32_t* __restrict__ sorted_i3, const int32_t* __restrict__ sorted_bag,
    const float* __restrict__ g1, const float* __restrict__ g2, const float* __restrict__ g3,
    const float* __restrict__ gout, double* __restrict__ a1, double* __restrict__ a2,
    double* __restrict__ a3, int32_t D) {
    extern __shared__ double smd[];
    const int32_t c = blockIdx.x;
    if (c >= ctrl[CTRL_NUM_CHUNKS]) return;
    const int32_t g = chunk_group[c];
    const int32_t key = group_key[g];
    const TabDev d = desc[find_table(desc, T, key)];
    const int32_t local = key - d.key_base;
    const int32_t i2 = local / d.m1, i1 = local % d.m1;
    const int32_t R = d.R, n1 = d.n1, n2 = d.n2, n3 = d.n3;
    const int32_t np = n1 * n2;
    double* dP = smd;                                      // [np][R]
    float* P = reinterpret_cast<float*>(smd + np * R);     // [np][R]
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
    // (fp64: a hot row's lookups add up many large, cancelling terms)
    for (int e = threadIdx.x; e < np * R; e += blockDim.x) {
        const int p = e / R, r2 = e % R;
        double s = 0.0;
        for (int32_t l = b; l < e_end; ++l) {
            const float* gr = gout + (int64_t)sorted_bag[l] * D + p * n3;
            const float* Cs = C0 + (int64_t)sorted_i3[l] * R * n3 + r2 * n3;
            for (int j3 = 0; j3 < n3; ++j3) s = fma((double)gr[j3], (double)Cs[j3], s);
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
        double s = 0.0;
        for (int p = 0; p < np; ++p) s = fma((double)P[p * R + r2], (double)gr[p * n3 + j3], s);
        atomicAdd(&a3[d.o3 + (int64_t)sorted_i3[l] * R * n3 + r2 * n3 + j3], s);
    }
    __syncthreads();
    // dG1[i1][j1][r1] += sum_{j2,r2} dP[j1*n2+j2][r2] G2[i2][r1][j2][r2]
    for (int e = threadIdx.x; e < n1 * R; e += blockDim.x) {
        const int j1 = e / R, r1 = e % R;
        double s = 0.0;
        for (int j2 = 0; j2 < n2; ++j2)
            for (int r2 = 0; r2 < R; ++r2)
                s = fma(dP[(j1 * n2 + j2) * R + r2], (double)Bc[(r1 * n2 + j2) * R + r2], s);
        atomicAdd(&a1[d.o1 + (int64_t)i1 * n1 * R + e], s);
    }
    // dG2[i2][r1][j2][r2] += sum_j1 G1[i1][j1][r1] dP[j1*n2+j2][r2]
    for (int e = threadIdx.x; e < R * n2 * R; e += blockDim.x) {
        const int r1 = e / (n2 * R);
        const int rem = e % (n2 * R);
        const int j2 = rem / R, r2 = rem % R;
        double s = 0.0;
        for (int j1 = 0; j1 < n1; ++j1) s = fma((double)A[j1 * R + r1], dP[(j1 * n2 + j2) * R + r2], s);
        atomicAdd(&a2[d.o2 + (int64_t)i2 * R * n2 * R + e], s);
    }
}

// Where the backward's gradient elements go: into the gradient buffers, or,
// for the backward fused with the SGD step, into the cores themselves,
// G <- G - lr * dG with dG rounded to fp32 first (the same operations as the
// SGD kernel, so the same bits). The fused form writes only the slices that
// some lookup touches.
struct GradOut {
    float neg_lr;
    int32_t sgd;
};
__device__ __forceinline__ void put_grad(float* p, float g, GradOut o) {
    if (o.sgd) *p = fmaf(o.neg_lr, g, *p);
    else *p = g;
}

// dG1 (and dG3 when n3 > 0) from their fp64 accumulators (fused SGD: an
// element whose sum is zero, untouched, is left alone).
__global__ __launch_bounds__(256) void k_bwd_finish(const double* __restrict__ a1, float* __restrict__ dg1,
                                                    int64_t n1, const double* __restrict__ a3,
                                                    float* __restrict__ dg3, int64_t n3, int32_t* ctrl,
                                                    GradOut go, const float* __restrict__ b2,
                                                    float* __restrict__ g2, int64_t n2) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    if (tid == 0) ctrl[CTRL_NUM_XPIECES] = 0;   // the next backward on this plan appends from 0
    for (int64_t i = tid; i < n1; i += nth) {
        const double a = a1[i];
        if (!go.sgd || a != 0.0) put_grad(dg1 + i, (float)a, go);
    }
    // fused SGD: G2 from the dG2 buffer (rounded to fp32 already; zero on the
    // slices no lookup touched, which keep their values), four elements per
    // thread and step when both buffers are 16-byte aligned
    int64_t done = 0;
    if ((((uintptr_t)b2 | (uintptr_t)g2) & 15) == 0) {
        const int64_t n4 = n2 / 4;
        const floatx4* b4 = reinterpret_cast<const floatx4*>(b2);
        floatx4* g4 = reinterpret_cast<floatx4*>(g2);
        for (int64_t i = tid; i < n4; i += nth) {
            const floatx4 b = b4[i];
            if (b[0] != 0.f || b[1] != 0.f || b[2] != 0.f || b[3] != 0.f) {
                floatx4 g = g4[i];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (b[e] != 0.f) g[e] = fmaf(go.neg_lr, b[e], g[e]);
                g4[i] = g;
            }
        }
        done = n4 * 4;
    }
    for (int64_t i = done + tid; i < n2; i += nth) {
        const float b = b2[i];
        if (b != 0.f) put_grad(g2 + i, b, go);
    }
    for (int64_t i = tid; i < n3; i += nth) {
        const double a = a3[i];
        if (!go.sgd || a != 0.0) put_grad(dg3 + i, (float)a, go);
    }
}

// G_k <- G_k - lr * dG_k for the three cores in one launch (16-byte accesses
// where both buffers allow them).
struct SgdArgs {
    float* g[3];
    const float* dg[3];
    int64_t n[3];
};

__global__ __launch_bounds__(256) void k_sgd(SgdArgs a, float lr) {
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float* g = a.g[k];
        const float* dg = a.dg[k];
        const int64_t n = a.n[k];
        int64_t done = 0;
        if ((((uintptr_t)g | (uintptr_t)dg) & 15) == 0) {
            const int64_t n4 = n / 4;
            floatx4* g4 = reinterpret_cast<floatx4*>(g);
            const floatx4* d4 = reinterpret_cast<const floatx4*>(dg);
            for (int64_t i = t0; i < n4; i += stride) {
                const floatx4 x = g4[i], d = d4[i];
                g4[i] = floatx4{fmaf(-lr, d[0], x[0]), fmaf(-lr, d[1], x[1]), fmaf(-lr, d[2], x[2]),
                                fmaf(-lr, d[3], x[3])};
            }
            done = 4 * n4;
        }
        for (int64_t i = done + t0; i < n; i += stride) g[i] = fmaf(-lr, dg[i], g[i]);
    }
}


// ---------------------------------------------------------------------------
// Matrix-core backward for the common shapes (n1 = 4, n3 = 4, shared by all
// tables). The kernels, all on row runs (one run per distinct table row of a
// group, the same runs the forward contracts):
//
// bwd_prep      (the first workgroups of the k_bwd_sum launch) zeroes the
//               fp64 accumulators (dG1; dG3 when it is added with atomics),
//               the completion and claim counters, scans the dG3 buckets'
//               run counts, and lists the pieces of the groups of more than
//               kRunRange runs (a group whose pieces would not fit the list
//               runs whole)
// k_bwd_sum     one wave per window of 64 sorted positions: for every run,
//               S = sum of the grad_out rows of its lookups, accumulated in
//               fp64. A run inside one window is stored once, rounded to fp32;
//               the pieces of a run cut by window ends go to fp64 slots, one
//               per piece. Memory-bound.
// k_bwd_cross   adds up the pieces of the cut runs in fp64 and rounds them
//               into their S rows (a hot row's run spans many windows: an
//               fp32 sum of its pieces would lose the fp32 tolerance on the
//               slices it feeds); its extra workgroups write the dG3 bucket
//               lists
// k_bwd_pfx     forms P of every group (persistent workgroups over the
//               forward's batch list) into the P buffer; skipped when the
//               training forward kept P
// k_bwd_runs_c3 one wave per unit (a listed piece of up to kRunRange runs of
//               one group, or a whole group), claimed from 32 counters, the
//               group's P in registers; per tile of 4 runs, on the matrix
//               cores,
//                 c3[run]  = P^T S          (R x n3, fp32; over the run's S)
//                 dP_g    += S G3[i3]^T     (n1*n2 x R, fp64, in registers)
//               dP is stored over the group's P (a split group's pieces go to
//               fp64 slots, the last piece adds them); k_bwd_runs adds P^T S
//               to the fp64 dG3 accumulator with atomics instead
// k_bwd_dg123   three kinds of workgroups in one launch:
//               dG3: one per G3 row, dG3[i3] = sum of its runs' c3 rows
//               dG1: one wave per batch slot, slice-major,
//                 dG1[i1] += dP G2[i2]^T    (fp64 products, one fp64 atomic
//                                            per element and group)
//               dG2: one wave per (slice, 16-column tile of dG2[i2]),
//                 dG2[i2] = sum G1[i1]^T dP (fp64 products, plain stores, owned)
// k_bwd_finish  dG1 (and atomics-mode dG3) <- their fp64 accumulators, rounded
//               to fp32
// With the fused SGD (GradOut::sgd) the gradients are not stored: dG3's
// workgroups and k_bwd_finish apply G <- G - lr * dG to the core elements
// instead, only on the rows and slices the batch touches; dG2 goes to a
// buffer (zero on untouched slices) that k_bwd_finish applies to G2, since
// G2 is read for dG1 in the same launch.

__device__ __forceinline__ bool row_head(const int32_t* __restrict__ skey, int64_t s) {
    return s == 0 || skey[s - 1] != skey[s];
}

// The grad-row sums run over fixed windows of kWin sorted positions (one
// wave each). A row run that crosses a window end is summed piece by piece:
// the piece of window w that starts at w's first position (when that is not a
// run head) goes to fp64 slot 2w, the piece that starts at a head inside w and
// runs past w's end goes to slot 2w + 1. No two pieces share a slot.
constexpr int kWin = 64;


struct CrossRef {
    const int32_t* skey;
    const int32_t* rid;
    const int32_t* run_start;
    int64_t L;
};

struct PrepArgs {
    double* dg1;
    int64_t n1;
    double* dg3;
    int64_t n3;
    int32_t* xcnt;
    int64_t nwin;
    int32_t* claims;
    const int32_t* i3cnt;
    int32_t m3;
    int32_t* i3start;
    const int32_t* group_rbase;
    int32_t* xpiece;
    int64_t xcap;
    int32_t* gdone;
    int32_t* ctrl;
};

// The backward's set-up, run by the first kPrepBlocks workgroups of the
// grad-sum launch (nothing it writes is read before the kernels after it).
constexpr int kPrepBlocks = 256;

__device__ __forceinline__ void bwd_prep(const PrepArgs& pa, int64_t blk) {
    double* __restrict__ dg1 = pa.dg1;
    double* __restrict__ dg3 = pa.dg3;
    const int64_t n1 = pa.n1, n3 = pa.n3, nwin = pa.nwin;
    const int32_t m3 = pa.m3;
    int32_t* ctrl = pa.ctrl;
    const int64_t tid = blk * blockDim.x + threadIdx.x;
    const int64_t nth = (int64_t)kPrepBlocks * blockDim.x;
    if (m3 > 0 && blk == 0) {
        // first run slot of each dG3 bucket: exclusive scan of the planner's
        // counts, 1024 at a time (four per thread)
        __shared__ int32_t wtot[4];
        __shared__ int32_t carry;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        if (threadIdx.x == 0) carry = 0;
        for (int base = 0; base < m3; base += 4 * 256) {
            int32_t c[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = base + 4 * threadIdx.x + j;
                c[j] = i < m3 ? pa.i3cnt[(int64_t)i * kI3Pad] : 0;
                sum += c[j];
            }
            int32_t inc = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            if (lane == 63) wtot[w] = inc;
            __syncthreads();
            int32_t run = carry + inc - sum;
            for (int ww = 0; ww < w; ++ww) run += wtot[ww];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = base + 4 * threadIdx.x + j;
                if (i < m3) pa.i3start[i] = run;
                run += c[j];
            }
            __syncthreads();   // every thread has read carry and wtot
            if (threadIdx.x == 255) carry = run;
            __syncthreads();
        }
        if (threadIdx.x == 0) pa.i3start[m3] = carry;   // the total
    }
    for (int64_t i = tid; i < n1; i += nth) dg1[i] = 0.0;
    for (int64_t i = tid; i < n3; i += nth) dg3[i] = 0.0;
    for (int64_t i = tid; i < nwin; i += nth) pa.xcnt[i] = 0;
    if (tid < kRunCounters) pa.claims[tid * 32] = 0;
    // groups of more than kRunRange runs are split into pieces of kRunRange
    // runs: list their pieces, a group's pieces together and in order (the
    // run kernel takes these first, then one piece per other group)
    // (at most xcap pieces: a group whose pieces do not all fit is not listed,
    // gdone = -1, and runs whole; the slots it took below xcap are marked
    // empty with group -1)
    const int64_t U = ctrl[CTRL_NUM_GROUPS];
    for (int64_t g = tid; g < U; g += nth) {
        int32_t gd = 0;
        const int32_t np = (pa.group_rbase[g + 1] - pa.group_rbase[g] + kRunRange - 1) / kRunRange;
        if (np > 1) {
            const int32_t base = atomicAdd(ctrl + CTRL_NUM_XPIECES, np);
            const bool fits = (int64_t)base + np <= pa.xcap;
            if (!fits) gd = -1;
            for (int32_t k = 0; k < np && (int64_t)base + k < pa.xcap; ++k) {
                pa.xpiece[2 * (base + k)] = fits ? (int32_t)g : -1;
                pa.xpiece[2 * (base + k) + 1] = k;
            }
        }
        pa.gdone[g] = gd;
    }
}

// S of the cut runs. Windows go in spans of WV = 16 (one workgroup per
// span, wave v on window 16*span + v). Wave v checks its window for a run that
// starts in it and runs past its end (the check's loads go out in two
// rounds). A run whose pieces lie in at most SHORT + 1 windows is summed by
// that wave alone: its end piece plus the start pieces of the windows up to
// the one holding its last lookup, all loads in flight at once, in fp64.
// A longer run (a hot row, spanning up to thousands of windows) is summed by
// every span it touches: each adds the start pieces of its own windows (one
// per wave, added across the waves in LDS) into the run's end-piece slot with
// fp64 device atomics, then counts itself in the run's counter; the span that
// completes the count rounds the slot into the run's S row. At most one long
// run starts in a span and at most one enters it from before.
struct SlotArgs {
    const int32_t* i3start;
    const int32_t* run_bkt;
    const int32_t* run_rank;
    int32_t* bucket_runs;
};

// Workgroups past the first nspan (when bucketing dG3): each run's place in
// the list of its bucket's runs (its bucket's start plus its rank in the
// bucket), read by dG3's workgroups of k_bwd_dg123.
template <int DL>
__global__ __launch_bounds__(1024) void k_bwd_cross(double* __restrict__ xpart, int32_t* __restrict__ xcnt,
                                                    CrossRef x, float* __restrict__ S,
                                                    const int32_t* __restrict__ ctrl, int64_t nspan,
                                                    SlotArgs sl) {
    constexpr int D = 64 * DL, WV = 16, SHORT = 16;
    if ((int64_t)blockIdx.x >= nspan) {
        const int64_t r = ((int64_t)blockIdx.x - nspan) * blockDim.x + threadIdx.x;
        if (r < ctrl[CTRL_NUM_RUNS]) sl.bucket_runs[sl.i3start[sl.run_bkt[r]] + sl.run_rank[r]] = (int32_t)r;
        return;
    }
    static_assert(SHORT >= WV, "a long run leaves the span it starts in");
    __shared__ double red[WV][D];
    __shared__ int32_t s_run[2];      // long run that starts in the span / enters it (-1: none)
    __shared__ int64_t s_hw[2], s_lw[2];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwin = (x.L + kWin - 1) / kWin;
    const int32_t NR = ctrl[CTRL_NUM_RUNS];
    for (int64_t w0 = (int64_t)blockIdx.x * WV; w0 < nwin; w0 += nspan * WV) {
        const int64_t w = w0 + wv;
        const int64_t e = (w + 1) * kWin;   // first position after window w
        int32_t run = -1;
        int64_t last = 0;
        if (e < x.L) {
            const int32_t k0 = x.skey[e - 1], k1 = x.skey[e];
            const int32_t r1 = x.rid[e];
            if (k0 == k1) {   // the run holding position e - 1 continues past the window
                const int32_t rr = r1 - 1;
                const int32_t rs = x.run_start[rr];
                const int64_t re = rr + 1 < NR ? x.run_start[rr + 1] : x.L;
                if (rs >= e - kWin) {   // ... and starts in it
                    run = rr;
                    last = (re - 1) / kWin;
                }
            }
        }
        if (run >= 0 && last - w <= SHORT) {
            double v[SHORT + 1][DL];
#pragma unroll
            for (int u = 0; u <= SHORT; ++u) {
                const int64_t slot = u == 0 ? 2 * w + 1 : 2 * min(w + u, last);
#pragma unroll
                for (int k = 0; k < DL; ++k) v[u][k] = xpart[slot * D + lane * DL + k];
            }
            double acc[DL];
#pragma unroll
            for (int k = 0; k < DL; ++k) acc[k] = v[0][k];
#pragma unroll
            for (int u = 1; u <= SHORT; ++u)
                if (w + u <= last) {
#pragma unroll
                    for (int k = 0; k < DL; ++k) acc[k] += v[u][k];
                }
            float* dst = S + (int64_t)run * D + lane * DL;
#pragma unroll
            for (int k = 0; k < DL; ++k) dst[k] = (float)acc[k];
        }
        if (wv == 0 && lane == 0) {
            s_run[0] = -1;
            s_run[1] = -1;
            // the run holding the span's first position, when it started in
            // an earlier span and is long
            const int64_t f = w0 * kWin;
            if (f > 0 && x.skey[f - 1] == x.skey[f]) {
                const int32_t rr = x.rid[f] - 1;
                const int64_t rs = x.run_start[rr];
                const int64_t re = rr + 1 < NR ? x.run_start[rr + 1] : x.L;
                const int64_t hw = rs / kWin, lw = (re - 1) / kWin;
                if (lw - hw > SHORT) {
                    s_run[1] = rr;
                    s_hw[1] = hw;
                    s_lw[1] = lw;
                }
            }
        }
        __syncthreads();
        if (run >= 0 && last - w > SHORT && lane == 0) {
            s_run[0] = run;
            s_hw[0] = w;
            s_lw[0] = last;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int32_t lr = s_run[c];
            if (lr < 0) continue;
            const int64_t hw = s_hw[c], lw = s_lw[c];
            // this span's windows holding start pieces of the run
            const int64_t j = w0 + wv;
            const bool mine = j > hw && j <= lw;
#pragma unroll
            for (int k = 0; k < DL; ++k) red[wv][lane * DL + k] = mine ? xpart[2 * j * D + lane * DL + k] : 0.0;
            __syncthreads();
            if (wv == 0) {
                double* accp = xpart + (2 * hw + 1) * D + lane * DL;
#pragma unroll
                for (int k = 0; k < DL; ++k) {
                    double t = 0.0;
#pragma unroll
                    for (int i = 0; i < WV; ++i) t += red[i][lane * DL + k];
                    atomicAdd(accp + k, t);
                }
                // counted once the adds have completed (device atomics are
                // performed at the level all XCDs share; no device-scope
                // fence, which would write back the whole L2)
                wait_vmem_done();
                int32_t done = 0;
                if (lane == 0) {
                    const int32_t need = (int32_t)(lw / WV - hw / WV + 1);
                    done = atomicAdd(xcnt + hw, 1) == need - 1 ? 1 : 0;
                }
                if (__builtin_amdgcn_readfirstlane(done)) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                    float* dst = S + (int64_t)lr * D + lane * DL;
#pragma unroll
                    for (int k = 0; k < DL; ++k)
                        dst[k] = (float)__hip_atomic_load(accp + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();
        }
        __syncthreads();   // every wave is done with s_run before the next span rewrites it
    }
}

struct SumArgs {
    const int32_t* sorted_bag;
    const int32_t* skey;
    const int32_t* rid;
    const int32_t* run_start;
    int64_t L;
    const float* gout;
    float* S;
    double* xpart;
};

// S[run] = sum of the grad rows of the run's lookups, in fp64. One wave per
// window of kWin sorted positions (fixed stride over the windows): the
// window's bag ids, run ids and run heads come in one round of loads, then its
// grad rows FL at a time, added in order; a run is stored (rounded to fp32)
// when it starts and ends in the window, otherwise its piece goes to its
// fp64 slot (no atomics: every slot has one writer).
template <int DL>
__global__ __launch_bounds__(256) void k_bwd_sum(SumArgs a, PrepArgs pa) {
    constexpr int D = 64 * DL, FL = 32;   // grad_out rows in flight
    if (blockIdx.x < kPrepBlocks) {
        bwd_prep(pa, blockIdx.x);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t nwin = (a.L + kWin - 1) / kWin;
    const int64_t nw = ((int64_t)(gridDim.x - kPrepBlocks) * blockDim.x) >> 6;
    // the wave index is uniform: held in scalar registers, so the window's
    // control flow below is scalar branches, not lane masks
    const int64_t w0 = (int64_t)(blockIdx.x - kPrepBlocks) * (blockDim.x >> 6) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t w = w0; w < nwin; w += nw) {
        const int64_t s0 = w * kWin;
        const int n = (int)min((int64_t)kWin, a.L - s0);
        const int64_t s1 = s0 + n;
        const bool tail_whole = (s1 == a.L) || row_head(a.skey, s1);
        const int64_t sl = s0 + lane;
        const bool valid = lane < n;
        const bool hr = valid && row_head(a.skey, sl);
        const uint64_t m = __ballot(hr);
        const int32_t bagv = a.sorted_bag[valid ? sl : s0];
        const int32_t rrv = valid ? a.rid[sl] + (hr ? 1 : 0) - 1 : 0;
        int32_t cur = 0, cur_r = 0;
        bool cur_head = false;
        double sacc[DL];
#pragma unroll
        for (int k = 0; k < DL; ++k) sacc[k] = 0.0;
        // a piece that starts at a head and ends inside the window (or at its
        // end, the next window starting a new run) is the whole run; a run of
        // one lookup is not stored (the run kernel reads its grad row)
        auto flush = [&](bool ends_here, int r_end) {
            if (cur_head && ends_here && r_end - cur_r == 1) return;
            if (cur_head && ends_here) {
                float* dst = a.S + (int64_t)cur * D + lane * DL;
#pragma unroll
                for (int k = 0; k < DL; ++k) dst[k] = (float)sacc[k];
            } else {
                double* dst = a.xpart + (2 * w + (cur_head ? 1 : 0)) * D + lane * DL;
#pragma unroll
                for (int k = 0; k < DL; ++k) dst[k] = sacc[k];
            }
        };
        // the runs of one lookup (heads followed by a head or the window's
        // whole end): their sums are not kept, so their row loads read the
        // window's first row again (an L1 hit) instead of a grad row
        const uint64_t nexth = (m >> 1) | (tail_whole ? (1ull << (n - 1)) : 0ull);
        const uint64_t one = m & nexth;
        const int32_t bag0 = __builtin_amdgcn_readfirstlane(bagv);
        for (int r0 = 0; r0 < n; r0 += FL) {
            float v[FL][DL];
#pragma unroll
            for (int u = 0; u < FL; ++u) {
                const int r = min(r0 + u, 63);
                const int32_t bg = ((one >> r) & 1ull) ? bag0 : __builtin_amdgcn_readlane(bagv, r);
                const float* row = a.gout + (int64_t)bg * D + lane * DL;
#pragma unroll
                for (int k = 0; k < DL; ++k) v[u][k] = row[k];
            }
#pragma unroll
            for (int u = 0; u < FL; ++u) {
                const int r = r0 + u;
                if (r < n) {
                    if (r == 0 || ((m >> r) & 1ull)) {
                        if (r != 0) flush(true, r);   // the previous piece ends at a row head
                        cur = __builtin_amdgcn_readlane(rrv, r);
                        cur_r = r;
                        cur_head = ((m >> r) & 1ull) != 0;
#pragma unroll
                        for (int k = 0; k < DL; ++k) sacc[k] = 0.0;
                    }
#pragma unroll
                    for (int k = 0; k < DL; ++k) sacc[k] += (double)v[u][k];
                }
            }
        }
        flush(tail_whole, n);
    }
}

// P of every group, for the run kernel. Persistent workgroups walk the
// planner's prefix batches like the forward (the next batch's loads are in
// flight while the current one is formed) and store each group's P in the
// lane order the run kernel reads it (store_prefix_lanes). Skipped when the
// forward kept P on this plan for the same G1 and G2.
template <int N1, int N2, int R>
__global__ __launch_bounds__(256) void k_bwd_pfx(const BatchRec* __restrict__ recs, int64_t cap,
                                                 const int32_t* __restrict__ ctrl,
                                                 const int32_t* __restrict__ run_i3,
                                                 const float* __restrict__ g1, const float* __restrict__ g2,
                                                 float* __restrict__ pbuf) {
    using B = PrefixBatch<N1, N2, R>;
    constexpr int SG = B::SG;
    static_assert(64 * B::WAVES == 256, "shape");
    __shared__ __attribute__((aligned(16))) float sU[B::U_FLOATS];
    __shared__ int32_t sRb[SG + 1];
    extern __shared__ int32_t sI3[];
    const BatchWalk bw = batch_walk(ctrl);
    const int64_t end = bw.base + bw.n;
    int32_t rwA = rec_word(recs, bw.at(0), cap, end);
    int32_t rwB = rec_word(recs, bw.at(1), cap, end);
    BatchPf<N1, N2, R> f;
    batch_fetch<N1, N2, R>(rwA, run_i3, g1, g2, f);
    for (int64_t r = 0; bw.has(r); ++r) {
        const int32_t rwC = rec_word(recs, bw.at(r + 2), cap, end);
        BatchCtx c;
        const bool live = rec_field(rwA, RW_NG) > 0;
        if (live) batch_prefix<N1, N2, R>(rwA, run_i3, f, sU, sRb, sI3, c);
        batch_fetch<N1, N2, R>(rwB, run_i3, g1, g2, f);
        if (live) {
            store_prefix_lanes<N1, N2, R, 256>(sU, c.g0, c.ng, pbuf);
            __syncthreads();
        }
        rwA = rwB;
        rwB = rwC;
    }
}

// Run units. A piece is kRunRange consecutive runs of one group. Units
// 0..X-1 are the listed pieces of the groups with more than kRunRange runs
// (bwd_prep's list: a group's pieces together and in order, the largest work
// first; -1 in place of a group that did not fit the list's capacity); unit
// X + g is group g whole when it has at most kRunRange runs or was not
// listed, and nothing otherwise.
struct RunsArgs {
    const TabDev* desc;
    int32_t T;
    const int32_t* ctrl;
    const int32_t* xpiece;
    int64_t xcap;              // capacity of the piece list
    const int32_t* group_rbase;
    const int32_t* group_key;
    const int32_t* run_i3;
    const float* S;
    float* pbuf;               // P per group; each group's dP is written over it
    const float* g3;
    double* dg3;
    double* dpart;
    int32_t* gdone;            // per group: pieces finished (zeroed by bwd_prep); -1: not listed
    int32_t* claims;           // [kRunCounters][32]: unit counters (zeroed by bwd_prep)
    const int32_t* run_cslot;  // hot-row cache: each run's slot (-1: not hot); null without a cache
    float* hot;                // the hot rows' gradients dW [n_hot][D], or (fused SGD) W itself
    GradOut hgo;               // how a hot run's S goes into `hot`
    const int32_t* run_bag1;   // per run: the bag of a run of one lookup, else -1
    const float* gout;         // grad rows: S of a run of one lookup
};

// One wave per unit, the group's P in registers. Persistent waves claim their
// units: the waves of workgroup b from counter c = b mod kRunCounters, whose
// j-th claim is unit j*kRunCounters + c (the list's order inside each
// counter's share: listed pieces, the largest work, first). A wave claims its
// next unit when it starts the current one, so the claim's round trip hides
// behind the unit's work. A fixed stride over the units left the last wave
// ending 29% after the median one; the claims spread over kRunCounters
// addresses keep each counter's serialised atomics well inside the kernel's
// run time.
// four runs at a time (lane group q takes run t0 + q):
//   dG3[i3] += P^T S          fp32 products over p, handed to add3 (device
//                              atomics, or the run's own row, reduced later)
//   dP      += S G3[i3]^T     fp64 products and sums over the unit
// then dP is written, rounded to fp32, over the group's P (every piece of the
// group has read P by then), or, for a listed piece, its fp64 partial goes to
// the piece's own slot and the group's last piece to finish (a counter per
// group) adds the group's slots in piece order and writes the sum once. A
// whole group of more than kRunRange runs (one that did not fit the list) is
// walked kRunRange runs at a time, dP summed across them in registers.
template <int N1, int N2, int R, int N3, class Add3>
__device__ __forceinline__ void runs_body(const RunsArgs& a, Add3 add3) {
    constexpr int NP = N1 * N2, D = NP * N3, PR = NP * R, MT = NP / 16, RT = R / 16, KSP = NP / 4;
    constexpr int KQ = KSP / 4, CN = R * N3, W = kRunRange;
    static_assert(N3 == 4 && NP % 16 == 0 && R % 16 == 0 && W <= 64 && PR % 256 == 0, "shape");
    const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4;
    const int lk = col / N3, j3 = col % N3;
    const int32_t U = a.ctrl[CTRL_NUM_GROUPS];
    const int32_t X = (int32_t)min((int64_t)a.ctrl[CTRL_NUM_XPIECES], a.xcap);
    const int64_t nunits = (int64_t)X + U;
    const int cidx = (int)(blockIdx.x % kRunCounters);
    int32_t* ctr = a.claims + cidx * 32;
    auto claim_issue = [&]() { int32_t v = 0; if (lane == 0) v = atomicAdd(ctr, 1); return v; };
    auto claim_unit = [&](int32_t v) { return (int64_t)__builtin_amdgcn_readfirstlane(v) * kRunCounters + cidx; };
    // A unit's words (group, mode, runs) and, per lane j, the i3 of its run
    // s + j are fetched during the unit before it: the words at that unit's
    // start, the run i3 values after its tiles.
    struct Words {
        int64_t g;
        int32_t mode;          // 0: nothing, 1: a listed piece, 2: the whole group
        int32_t part, s, e;    // piece number; first run and end of the unit's runs
    };
    auto words_of = [&](int64_t kk, Words& w) {
        int64_t g = kk - X;
        int32_t part = 0, mode = 2;
        if (kk < X) {
            g = a.xpiece[2 * kk];
            part = a.xpiece[2 * kk + 1];
            mode = 1;
            if (g < 0) { g = 0; mode = 0; }
        }
        const int32_t gs = a.group_rbase[g], ge = a.group_rbase[g + 1];
        if (mode == 2 && ge - gs > W && a.gdone[g] >= 0) mode = 0;   // listed: done piece by piece
        w.g = g;
        w.mode = mode;
        w.part = part;
        w.s = mode == 1 ? gs + W * part : gs;
        w.e = mode == 1 ? min(ge, w.s + W) : ge;
    };
    int64_t k = claim_unit(claim_issue());
    if (k >= nunits) return;
    int32_t kn_raw = claim_issue();   // the next unit's claim, read at the next unit
    auto o3_of = [&](int64_t g) { return a.desc[find_table(a.desc, a.T, a.group_key[g])].o3; };
    // a tile's operands (S rows in both layouts, G3 rows of its runs) for the
    // runs t0 .. t0+3 of the walked range [s, e) (i3w: lane j holds the i3 of
    // run s + j; lanes past e read run t0 or e - 1, whose results go unused)
    struct TileOps {
        floatx4 av[MT], bq[RT];
        float bv[KSP];
        int32_t i3q;
        int32_t csq;           // hot-row slot of run t0 + q (-1: not hot)
    };
    // (b1w: lane j holds run s + j's bag when the run has one lookup, else -1:
    // then the run's S is that grad row)
    auto srow = [&](int32_t r, int32_t b1) {
        return b1 >= 0 ? a.gout + (int64_t)b1 * D : a.S + (int64_t)r * D;
    };
    auto load_tile = [&](int32_t t0, int32_t s, int32_t e, int32_t i3w, int32_t b1w, int64_t o3, TileOps& o) {
        const int32_t rq = t0 + q < e ? t0 + q : t0;
        o.i3q = __shfl(i3w, rq - s);
        o.csq = a.run_cslot ? a.run_cslot[rq] : -1;
        const float* Sq = srow(rq, __shfl(b1w, rq - s));
        const float* G3q = a.g3 + o3 + (int64_t)o.i3q * CN;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o.av[mt] = *reinterpret_cast<const floatx4*>(Sq + (16 * mt + col) * N3);
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) o.bq[nt] = *reinterpret_cast<const floatx4*>(G3q + (16 * nt + col) * N3);
        const int32_t rl = min(t0 + lk, e - 1);
        const float* Sl = srow(rl, __shfl(b1w, rl - s)) + j3;
#pragma unroll
        for (int s2 = 0; s2 < KSP; ++s2) o.bv[s2] = Sl[(4 * s2 + q) * N3];
    };
    Words cur;
    words_of(k, cur);
    int64_t o3 = o3_of(cur.g);
    int32_t i3l = a.run_i3[min(cur.s + lane, cur.e - 1)];   // lane j: i3 of run s + j
    int32_t b1l = a.run_bag1[min(cur.s + lane, cur.e - 1)];  // lane j: bag of run s + j (one lookup)
    for (;;) {
        const int64_t kn = claim_unit(kn_raw);
        kn_raw = claim_issue();
        const int64_t g = cur.g;
        const bool work = cur.mode != 0;
        // this unit's P and first tile go out first; the next unit's words,
        // G3 offset and run i3 values are fetched while they are in flight
        floatx4 preg[RT][KQ];
        TileOps TA, TB;
        if (work) {
            const floatx4* Pp = reinterpret_cast<const floatx4*>(a.pbuf + g * PR) + 16 * q + col;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int h = 0; h < KQ; ++h) preg[rt][h] = Pp[(rt * KQ + h) * 64];
            load_tile(cur.s, cur.s, min(cur.e, cur.s + W), i3l, b1l, o3, TA);
        }
        Words nxt;
        words_of(min(kn, nunits - 1), nxt);
        const int64_t o3n = o3_of(nxt.g);
        const int32_t i3n = a.run_i3[min(nxt.s + lane, nxt.e - 1)];
        const int32_t b1n = a.run_bag1[min(nxt.s + lane, nxt.e - 1)];
        if (work) {
        doublex4 dacc[MT][RT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) dacc[mt][nt] = doublex4{0.0, 0.0, 0.0, 0.0};
        for (int32_t s = cur.s;;) {
        const int32_t e = min(cur.e, s + W);
        auto tile = [&](int32_t t0, TileOps& o) {
            const bool okq = t0 + q < e;
            // a hot row's run: its S is the hot row's gradient, and it adds
            // nothing to the cores' gradients
            const bool hotq = okq && o.csq >= 0;
            // dG3: rows (run t0 + lk, j3) of P^T S; lane (col, q) gets run
            // t0 + q, r2 = 16rt + col, j3 = v
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KSP; ++s2)
                    cc = __builtin_amdgcn_mfma_f32_16x16x4f32(o.bv[s2], preg[rt][s2 / 4][s2 % 4], cc, 0, 0, 0);
                if (okq) add3(o3 + (int64_t)o.i3q * CN, (16 * rt + col) * N3, t0 + q,
                              hotq ? floatx4{0.f, 0.f, 0.f, 0.f} : cc);
            }
            if (hotq) {
                // lane (col, q) holds S[run t0 + q][(16mt + col)*n3 + 0..3]
                float* hr = a.hot + (int64_t)o.csq * D + col * N3;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) put_grad(hr + 16 * mt * N3 + v, o.av[mt][v], a.hgo);
            }
            // dP: K = (run q, j3 = step), fp64 products and sums (a hot
            // group's dP adds up hundreds of runs of large S); a run past the
            // piece adds zeros
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const floatx4 av = okq && !hotq ? o.av[mt] : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nt = 0; nt < RT; ++nt)
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        dacc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av[st], (double)o.bq[nt][st],
                                                                            dacc[mt][nt], 0, 0, 0);
            }
        };
        for (int32_t t0 = s;; t0 += 8) {
            load_tile(min(t0 + 4, e - 1), s, e, i3l, b1l, o3, TB);
            tile(t0, TA);
            if (t0 + 4 >= e) break;
            load_tile(min(t0 + 8, e - 1), s, e, i3l, b1l, o3, TA);
            tile(t0 + 4, TB);
            if (t0 + 8 >= e) break;
        }
        s = e;
        if (s >= cur.e) break;
        // a whole group's next kRunRange runs
        i3l = a.run_i3[min(s + lane, cur.e - 1)];
        b1l = a.run_bag1[min(s + lane, cur.e - 1)];
        load_tile(s, s, min(cur.e, s + W), i3l, b1l, o3, TA);
        }
        // the fp64 product's lane (col, q) holds dP[16mt + q + 4v][16nt + col];
        // a listed piece keeps its fp64 partial in its own slot
        const bool piece = cur.mode == 1;
        float* dst = a.pbuf + g * PR;
        double* dpp = a.dpart + k * PR;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < RT; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int idx = (16 * mt + q + 4 * v) * R + 16 * nt + col;
                    if (piece)   // device-scope stores: written through to the level all XCDs share
                        __hip_atomic_store(dpp + idx, dacc[mt][nt][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        dst[idx] = (float)dacc[mt][nt][v];
                }
        if (piece) {
            // count the piece once its slot's stores have completed (a wait,
            // not a device-scope fence: that one writes back the whole L2)
            const int32_t gs = a.group_rbase[g], ge = a.group_rbase[g + 1];
            const int32_t np = (ge - gs + W - 1) / W;
            wait_vmem_done();
            int32_t done = 0;
            if (lane == 0) done = atomicAdd(a.gdone + g, 1) == np - 1 ? 1 : 0;
            if (__builtin_amdgcn_readfirstlane(done)) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                const double* first = a.dpart + (k - cur.part) * PR;   // the group's pieces are listed in order
                for (int e0 = 0; e0 < PR; e0 += 64 * 4) {
                    double t[4] = {0.0, 0.0, 0.0, 0.0};
                    for (int32_t j = 0; j < np; ++j) {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            t[u] += __hip_atomic_load(first + (int64_t)j * PR + e0 + 64 * u + lane, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) dst[e0 + 64 * u + lane] = (float)t[u];
                }
            }
        }
        }
        if (kn >= nunits) break;
        i3l = i3n;
        b1l = b1n;
        o3 = o3n;
        cur = nxt;
        k = kn;
    }
}

// dG3 added straight to the fp64 accumulator with device atomics (tables
// whose G3 rows are not aligned to R*n3, or too many G3 rows)
template <int N1, int N2, int R, int N3>
__global__ __launch_bounds__(256) void k_bwd_runs(RunsArgs a) {
    runs_body<N1, N2, R, N3>(a, [&](int64_t row, int within, int32_t, const floatx4& c) {
#pragma unroll
        for (int v = 0; v < 4; ++v) atomicAdd(a.dg3 + row + within + v, (double)c[v]);
    });
}

// Each run's dG3 term P^T S is stored as a row of its own: row r of c3 (at
// row stride c3s; c3 is the S buffer itself when an S row holds R*n3 floats,
// each run's term then replacing its S, which only this wave reads), and
// k_bwd_dg123 sums the rows of each G3 row's bucket. Device atomics from every
// CU on the same few hundred G3 slices saturate the memory-side atomic
// units, and LDS float atomics are slow on the CU; plain stores avoid both.
template <int N1, int N2, int R, int N3>
__global__ __launch_bounds__(256, R >= 64 ? 2 : 3) void k_bwd_runs_c3(RunsArgs a, float* __restrict__ c3, int64_t c3s) {
    runs_body<N1, N2, R, N3>(a, [&](int64_t, int within, int32_t run, const floatx4& c) {
        *reinterpret_cast<floatx4*>(c3 + (int64_t)run * c3s + within) = c;
    });
}

// dG3[i3] = sum of the c3 rows of the runs in bucket i3 (bucket_runs lists
// them), in fp64: one workgroup of WAVES waves per G3 row, wave w on rows w,
// w + WAVES, ... of the bucket, GB rows in flight; the waves' sums are added
// in LDS at the end.
struct Dg3Args {
    const int32_t* i3start;
    const int32_t* bucket_runs;
    const float* c3;
    int64_t c3s;
    float* dg3;
    GradOut go;
};

template <int CN, int WAVES>
__device__ __forceinline__ void dg3_body(const Dg3Args& a, int32_t row, double (&red)[WAVES][CN]) {
    constexpr int PL = CN / 64, GB = 16;
    static_assert(CN % 64 == 0, "shape");
    const int32_t b = a.i3start[row], e = a.i3start[row + 1];
    if (a.go.sgd && b == e) return;   // an untouched G3 row keeps its values
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    double acc[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) acc[k] = 0.0;
    for (int32_t j0 = b + w; j0 < e; j0 += WAVES * GB) {
        // lane j < GB: the run of bucket row j0 + WAVES * j
        const int32_t rl = a.bucket_runs[min(j0 + WAVES * min(lane, GB - 1), e - 1)];
        float x[GB][PL];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            const float* src = a.c3 + (int64_t)__builtin_amdgcn_readlane(rl, j) * a.c3s + lane * PL;
#pragma unroll
            for (int k = 0; k < PL; ++k) x[j][k] = src[k];
        }
#pragma unroll
        for (int j = 0; j < GB; ++j)
            if (j0 + WAVES * j < e) {
#pragma unroll
                for (int k = 0; k < PL; ++k) acc[k] += (double)x[j][k];
            }
    }
#pragma unroll
    for (int k = 0; k < PL; ++k) red[w][lane * PL + k] = acc[k];
    __syncthreads();
    for (int t = threadIdx.x; t < CN; t += 64 * WAVES) {
        double x = 0.0;
#pragma unroll
        for (int k = 0; k < WAVES; ++k) x += red[k][t];
        put_grad(a.dg3 + (int64_t)row * CN + t, (float)x, a.go);
    }
}

// dG2[i2] = sum over the slice's groups of G1[i1]^T dP_g, one wave per
// (slice, 16-column tile of the n2*R columns), every r1 tile: K = the
// (group, j1) pairs taken four at a time (one group per fp64 matrix-core step
// when n1 = 4), operands read straight from memory (each dP element once;
// the next UNR steps' loads issued before the current ones' products), no
// LDS and no barrier. The wave owns its columns: plain stores.
struct Dg2Args {
    const TabDev* desc;
    int32_t T;
    const int32_t* ctrl;
    int64_t K;
    const uint64_t* key_scan;
    const int32_t* group_key;
    const float* dpg;
    const float* g1;
    float* dg2;
    int64_t n_i2;
    GradOut go;
};

template <int N1, int N2, int R>
__device__ __forceinline__ void dg2_body(const Dg2Args& x, int64_t blk) {
    const TabDev* __restrict__ desc = x.desc;
    const int32_t T = x.T;
    const int32_t* __restrict__ ctrl = x.ctrl;
    const int64_t K = x.K;
    const uint64_t* __restrict__ key_scan = x.key_scan;
    const int32_t* __restrict__ group_key = x.group_key;
    const float* __restrict__ dpg = x.dpg;
    const float* __restrict__ g1 = x.g1;
    float* __restrict__ dg2 = x.dg2;
    const int64_t n_i2 = x.n_i2;
    const GradOut go = x.go;
    constexpr int N2R = N2 * R, PR = N1 * N2R, RT = R / 16, CT = N2R / 16, UNR = 8;
    static_assert(16 % N1 == 0 && R % 16 == 0 && N2R % 16 == 0, "shape");
    const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4;
    // wave-uniform task: the group loop is scalar control flow (no exec-mask
    // loop, whose head waits for every load in flight)
    const int64_t task = blk * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (task >= n_i2 * CT) return;
    const int32_t bi = (int32_t)(task / CT);
    const int ct = (int)(task % CT);
    int t = 0;
    {
        int lo = 0, hi = T;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (desc[mid].i2_base <= bi) lo = mid; else hi = mid;
        }
        t = lo;
    }
    const TabDev d = desc[t];
    const int32_t i2 = bi - d.i2_base;
    const int64_t kb = (int64_t)d.key_base + (int64_t)i2 * d.m1;
    const int32_t U = ctrl[CTRL_NUM_GROUPS];
    const int32_t g0 = (int32_t)(key_scan[kb] >> 32);
    const int32_t ge = kb + d.m1 < K ? (int32_t)(key_scan[kb + d.m1] >> 32) : U;
    if (go.sgd && g0 >= ge) return;   // an untouched G2 slice keeps its values
    const float* G1c = g1 + d.o1 + col;          // + i1*N1*R + j1*R + 16*rt: G1[i1][j1][r1]
    const float* dPc = dpg + 16 * ct + col;      // + g*PR + j1*N2R: dP_g[j1][c]
    // two accumulator sets (even and odd steps) keep two independent product
    // chains per r1 tile in flight
    doublex4 acc[2][RT];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[x][rt] = doublex4{0.0, 0.0, 0.0, 0.0};
    for (int32_t gb = g0; gb < ge; gb += 64) {
        const int32_t i1l = group_key[min(gb + lane, ge - 1)] - (int32_t)kb;   // lane j: i1 of group gb + j
        const int n = min(64, ge - gb);
        const int ns = (n * N1 + 3) / 4;   // steps: lane q of step st takes pair 4st + q
        float av[2][UNR][RT], bv[2][UNR];
        auto load = [&](int j0, float (&a)[UNR][RT], float (&b)[UNR]) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const unsigned st = (unsigned)min(j0 + u, ns - 1);
                int gl, j1, i1;
                bool ok = true;
                if constexpr (N1 >= 4) {   // the lanes of a step share its group: wave-uniform
                    gl = (int)((4u * st) / N1);
                    j1 = (int)((4u * st) % N1) + q;
                    i1 = __builtin_amdgcn_readlane(i1l, gl);
                } else {
                    const unsigned f = 4u * st + (unsigned)q;
                    ok = (int)(f / N1) < n;   // a pair past the last group adds zero
                    gl = min((int)(f / N1), n - 1);
                    j1 = (int)(f % N1);
                    i1 = __shfl(i1l, gl);
                }
                const float* ga = G1c + (int64_t)i1 * N1 * R + j1 * R;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) a[u][rt] = ga[16 * rt];
                const float x = dPc[(int64_t)(gb + gl) * PR + j1 * N2R];
                b[u] = ok ? x : 0.f;
            }
        };
        auto math = [&](int j0, const float (&a)[UNR][RT], const float (&b)[UNR]) {
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                if (j0 + u < ns) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[u & 1][rt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[u][rt], (double)b[u],
                                                                             acc[u & 1][rt], 0, 0, 0);
                }
        };
        load(0, av[0], bv[0]);
        for (int j0 = 0;; j0 += 2 * UNR) {
            load(min(j0 + UNR, ns - 1), av[1], bv[1]);
            math(j0, av[0], bv[0]);
            if (j0 + UNR >= ns) break;
            load(min(j0 + 2 * UNR, ns - 1), av[0], bv[0]);
            math(j0 + UNR, av[1], bv[1]);
            if (j0 + 2 * UNR >= ns) break;
        }
    }
    // the fp64 product's lane (col, q) holds rows r1 = 16rt + q + 4v, column c = 16ct + col
    float* D2 = dg2 + d.o2 + (int64_t)i2 * R * N2R + 16 * ct + col;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            put_grad(D2 + (int64_t)(16 * rt + q + 4 * v) * N2R, (float)(acc[0][rt][v] + acc[1][rt][v]), go);
}

// dG1[i1] += dP_g G2[i2]^T, one wave per prefix batch (up to 8 groups of one
// slice: n1/2 row tiles of 16 (group, j1) rows), every r1 tile: rows (group,
// j1), K = the n2*R columns, taken 16 at a time as 16-byte loads per lane (dP
// once, G2 once per r1 tile for all row tiles) feeding four fp64
// matrix-core steps per row and r1 tile. A group's sum over K is complete in
// the wave, so each dG1 element takes one fp64 atomic per group (groups of
// every slice add to the same i1). A wave per half batch read the 32 KB G2
// slice twice per batch, and that L2 traffic set its time.
// Waves take the batch slots in slice-major order (the planner's place map),
// so waves that run together work on different i1 rows of dG1 rather than
// piling atomics on the same ones.
struct Dg1Args {
    const BatchRec* recs;
    int64_t cap;
    const int32_t* ctrl;
    const int32_t* place;
    const float* dpg;
    const float* g2;
    double* dg1;
};

template <int N1, int N2, int R>
__device__ __forceinline__ void dg1_body(const Dg1Args& x, int64_t blk) {
    const BatchRec* __restrict__ recs = x.recs;
    const int64_t cap = x.cap;
    const int32_t* __restrict__ ctrl = x.ctrl;
    const int32_t* __restrict__ place = x.place;
    const float* __restrict__ dpg = x.dpg;
    const float* __restrict__ g2 = x.g2;
    double* __restrict__ dg1 = x.dg1;
    constexpr int N2R = N2 * R, PR = N1 * N2R, RT = R / 16, KS = N2R / 16, UNR = 2, MT = kFwdBatch * N1 / 16;
    static_assert(16 % N1 == 0 && MT >= 1 && R % 16 == 0 && N2R % 16 == 0 && KS % (2 * UNR) == 0, "shape");
    const int lane = threadIdx.x & 63, col = lane & 15, q = lane >> 4;
    const int64_t k = blk * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (k >= cap) return;
    const int32_t pos = place[k];
    const int64_t nl = ctrl[CTRL_NUM_BATCHES];
    if (pos < 0 || pos >= nl) return;
    const int64_t b = pos;
    const int32_t rw = rec_word(recs, b, cap, nl);
    const int ng = rec_field(rw, RW_NG);
    if (ng <= 0) return;
    const int32_t g0 = rec_field(rw, RW_G0);
    // A row i of row tile mt = (group, j1) of row 16mt + i: lane (col, q) reads row col
    const floatx4* A[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int rho = 16 * mt + col;
        A[mt] = reinterpret_cast<const floatx4*>(dpg + (int64_t)(g0 + min(rho / N1, ng - 1)) * PR +
                                                 (rho % N1) * N2R) + q;
    }
    const floatx4* Bm = reinterpret_cast<const floatx4*>(g2 + rec_field64(rw, RW_O2) +
                                                          (int64_t)rec_field(rw, RW_I2) * R * N2R +
                                                          (int64_t)col * N2R) + q;   // + 16*rt rows
    doublex4 acc[MT][RT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = doublex4{0.0, 0.0, 0.0, 0.0};
    floatx4 a4[2][UNR][MT], b4[2][UNR][RT];
    auto load = [&](int s0, floatx4 (&a)[UNR][MT], floatx4 (&bb)[UNR][RT]) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[u][mt] = A[mt][4 * (s0 + u)];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) bb[u][rt] = Bm[(16 * rt) * (N2R / 4) + 4 * (s0 + u)];
        }
    };
    auto math = [&](const floatx4 (&a)[UNR][MT], const floatx4 (&bb)[UNR][RT]) {
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[mt][rt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[u][mt][e], (double)bb[u][rt][e],
                                                                          acc[mt][rt], 0, 0, 0);
    };
    load(0, a4[0], b4[0]);
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += 2 * UNR) {
        load(s0 + UNR, a4[1], b4[1]);
        math(a4[0], b4[0]);
        if (s0 + 2 * UNR < KS) load(s0 + 2 * UNR, a4[0], b4[0]);
        math(a4[1], b4[1]);
    }
    // the fp64 product's lane (col, q) holds rows q + 4v of tile mt, that is
    // (group, j1) of row 16mt + q + 4v, column r1 = 16rt + col
    double* D1 = dg1 + rec_field64(rw, RW_O1) + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rho = 16 * mt + q + 4 * v, gi = rho / N1, j1 = rho % N1;
            int32_t i1;
            if constexpr (N1 >= 4) {   // gi = (16mt + 4v) / N1: wave-uniform
                if ((16 * mt + 4 * v) / N1 >= ng) continue;
                i1 = __builtin_amdgcn_readlane(rw, RW_I1 + (16 * mt + 4 * v) / N1);
            } else {
                i1 = __shfl(rw, RW_I1 + min(gi, kFwdBatch - 1));
                if (gi >= ng) continue;
            }
            double* dst = D1 + (int64_t)i1 * N1 * R + j1 * R;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) atomicAdd(dst + 16 * rt, acc[mt][rt][v]);
        }
}

// dG3, dG1 and dG2 in one launch: workgroups below nb3 reduce one G3 row's
// c3 rows each, the next nb1 take dG1's batch slots, the rest dG2's (slice,
// column tile) tasks. None reads what another writes (with the fused SGD,
// dG2 goes to a buffer of its own that k_bwd_finish applies, as G2 is read
// for dG1; G3, updated here, is read by none of them). The dG1 and dG2 waves
// run chains of loads and fp64 matrix-core steps, the dG3 waves stream c3
// rows: together they keep more waves on each SIMD than any one of them.
template <int N1, int N2, int R, int CN>
__global__ __launch_bounds__(256, 5) void k_bwd_dg123(Dg3Args a3, Dg1Args a1, Dg2Args a2, int64_t nb3, int64_t nb1) {
    __shared__ double red[4][CN];
    const int64_t blk = blockIdx.x;
    if (blk < nb3) dg3_body<CN, 4>(a3, (int32_t)blk, red);
    else if (blk < nb3 + nb1) dg1_body<N1, N2, R>(a1, blk - nb3);
    else dg2_body<N1, N2, R>(a2, blk - nb3 - nb1);
}

// Fused SGD (go.sgd): dg1/dg2/dg3 are the cores g1/g2/g3 themselves. Every
// kernel reads the cores it needs before any kernel updates them: the run
// kernel (G3) precedes k_bwd_dg123, which updates G3, reads G1 and G2 and
// writes dG2 to a buffer; k_bwd_finish then updates G1 and G2.
template <int N1, int N2, int R, int N3>
static tt_status launch_bwd_mfma(const tt_emb_plan_s* p, const float* g1, const float* g2,
                                 const float* g3, const float* gout, float* dg1, float* dg2,
                                 float* dg3, bool kept, GradOut go, hipStream_t s, float* hot) {
    // dG3 reduced per G3 row from per-run terms (k_bwd_dg123 writes every row
    // of the buffer, gaps included), unless some table's G3 rows are not
    // aligned to R*n3: then device atomics into an fp64 accumulator
    const bool bucket3 = p->nb3 > 0 && p->L > 0;
    // dG2's destination: the gradient, or, with the fused SGD, a buffer that
    // k_bwd_finish applies to G2 (k_bwd_dg123 reads G2 for dG1 meanwhile)
    float* d2 = go.sgd ? p->at<float>(p->lay.acc2) : dg2;
    if (!p->packed) {
        // elements outside every table's slices are zero in the gradients
        tt_status st = fill32(p, d2, 0u, p->extent[1], s);
        if (st != TT_OK) return st;
    }
    constexpr int DL = N1 * N2 * N3 / 64, D = N1 * N2 * N3, CN = R * N3;
    double* acc1 = p->at<double>(p->lay.acc1);
    double* acc3 = p->at<double>(p->lay.acc3);
    double* xpart = p->at<double>(p->lay.xsum);
    float* S = p->at<float>(p->lay.stage);
    float* pbuf = p->at<float>(p->lay.pbuf);
    // each run's dG3 term over its own S row when the row holds it
    float* c3 = CN <= D ? S : p->at<float>(p->lay.c3);
    const int64_t c3s = CN <= D ? D : CN;
    const CrossRef xr{p->at<int32_t>(p->lay.skey), p->at<int32_t>(p->lay.rid),
                      p->at<int32_t>(p->lay.run_start), p->L};
    const int64_t nwin = (p->L + kWin - 1) / kWin;
    // set-up (first kPrepBlocks workgroups) and the grad-row sums in one launch
    const PrepArgs pa{acc1, p->extent[0], acc3, bucket3 ? 0 : p->extent[2], p->at<int32_t>(p->lay.xcnt), nwin,
                      p->at<int32_t>(p->lay.claims),
                      p->at<int32_t>(p->lay.i3cnt), bucket3 ? p->nb3 : 0, p->at<int32_t>(p->lay.i3start),
                      p->at<int32_t>(p->lay.group_rbase), p->at<int32_t>(p->lay.xpiece), p->lay.xcap,
                      p->at<int32_t>(p->lay.gdone), p->ctrl()};
    static_assert(kPrepBlocks * 256 >= kRunCounters, "prep zeroes the counters");
    const SumArgs sa{p->at<int32_t>(p->lay.sorted_bag), p->at<int32_t>(p->lay.skey), p->at<int32_t>(p->lay.rid),
                     p->at<int32_t>(p->lay.run_start), p->L, gout, S, xpart};
    // hot rows: dW starts at zero (every row written, also with no lookups);
    // the fused step updates W in place
    if (p->cached && !go.sgd && p->n_hot > 0) {
        tt_status st = fill32(p, hot, 0u, p->n_hot * (int64_t)D, s);
        if (st != TT_OK) return st;
    }
    TT_LAUNCH(p, "k_bwd_sum", s, k_bwd_sum<DL>, dim3(kPrepBlocks + (p->L > 0 ? persistent_grid(4) : 0u)), dim3(256), 0, s,
                       sa, pa);
    TT_LAUNCH_CHECK();
    if (p->L > 0) {
        // cut-run sums (nspan workgroups) and, with buckets, the bucket lists
        const int64_t nspan = std::min<int64_t>(std::max<int64_t>((nwin + 15) / 16, 1), 1024);
        const SlotArgs sl{p->at<int32_t>(p->lay.i3start), p->at<int32_t>(p->lay.run_bkt),
                          p->at<int32_t>(p->lay.run_rank), p->at<int32_t>(p->lay.bucket_runs)};
        const int64_t nslot = bucket3 ? (p->L + 1023) / 1024 : 0;
        TT_LAUNCH(p, "k_bwd_cross", s, k_bwd_cross<DL>, dim3((unsigned)(nspan + nslot)), dim3(1024), 0, s, xpart,
                           p->at<int32_t>(p->lay.xcnt), xr, S, p->ctrl(), nspan, sl);
        TT_LAUNCH_CHECK();
        if (!kept) {
            const size_t lds = sizeof(int32_t) * (size_t)kFwdBatch * (size_t)p->M3;
            const int64_t grid = batch_grid(p->n_fb, kFwdPersistBlocks);
            TT_LAUNCH(p, "k_bwd_pfx", s, (k_bwd_pfx<N1, N2, R>), dim3((unsigned)grid), dim3(64 * PrefixBatch<N1, N2, R>::WAVES), lds, s,
                               p->at<BatchRec>(p->lay.batch), p->n_fb, p->ctrl(), p->at<int32_t>(p->lay.run_i3), g1, g2, pbuf);
            TT_LAUNCH_CHECK();
        }
        RunsArgs ra{p->desc(), p->T, p->ctrl(), p->at<int32_t>(p->lay.xpiece), p->lay.xcap,
                    p->at<int32_t>(p->lay.group_rbase), p->at<int32_t>(p->lay.group_key),
                    p->at<int32_t>(p->lay.run_i3), S, pbuf, g3, acc3, p->at<double>(p->lay.dpart),
                    p->at<int32_t>(p->lay.gdone), p->at<int32_t>(p->lay.claims),
                    p->cached ? p->at<int32_t>(p->lay.run_cslot) : nullptr, hot, go,
                    p->at<int32_t>(p->lay.run_bag1), gout};
        if (bucket3) {
            TT_LAUNCH(p, "k_bwd_runs_c3", s, (k_bwd_runs_c3<N1, N2, R, N3>), dim3(persistent_grid(3)), dim3(256), 0, s, ra, c3,
                               c3s);
            TT_LAUNCH_CHECK();
        } else {
            TT_LAUNCH(p, "k_bwd_runs", s, (k_bwd_runs<N1, N2, R, N3>), dim3(persistent_grid(4)), dim3(256), 0, s, ra);
        }
        TT_LAUNCH_CHECK();
    }
    {
        // dP of every group now sits over its P, each run's c3 row over its
        // S: dG3, dG1 and dG2 in one launch
        const int64_t nb3 = bucket3 ? p->nb3 : 0;
        const int64_t nb1 = (p->n_fb + 3) / 4;
        const int64_t nb2 = (p->n_i2 * (N2 * R / 16) + 3) / 4;
        const Dg3Args a3{p->at<int32_t>(p->lay.i3start), p->at<int32_t>(p->lay.bucket_runs), c3, c3s, dg3, go};
        const Dg1Args a1{p->at<BatchRec>(p->lay.batch), p->n_fb, p->ctrl(), p->at<int32_t>(p->lay.batch_place),
                         pbuf, g2, acc1};
        const Dg2Args a2{p->desc(), p->T, p->ctrl(), p->K, p->at<uint64_t>(p->lay.key_scan),
                         p->at<int32_t>(p->lay.group_key), pbuf, g1, d2, p->n_i2, GradOut{0.f, 0}};
        if (nb3 + nb1 + nb2 > 0) {
            TT_LAUNCH(p, "k_bwd_dg123", s, (k_bwd_dg123<N1, N2, R, CN>), dim3((unsigned)(nb3 + nb1 + nb2)), dim3(256), 0,
                      s, a3, a1, a2, nb3, nb1);
            TT_LAUNCH_CHECK();
        }
    }
    TT_LAUNCH(p, "k_bwd_finish", s, k_bwd_finish, dim3(go.sgd ? 1024 : 256), dim3(256), 0, s, acc1, dg1, p->extent[0],
              acc3, dg3, bucket3 ? 0 : p->extent[2], p->ctrl(), go, d2, dg2, go.sgd ? p->extent[1] : 0);
    TT_LAUNCH_CHECK();
    return TT_OK;
}

// The plan's shape and the cores' alignment admit the matrix-core backward.
bool bwd_mfma_ok(const tt_emb_plan_s* p, const float* g1, const float* g2) {
    // the prologue reads G1 rows and the G2 slice as 16-byte vectors
    if (!p->uniform || !p->off4 || ((uintptr_t)g1 & 15) != 0 || ((uintptr_t)g2 & 15) != 0) return false;
    // dG2 is stored once per table slice: tables sharing G2 take the
    // general path, which adds every table's terms
    if (p->g2_overlap) return false;
    // the batch's run i3 list is staged in LDS
    if ((int64_t)sizeof(int32_t) * kFwdBatch * p->M3 > kMaxBatchI3Bytes) return false;
    return mfma_shape(p->n1, p->n2, p->n3, p->R, true);
}

// One entry of the shape list: launches the backward when the plan has this
// shape (instantiated only for the shapes the backward's kernels serve).
template <int N1, int N2, int R, int N3, bool BW>
static bool bwd_case(const tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3,
                     const float* gout, float* dg1, float* dg2, float* dg3, bool kept, GradOut go,
                     hipStream_t s, tt_status* st, float* hot) {
    if constexpr (BW) {
        if (p->n1 == N1 && p->n2 == N2 && p->n3 == N3 && p->R == R) {
            *st = launch_bwd_mfma<N1, N2, R, N3>(p, g1, g2, g3, gout, dg1, dg2, dg3, kept, go, s, hot);
            return true;
        }
    }
    return false;
}

static tt_status launch_bwd(const tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3,
                            const float* gout, float* dg1, float* dg2, float* dg3, bool kept, GradOut go,
                            hipStream_t s, float* hot = nullptr) {
    tt_status st = TT_ERR_UNSUPPORTED;
#define TT_BWD_CASE(a, b, c, d, bw) \
    if (bwd_case<a, b, d, c, bw>(p, g1, g2, g3, gout, dg1, dg2, dg3, kept, go, s, &st, hot)) return st;
    TT_MFMA_SHAPES(TT_BWD_CASE)
#undef TT_BWD_CASE
    return st;
}

}  // namespace tt

using namespace tt;

static tt_status backward_impl(tt_emb_plan_t p, const float* g1, const float* g2, const float* g3,
                               const float* grad_out, float* dg1, float* dg2, float* dg3, bool kept,
                               void* stream, float* hot_dw = nullptr) {
    hipStream_t s = (hipStream_t)stream;
    // the backward overwrites the kept products (P, then dP over it)
    p->kept_token = 0;
    if (bwd_mfma_ok(p, g1, g2))
        return launch_bwd(p, g1, g2, g3, grad_out, dg1, dg2, dg3, kept, GradOut{0.f, 0}, s, hot_dw);
    if (p->cached) return TT_ERR_UNSUPPORTED;   // hot rows need the matrix-core kernels
    // generic kernels: every core's gradient summed in fp64 accumulators
    // (cleared here), then rounded into the caller's buffers
    double* a1 = p->at<double>(p->lay.acc1);
    double* a2 = p->at<double>(p->lay.acc2);
    double* a3 = p->at<double>(p->lay.acc3);
    tt_status st = TT_OK;
    if ((st = fill32(p, a1, 0u, 2 * p->extent[0], s)) != TT_OK) return st;
    if ((st = fill32(p, a2, 0u, 2 * p->extent[1], s)) != TT_OK) return st;
    if ((st = fill32(p, a3, 0u, 2 * p->extent[2], s)) != TT_OK) return st;
    if (p->lay.Cmax > 0) {
        int maxp = 0;
        for (int32_t t = 0; t < p->T; ++t)
            maxp = std::max(maxp, p->tables[t].n[0] * p->tables[t].n[1] * p->tables[t].rank);
        const size_t lds = (sizeof(double) + sizeof(float)) * (size_t)maxp;
        TT_LAUNCH(p, "k_bwd_generic", s, k_bwd_generic, dim3((unsigned)p->lay.Cmax), dim3(256), lds, s, p->desc(),
                  p->T, p->ctrl(), p->at<int32_t>(p->lay.group_key), p->at<int32_t>(p->lay.chunk_group),
                  p->at<int32_t>(p->lay.chunk_begin), p->at<int32_t>(p->lay.chunk_end),
                  p->at<int32_t>(p->lay.sorted_i3), p->at<int32_t>(p->lay.sorted_bag), g1, g2, g3, grad_out, a1,
                  a2, a3, p->D);
        TT_LAUNCH_CHECK();
    }
    const GradOut go{0.f, 0};
    TT_LAUNCH(p, "k_bwd_finish", s, k_bwd_finish, dim3(256), dim3(256), 0, s, a1, dg1, p->extent[0], a3, dg3,
              p->extent[2], p->ctrl(), go, nullptr, nullptr, (int64_t)0);
    TT_LAUNCH_CHECK();
    TT_LAUNCH(p, "k_bwd_finish", s, k_bwd_finish, dim3(256), dim3(256), 0, s, a2, dg2, p->extent[1], a3, dg3,
              (int64_t)0, p->ctrl(), go, nullptr, nullptr, (int64_t)0);
    TT_LAUNCH_CHECK();
    return TT_OK;
}

static bool backward_args_ok(tt_emb_plan_t p, const float* g1, const float* g2, const float* g3,
                             const float* grad_out, const float* dg1, const float* dg2, const float* dg3) {
    return p && g1 && g2 && g3 && dg1 && dg2 && dg3 && (grad_out || p->TB == 0);
}

// A kept token names the products the plan holds for these G1 and G2.
static bool token_ok(tt_emb_plan_t p, uint64_t tok, const float* g1, const float* g2) {
    return tok != 0 && tok == p->kept_token && g1 == p->kept_g1 && g2 == p->kept_g2;
}

extern "C" tt_status tt_emb_backward(tt_emb_plan_t p, const float* g1, const float* g2,
                                     const float* g3, const float* grad_out, float* dg1,
                                     float* dg2, float* dg3, void* stream) {
    if (!backward_args_ok(p, g1, g2, g3, grad_out, dg1, dg2, dg3)) return TT_ERR_INVALID_ARG;
    if (p->cached) return TT_ERR_CACHE;
    return backward_impl(p, g1, g2, g3, grad_out, dg1, dg2, dg3, false, stream);
}

extern "C" tt_status tt_emb_backward_kept(tt_emb_plan_t p, uint64_t kept_token, const float* g1,
                                          const float* g2, const float* g3, const float* grad_out,
                                          float* dg1, float* dg2, float* dg3, void* stream) {
    if (!backward_args_ok(p, g1, g2, g3, grad_out, dg1, dg2, dg3)) return TT_ERR_INVALID_ARG;
    if (p->cached) return TT_ERR_CACHE;
    if (!token_ok(p, kept_token, g1, g2) || !bwd_mfma_ok(p, g1, g2)) return TT_ERR_STALE;
    return backward_impl(p, g1, g2, g3, grad_out, dg1, dg2, dg3, true, stream);
}

extern "C" tt_status tt_emb_backward_cached(tt_emb_plan_t p, uint64_t kept_token, const float* g1,
                                            const float* g2, const float* g3, const float* grad_out,
                                            float* dg1, float* dg2, float* dg3, float* hot_dw, void* stream) {
    if (!backward_args_ok(p, g1, g2, g3, grad_out, dg1, dg2, dg3)) return TT_ERR_INVALID_ARG;
    if (!p->cached) return TT_ERR_CACHE;
    if (!hot_dw && p->n_hot > 0) return TT_ERR_INVALID_ARG;
    if (!bwd_mfma_ok(p, g1, g2)) return TT_ERR_UNSUPPORTED;
    if (kept_token != 0 && !token_ok(p, kept_token, g1, g2)) return TT_ERR_STALE;
    return backward_impl(p, g1, g2, g3, grad_out, dg1, dg2, dg3, kept_token != 0, stream, hot_dw);
}

static tt_status backward_sgd(tt_emb_plan_t p, uint64_t kept_token, float* g1, float* g2, float* g3,
                              float* hot_w, const float* grad_out, float lr, void* stream) {
    if (!p || !g1 || !g2 || !g3 || (!grad_out && p->TB > 0)) return TT_ERR_INVALID_ARG;
    if (!bwd_mfma_ok(p, g1, g2)) return TT_ERR_UNSUPPORTED;
    if (kept_token != 0 && !token_ok(p, kept_token, g1, g2)) return TT_ERR_STALE;
    const bool kept = kept_token != 0;
    p->kept_token = 0;   // consumed, and the cores change
    return launch_bwd(p, g1, g2, g3, grad_out, g1, g2, g3, kept, GradOut{-lr, 1}, (hipStream_t)stream, hot_w);
}

extern "C" tt_status tt_emb_backward_sgd(tt_emb_plan_t p, uint64_t kept_token, float* g1, float* g2,
                                         float* g3, const float* grad_out, float lr, void* stream) {
    if (p && p->cached) return TT_ERR_CACHE;
    return backward_sgd(p, kept_token, g1, g2, g3, nullptr, grad_out, lr, stream);
}

extern "C" tt_status tt_emb_backward_sgd_cached(tt_emb_plan_t p, uint64_t kept_token, float* g1, float* g2,
                                                float* g3, float* hot_w, const float* grad_out, float lr,
                                                void* stream) {
    if (p && !p->cached) return TT_ERR_CACHE;
    if (p && !hot_w && p->n_hot > 0) return TT_ERR_INVALID_ARG;
    return backward_sgd(p, kept_token, g1, g2, g3, hot_w, grad_out, lr, stream);
}

extern "C" tt_status tt_emb_sgd(tt_emb_plan_t p, float* g1, float* g2, float* g3,
                                const float* dg1, const float* dg2, const float* dg3, float lr,
                                void* stream) {
    if (!p || !g1 || !g2 || !g3 || !dg1 || !dg2 || !dg3) return TT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    p->kept_token = 0;   // the cores change: kept products no longer match them
    const SgdArgs a{{g1, g2, g3}, {dg1, dg2, dg3}, {p->extent[0], p->extent[1], p->extent[2]}};
    const int64_t nmax = std::max(p->extent[0], std::max(p->extent[1], p->extent[2]));
    if (nmax <= 0) return TT_OK;
    TT_LAUNCH(p, "k_sgd", s, k_sgd, dim3(std::min<unsigned>(grid_for(nmax / 4 + 1, 256), 2048u)), dim3(256), 0, s, a, lr);
    TT_LAUNCH_CHECK();
    return TT_OK;
}
