/*
 * CPU oracle for the sum-pooled Tensor-Train embedding gather (TT-EmbeddingBag).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header, table or constant with the HIP
 * library.
 *
 * What it computes follows the pages' description of the TT lookup: a row of
 * the table is replaced by a chain of contractions over three TT cores
 * ("FlowTT: Exploiting Computation Flow Reuse in Irregular Tensor-Train
 * Embedding", summary card, problem statement; "Georgia Tech & Facebook Tensor
 * Train Approach Achieves 112x Size Reduction", method paragraph: embedding
 * vectors become a TT-core multiplication), pooled by sum per bag (the
 * "TT-EmbeddingBag" of the TT-Rec abstract). The pages give no formula; the
 * index split, core layout, output flattening and gradient conventions used
 * here are the readings listed in the repository's design notes:
 *
 *   idx = (i1*m2 + i2)*m3 + i3                       (i1 most significant)
 *   G1[i1][j1][r1], G2[i2][r1][j2][r2], G3[i3][r2][j3]  (row-major, fp32 in)
 *   E(idx)[(j1*n2 + j2)*n3 + j3] = sum_{r1,r2} G1[i1][j1][r1] G2[i2][r1][j2][r2] G3[i3][r2][j3]
 *   out[q] = sum over lookups l of bag q of E(idx_l); empty bag -> 0
 *
 * Backward: with the loss <grad_out, out>, the gradient of each core slice is
 * the sum over the lookups that use that slice of the product of grad_out's row
 * with the two other cores (plain multilinear calculus on the formula above).
 *
 * Arithmetic: every product and sum in double precision, one lookup at a time,
 * with no reuse across lookups (no prefix grouping: that is what the GPU path
 * does and what this oracle is meant to check). OpenMP splits work so that
 * every output element is summed by exactly one thread in increasing lookup
 * order; results do not depend on the thread count.
 *
 * Parity pins (see tests): brute-force materialisation of the full table by a
 * different contraction order, the rank-1 Kronecker closed form, gauge
 * invariance, and the exact adjoint identity for the backward pass.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TTO_OK 0
#define TTO_BAD_ARG (-1)
#define TTO_BAD_INDEX (-2)
#define TTO_BAD_OFFSETS (-3)
#define TTO_NO_MEMORY (-4)

/* Per-table description handed in as plain int64 columns. */
typedef struct {
    int64_t N, m1, m2, m3, n1, n2, n3, R, o1, o2, o3;
} tto_tab;

static int load_tables(int32_t T, const int64_t* num_rows, const int64_t* m,
                       const int64_t* n, const int64_t* rank, const int64_t* goff,
                       tto_tab* tabs, int64_t* D_out) {
    int64_t D = -1;
    for (int32_t t = 0; t < T; ++t) {
        tto_tab* x = &tabs[t];
        x->N = num_rows[t];
        x->m1 = m[3 * t]; x->m2 = m[3 * t + 1]; x->m3 = m[3 * t + 2];
        x->n1 = n[3 * t]; x->n2 = n[3 * t + 1]; x->n3 = n[3 * t + 2];
        x->R = rank[t];
        x->o1 = goff[3 * t]; x->o2 = goff[3 * t + 1]; x->o3 = goff[3 * t + 2];
        if (x->N < 1 || x->m1 < 1 || x->m2 < 1 || x->m3 < 1 || x->n1 < 1 || x->n2 < 1 ||
            x->n3 < 1 || x->R < 1)
            return TTO_BAD_ARG;
        if (x->m1 * x->m2 * x->m3 < x->N) return TTO_BAD_ARG;
        int64_t d = x->n1 * x->n2 * x->n3;
        if (D >= 0 && d != D) return TTO_BAD_ARG;
        D = d;
    }
    *D_out = D;
    return TTO_OK;
}

static int check_offsets(const int64_t* offsets, int64_t nbag_total, int64_t L) {
    if (offsets[0] != 0 || offsets[nbag_total] != L) return TTO_BAD_OFFSETS;
    for (int64_t q = 0; q < nbag_total; ++q)
        if (offsets[q + 1] < offsets[q]) return TTO_BAD_OFFSETS;
    return TTO_OK;
}

/* E(idx) of one table row, accumulated (added) into acc[D] in double.
 * The chain is taken left to right, one lookup at a time: first the row of
 * G1[i1] times G2[i2] (a length-R vector per (j1,j2)), then that vector times
 * G3[i3]. No intermediate is kept from one lookup to the next. */
static void add_row(const tto_tab* x, const float* g1, const float* g2, const float* g3,
                    int64_t idx, double* acc) {
    const int64_t i3 = idx % x->m3;
    const int64_t i2 = (idx / x->m3) % x->m2;
    const int64_t i1 = idx / (x->m2 * x->m3);
    const int64_t n1 = x->n1, n2 = x->n2, n3 = x->n3, R = x->R;
    const float* a = g1 + x->o1 + i1 * n1 * R;            /* [n1][R]      */
    const float* b = g2 + x->o2 + i2 * R * n2 * R;        /* [R][n2][R]   */
    const float* c = g3 + x->o3 + i3 * R * n3;            /* [R][n3]      */
    double* v = (double*)malloc(sizeof(double) * (size_t)R);
    for (int64_t j1 = 0; j1 < n1; ++j1)
        for (int64_t j2 = 0; j2 < n2; ++j2) {
            for (int64_t r2 = 0; r2 < R; ++r2) {
                double s = 0.0;
                for (int64_t r1 = 0; r1 < R; ++r1)
                    s += (double)a[j1 * R + r1] * (double)b[(r1 * n2 + j2) * R + r2];
                v[r2] = s;
            }
            for (int64_t j3 = 0; j3 < n3; ++j3) {
                double s = 0.0;
                for (int64_t r2 = 0; r2 < R; ++r2) s += v[r2] * (double)c[r2 * n3 + j3];
                acc[(j1 * n2 + j2) * n3 + j3] += s;
            }
        }
    free(v);
}

/*
 * Forward: pooled output for the listed bags (bags == NULL: every bag
 * 0..T*B-1 in order). out is [nbags][D] doubles, overwritten.
 * Returns TTO_BAD_INDEX if any index of a listed bag is outside [0, N_t).
 */
int tto_forward(int32_t T, const int64_t* num_rows, const int64_t* m, const int64_t* n,
                const int64_t* rank, const int64_t* goff, const float* g1, const float* g2,
                const float* g3, const int64_t* indices, const int64_t* offsets, int64_t L,
                int64_t B, const int64_t* bags, int64_t nbags, double* out) {
    if (T < 1 || B < 0 || L < 0 || !offsets) return TTO_BAD_ARG;
    tto_tab* tabs = (tto_tab*)calloc((size_t)T, sizeof(tto_tab));
    if (!tabs) return TTO_NO_MEMORY;
    int64_t D = 0;
    int rc = load_tables(T, num_rows, m, n, rank, goff, tabs, &D);
    if (rc == TTO_OK) rc = check_offsets(offsets, (int64_t)T * B, L);
    if (rc != TTO_OK) { free(tabs); return rc; }
    const int64_t nb = bags ? nbags : (int64_t)T * B;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t k = 0; k < nb; ++k) {
        const int64_t q = bags ? bags[k] : k;
        double* acc = out + k * D;
        for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
        if (q < 0 || q >= (int64_t)T * B) { bad |= 1; continue; }
        const tto_tab* x = &tabs[q / B];
        for (int64_t l = offsets[q]; l < offsets[q + 1]; ++l) {
            const int64_t idx = indices[l];
            if (idx < 0 || idx >= x->N) { bad |= 2; continue; }
            add_row(x, g1, g2, g3, idx, acc);
        }
    }
    free(tabs);
    if (bad & 1) return TTO_BAD_ARG;
    if (bad & 2) return TTO_BAD_INDEX;
    return TTO_OK;
}

/*
 * Backward: dg1/dg2/dg3 (same packing and size as the cores, doubles) are
 * zeroed, then every lookup l with mask[l] != 0 (mask == NULL: every lookup)
 * adds its contribution, with g = grad_out[bag of l] viewed as [n1][n2][n3]:
 *
 *   dG1[i1][j1][r1]     += sum_{j2,j3,r2} g[j1,j2,j3] G2[i2][r1][j2][r2] G3[i3][r2][j3]
 *   dG2[i2][r1][j2][r2] += sum_{j1,j3}    G1[i1][j1][r1] g[j1,j2,j3] G3[i3][r2][j3]
 *   dG3[i3][r2][j3]     += sum_{j1,j2,r1} G1[i1][j1][r1] G2[i2][r1][j2][r2] g[j1,j2,j3]
 *
 * Each core is handled in its own pass that walks slice by slice, visiting that
 * slice's lookups in increasing l for each element (parallel over blocks of a
 * slice's elements, so a slice that most lookups touch is not left to one
 * thread).
 */
typedef struct {
    int64_t t, i1, i2, i3, q;
} tto_lk;

/* The three contributions of one lookup k to elements [e0, e1) of the slice
 * it touches (element numbering: the slice's own row-major order). Each
 * element's term is a plain triple sum, added to the running total. */
static void contrib_dg1(const tto_tab* x, const float* g2, const float* g3, const tto_lk* k,
                        const float* g, double* d1 /* [n1][R] of slice i1 */, int64_t e0,
                        int64_t e1) {
    const int64_t n2 = x->n2, n3 = x->n3, R = x->R;
    const float* b = g2 + x->o2 + k->i2 * R * n2 * R;
    const float* c = g3 + x->o3 + k->i3 * R * n3;
    for (int64_t e = e0; e < e1; ++e) {
        const int64_t j1 = e / R, r1 = e % R;
        double s = 0.0;
        for (int64_t j2 = 0; j2 < n2; ++j2)
            for (int64_t j3 = 0; j3 < n3; ++j3)
                for (int64_t r2 = 0; r2 < R; ++r2)
                    s += (double)g[(j1 * n2 + j2) * n3 + j3] *
                         (double)b[(r1 * n2 + j2) * R + r2] * (double)c[r2 * n3 + j3];
        d1[e] += s;
    }
}

static void contrib_dg2(const tto_tab* x, const float* g1, const float* g3, const tto_lk* k,
                        const float* g, double* d2 /* [R][n2][R] of slice i2 */, int64_t e0,
                        int64_t e1) {
    const int64_t n1 = x->n1, n2 = x->n2, n3 = x->n3, R = x->R;
    const float* a = g1 + x->o1 + k->i1 * n1 * R;
    const float* c = g3 + x->o3 + k->i3 * R * n3;
    for (int64_t e = e0; e < e1; ++e) {
        const int64_t r1 = e / (n2 * R), j2 = (e / R) % n2, r2 = e % R;
        double s = 0.0;
        for (int64_t j1 = 0; j1 < n1; ++j1)
            for (int64_t j3 = 0; j3 < n3; ++j3)
                s += (double)a[j1 * R + r1] * (double)g[(j1 * n2 + j2) * n3 + j3] *
                     (double)c[r2 * n3 + j3];
        d2[e] += s;
    }
}

static void contrib_dg3(const tto_tab* x, const float* g1, const float* g2, const tto_lk* k,
                        const float* g, double* d3 /* [R][n3] of slice i3 */, int64_t e0,
                        int64_t e1) {
    const int64_t n1 = x->n1, n2 = x->n2, n3 = x->n3, R = x->R;
    const float* a = g1 + x->o1 + k->i1 * n1 * R;
    const float* b = g2 + x->o2 + k->i2 * R * n2 * R;
    for (int64_t e = e0; e < e1; ++e) {
        const int64_t r2 = e / n3, j3 = e % n3;
        double s = 0.0;
        for (int64_t j1 = 0; j1 < n1; ++j1)
            for (int64_t j2 = 0; j2 < n2; ++j2)
                for (int64_t r1 = 0; r1 < R; ++r1)
                    s += (double)a[j1 * R + r1] * (double)b[(r1 * n2 + j2) * R + r2] *
                         (double)g[(j1 * n2 + j2) * n3 + j3];
        d3[e] += s;
    }
}

/* 1 when two tables' core `which` (1, 2 or 3) occupy overlapping elements of
 * the packed buffer (tables may share a core); their slices then write the
 * same gradient elements and must not be accumulated concurrently. */
static int cores_overlap(int32_t T, const tto_tab* tabs, int which) {
    for (int32_t a = 0; a < T; ++a)
        for (int32_t b = a + 1; b < T; ++b) {
            const tto_tab* x = &tabs[a];
            const tto_tab* y = &tabs[b];
            const int64_t ox = which == 1 ? x->o1 : which == 2 ? x->o2 : x->o3;
            const int64_t oy = which == 1 ? y->o1 : which == 2 ? y->o2 : y->o3;
            const int64_t sx = which == 1 ? x->m1 * x->n1 * x->R
                               : which == 2 ? x->m2 * x->R * x->n2 * x->R : x->m3 * x->R * x->n3;
            const int64_t sy = which == 1 ? y->m1 * y->n1 * y->R
                               : which == 2 ? y->m2 * y->R * y->n2 * y->R : y->m3 * y->R * y->n3;
            if (ox < oy + sy && oy < ox + sx) return 1;
        }
    return 0;
}

/* Bucket the selected lookups by (table, slice) of core `which` (1, 2 or 3):
 * CSR over the global slice id, lookups in increasing l inside each bucket. */
static int bucket(int32_t T, const tto_tab* tabs, const tto_lk* lk, const unsigned char* sel,
                  int64_t L, int which, int64_t** start_out, int64_t** list_out,
                  int64_t** tbase_out, int64_t* nslices_out) {
    int64_t* tbase = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
    if (!tbase) return TTO_NO_MEMORY;
    tbase[0] = 0;
    for (int32_t t = 0; t < T; ++t) {
        const int64_t ms = which == 1 ? tabs[t].m1 : which == 2 ? tabs[t].m2 : tabs[t].m3;
        tbase[t + 1] = tbase[t] + ms;
    }
    const int64_t S = tbase[T];
    int64_t* start = (int64_t*)calloc((size_t)(S + 1), sizeof(int64_t));
    int64_t* list = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    int64_t* fill = (int64_t*)calloc((size_t)(S + 1), sizeof(int64_t));
    if (!start || !list || !fill) { free(tbase); free(start); free(list); free(fill); return TTO_NO_MEMORY; }
    for (int64_t l = 0; l < L; ++l) {
        if (!sel[l]) continue;
        const int64_t s = tbase[lk[l].t] + (which == 1 ? lk[l].i1 : which == 2 ? lk[l].i2 : lk[l].i3);
        start[s + 1]++;
    }
    for (int64_t s = 0; s < S; ++s) start[s + 1] += start[s];
    for (int64_t l = 0; l < L; ++l) {
        if (!sel[l]) continue;
        const int64_t s = tbase[lk[l].t] + (which == 1 ? lk[l].i1 : which == 2 ? lk[l].i2 : lk[l].i3);
        list[start[s] + fill[s]++] = l;
    }
    free(fill);
    *start_out = start; *list_out = list; *tbase_out = tbase; *nslices_out = S;
    return TTO_OK;
}

int tto_backward(int32_t T, const int64_t* num_rows, const int64_t* m, const int64_t* n,
                 const int64_t* rank, const int64_t* goff, const float* g1, const float* g2,
                 const float* g3, const int64_t* indices, const int64_t* offsets, int64_t L,
                 int64_t B, const float* grad_out, const unsigned char* mask, double* dg1,
                 int64_t size1, double* dg2, int64_t size2, double* dg3, int64_t size3) {
    if (T < 1 || B < 0 || L < 0 || !offsets || !grad_out) return TTO_BAD_ARG;
    tto_tab* tabs = (tto_tab*)calloc((size_t)T, sizeof(tto_tab));
    if (!tabs) return TTO_NO_MEMORY;
    int64_t D = 0;
    int rc = load_tables(T, num_rows, m, n, rank, goff, tabs, &D);
    if (rc == TTO_OK) rc = check_offsets(offsets, (int64_t)T * B, L);
    if (rc != TTO_OK) { free(tabs); return rc; }
    memset(dg1, 0, sizeof(double) * (size_t)size1);
    memset(dg2, 0, sizeof(double) * (size_t)size2);
    memset(dg3, 0, sizeof(double) * (size_t)size3);

    tto_lk* lk = (tto_lk*)malloc(sizeof(tto_lk) * (size_t)(L > 0 ? L : 1));
    unsigned char* sel = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
    if (!lk || !sel) { free(tabs); free(lk); free(sel); return TTO_NO_MEMORY; }
    for (int64_t q = 0; q < (int64_t)T * B; ++q)
        for (int64_t l = offsets[q]; l < offsets[q + 1]; ++l) {
            const tto_tab* x = &tabs[q / B];
            const int64_t idx = indices[l];
            if (idx < 0 || idx >= x->N) { free(tabs); free(lk); free(sel); return TTO_BAD_INDEX; }
            lk[l].t = q / B;
            lk[l].q = q;
            lk[l].i3 = idx % x->m3;
            lk[l].i2 = (idx / x->m3) % x->m2;
            lk[l].i1 = idx / (x->m2 * x->m3);
            sel[l] = mask ? (mask[l] != 0) : 1;
        }

    for (int which = 1; which <= 3 && rc == TTO_OK; ++which) {
        int64_t *start = NULL, *list = NULL, *tbase = NULL, S = 0;
        rc = bucket(T, tabs, lk, sel, L, which, &start, &list, &tbase, &S);
        if (rc != TTO_OK) break;
        /* Work items are (slice, block of kEB elements of the slice): every
         * element is summed by one thread over its slice's lookups in
         * increasing l, so the result does not depend on the thread count.
         * Items run in parallel unless slices of two tables share elements. */
        const int shared = cores_overlap(T, tabs, which);
        const int64_t kEB = 16;
        int64_t* ibase = (int64_t*)malloc(sizeof(int64_t) * (size_t)(S + 1));
        if (!ibase) { free(start); free(list); free(tbase); rc = TTO_NO_MEMORY; break; }
        ibase[0] = 0;
        for (int64_t s = 0, t = 0; s < S; ++s) {
            while (tbase[t + 1] <= s) ++t;
            const tto_tab* x = &tabs[t];
            const int64_t ne = which == 1 ? x->n1 * x->R : which == 2 ? x->R * x->n2 * x->R : x->R * x->n3;
            ibase[s + 1] = ibase[s] + (start[s] == start[s + 1] ? 0 : (ne + kEB - 1) / kEB);
        }
        const int64_t nitems = ibase[S];
#pragma omp parallel for schedule(dynamic, 1) if (!shared)
        for (int64_t it = 0; it < nitems; ++it) {
            int64_t lo = 0, hi = S;   /* the slice s with ibase[s] <= it < ibase[s + 1] */
            while (hi - lo > 1) {
                const int64_t mid = (lo + hi) / 2;
                if (ibase[mid] <= it) lo = mid; else hi = mid;
            }
            const int64_t s = lo;
            int32_t t = 0;
            while (tbase[t + 1] <= s) ++t;
            const tto_tab* x = &tabs[t];
            const int64_t local = s - tbase[t];
            const int64_t ne = which == 1 ? x->n1 * x->R : which == 2 ? x->R * x->n2 * x->R : x->R * x->n3;
            const int64_t e0 = (it - ibase[s]) * kEB, e1 = e0 + kEB < ne ? e0 + kEB : ne;
            for (int64_t p = start[s]; p < start[s + 1]; ++p) {
                const tto_lk* k = &lk[list[p]];
                const float* g = grad_out + k->q * D;
                if (which == 1)
                    contrib_dg1(x, g2, g3, k, g, dg1 + x->o1 + local * x->n1 * x->R, e0, e1);
                else if (which == 2)
                    contrib_dg2(x, g1, g3, k, g, dg2 + x->o2 + local * x->R * x->n2 * x->R, e0, e1);
                else
                    contrib_dg3(x, g1, g2, k, g, dg3 + x->o3 + local * x->R * x->n3, e0, e1);
            }
        }
        free(ibase);
        free(start); free(list); free(tbase);
    }
    free(tabs); free(lk); free(sel);
    return rc;
}

int tto_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
