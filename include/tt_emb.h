/*
 * tt_emb.h — C ABI of the MI355X (gfx950) TT-EmbeddingBag library, libtt_emb.so.
 *
 * The operation: an embedding table of N rows x D columns is stored as three
 * Tensor-Train cores, and a batch of lookups is answered by contracting, for
 * every requested row, the chain of core slices picked by the row's digits,
 * then summing the rows of each bag. The pages describe the lookup as a chain
 * of tensor contractions across TT cores (FlowTT summary card, problem
 * statement), the table as replaced by a sequence of matrix products whose
 * embedding vectors become a TT-core multiplication (the TT-Rec news article,
 * method paragraph), the pooled kernel by its name, TT-EmbeddingBag (TT-Rec
 * abstract), and the fast path as prefix-based grouping of lookups that share
 * high-order core indices, a fused chain that keeps the shared partial product
 * on chip, and persistent threads with chunk-based work stealing (FlowTT
 * abstract; summary card, key innovations). Training through the lookup is
 * part of both pages' evaluations (FlowTT abstract: training latency).
 *
 * Conventions (the pages give no formulas; these are this library's):
 *   row index       idx = (i1*m2 + i2)*m3 + i3, 0 <= idx < N <= m1*m2*m3
 *   cores (fp32)    G1[m1][n1][R], G2[m2][R][n2][R], G3[m3][R][n3], row-major;
 *                   the slices are 1 x n1 x R, R x n2 x R and R x n3 x 1 with
 *                   the unit boundary ranks dropped
 *   row vector      E[(j1*n2 + j2)*n3 + j3] =
 *                       sum_{r1,r2} G1[i1][j1][r1] G2[i2][r1][j2][r2] G3[i3][r2][j3]
 *   bags            CSR: T tables x B bags each, bag q = t*B + b holds lookups
 *                   offsets[q] .. offsets[q+1]-1; out[q] = sum of its rows
 *                   (sum pooling; an empty bag gives a zero row)
 *   gradients       of the loss <grad_out, out> with respect to each core
 *
 * Memory: every device buffer is owned by the caller (cores, indices,
 * offsets, outputs, gradients and the planning workspace). The library
 * allocates no device memory; the plan handle is a small host object.
 * Several tables are served by one call: their cores are packed one after
 * another in three flat buffers (one per core kind), located by g_offset.
 *
 * Streams: every call that takes `stream` enqueues its kernels on that HIP
 * stream (a hipStream_t passed as void*; NULL is the null stream) and returns
 * without waiting, except tt_emb_get_error and tt_emb_plan_counts, which
 * synchronise that stream. Calls on one plan must be ordered: on one stream,
 * or across streams with events. Plans on separate workspaces share no device
 * state, so their calls may run at the same time on different streams: a
 * training loop can build the next batch's plan on a second stream, in a
 * second workspace, while the current batch's forward and backward run
 * (the caller orders every call that reads cores after the update that
 * writes them, and each plan after the last call on its workspace).
 *
 * Errors: every call returns a tt_status. Arguments that can be checked on
 * the host (null pointers, non-positive or inconsistent dims, sizes beyond
 * int32, a workspace that is too small, unsupported shapes) are rejected
 * before any launch. Data errors found on the device (an index outside
 * [0, N_t), offsets that are not non-decreasing from 0 to L) set a flag in
 * the workspace; the results of that plan are then unspecified, and
 * tt_emb_get_error reports the flag.
 */
#ifndef TT_EMB_H
#define TT_EMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TT_OK = 0,
    TT_ERR_INVALID_ARG = -1,  /* null pointer, bad dims, inconsistent sizes          */
    TT_ERR_UNSUPPORTED = -2,  /* valid but outside the library's limits (see below)  */
    TT_ERR_WORKSPACE = -3,    /* workspace smaller than tt_emb_workspace_bytes      */
    TT_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed          */
    TT_ERR_DEVICE_FLAG = -5,  /* returned by tt_emb_get_error when the flag is set   */
    TT_ERR_STALE = -6,        /* tt_emb_backward_kept: the token does not name the   */
                              /* products the plan holds (see below)                 */
    TT_ERR_SCRATCH = -7,      /* tt_emb_forward_scratch: the batch needs more than   */
                              /* the library's static scratch buffer holds           */
    TT_ERR_CACHE = -8         /* a plan with a hot-row cache given to a call without */
                              /* the hot rows, or the reverse (see below)            */
} tt_status;

/* Device error flag bits (tt_emb_get_error). */
#define TT_FLAG_BAD_INDEX 1   /* some index outside [0, N_t)                         */
#define TT_FLAG_BAD_OFFSETS 2 /* offsets[0] != 0, offsets[T*B] != L or a decrease   */
#define TT_FLAG_INTERNAL 4    /* a scan's wait for an earlier tile hit its bound     */

/* Limits of the library: N_t < 2^31, L < 2^31, T*B < 2^31, sum over tables of
 * m1*m2 < 2^30, R <= 64, n1*n2 <= 64, n3 <= 16, D <= 1024, T <= 4096. */

/* One table (host memory). All tables of a call must have the same D. */
typedef struct {
    int64_t num_rows;    /* N: valid indices are [0, N)                              */
    int32_t m[3];        /* row radices (m1, m2, m3), m1*m2*m3 >= N                  */
    int32_t n[3];        /* dim factors (n1, n2, n3), D = n1*n2*n3                   */
    int32_t rank;        /* R, the two internal TT ranks                              */
    int32_t reserved;    /* must be 0                                                 */
    int64_t g_offset[3]; /* element offset of this table's G1, G2, G3 in the packed  */
                         /* core buffers (and in the matching gradient buffers)       */
} tt_emb_table;

typedef struct tt_emb_plan_s* tt_emb_plan_t;  /* opaque, host-side, library-owned */

/* Bytes of device workspace tt_emb_plan needs for these tables, L lookups,
 * B bags per table and chunk size `chunk` (>= 1). Returns 0 when the
 * arguments are invalid or unsupported. Pure host computation. */
size_t tt_emb_workspace_bytes(const tt_emb_table* tables, int32_t T, int64_t L, int64_t B,
                              int32_t chunk);

/* Planning: index split, prefix grouping and chunking, all on the device.
 *   tables    host array of T descriptors (copied; may be freed after return)
 *   indices   device int64[L]
 *   offsets   device int64[T*B + 1]
 *   chunk     maximum lookups per chunk (work unit); groups larger than this
 *             are cut into several chunks
 *   workspace device buffer of at least tt_emb_workspace_bytes(...) bytes,
 *             256-byte aligned; it holds the plan's tables and stays in use
 *             until the plan is destroyed
 * On success *plan_out receives a new handle. The plan keeps pointers to
 * `workspace` only (indices and offsets are read by the enqueued kernels and
 * may be reused once they have run).
 *
 * Planner output, all int32 in the workspace (tt_emb_plan_view):
 *   key[l]      = base_t + i2*m1 + i1 (base_t = sum of m1*m2 over earlier tables)
 *   i3[l], bag_of[l]
 *   perm        stable sort of lookups by (key, i3): groups in key order, inside a
 *               group by i3, equal (key, i3) keeping increasing l (repeats of one
 *               table row are adjacent and contracted once)
 *   groups      maximal runs of equal key in sorted order: group_key[g],
 *               group_start[g] (and group_start[U] = L)
 *   chunks      each group cut into consecutive pieces of exactly `chunk`
 *               lookups, the last possibly shorter; no chunk spans groups  */
tt_status tt_emb_plan(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                      const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                      void* workspace, size_t workspace_bytes, void* stream,
                      tt_emb_plan_t* plan_out);

/* Forward: out (device float[T*B][D]) is fully overwritten with the pooled
 * rows. g1/g2/g3 are the packed device cores. */
tt_status tt_emb_forward(tt_emb_plan_t plan, const float* g1, const float* g2,
                         const float* g3, float* out, void* stream);

/* Forward for training: the same result as tt_emb_forward, and the plan
 * also keeps each prefix group's shared partial product P = G1[i1] x G2[i2]
 * in its workspace, for one following tt_emb_backward_kept on this plan
 * (the FlowTT pages' sharing of reusable intermediates through checkpoint
 * buffers: summary card, key innovations; abstract).
 *   kept_token  receives a nonzero token naming the kept products, or 0 when
 *               the plan's shape has no matrix-core backward and nothing was
 *               kept (use tt_emb_backward then). May be NULL.
 * The token stays valid until the next call on this plan that changes or
 * uses the kept products: tt_emb_forward_train (a new token),
 * tt_emb_backward or tt_emb_backward_kept (they overwrite them), tt_emb_sgd
 * (the cores change). tt_emb_forward leaves it valid. */
tt_status tt_emb_forward_train(tt_emb_plan_t plan, const float* g1, const float* g2,
                               const float* g3, float* out, uint64_t* kept_token, void* stream);

/* Backward: dg1/dg2/dg3 (device, same packing and sizes as the cores) are
 * fully overwritten with the gradients of <grad_out, out>; slices that no
 * lookup touches are zero. grad_out is device float[T*B][D]. Forms every
 * prefix product again (it never uses products kept by
 * tt_emb_forward_train) and ends the validity of any kept token. */
tt_status tt_emb_backward(tt_emb_plan_t plan, const float* g1, const float* g2,
                          const float* g3, const float* grad_out, float* dg1, float* dg2,
                          float* dg3, void* stream);

/* Backward that reuses the prefix products kept by the tt_emb_forward_train
 * call that returned `kept_token`, instead of forming them again. Same
 * results as tt_emb_backward, provided the caller has not changed the
 * contents of G1 or G2 since that forward (the library cannot see such a
 * change). Returns TT_ERR_STALE, and launches nothing, when the token is 0,
 * is not the plan's current token (see tt_emb_forward_train), or g1/g2 are
 * not the pointers the forward was given. The kept products are consumed:
 * the token is no longer valid afterwards. */
tt_status tt_emb_backward_kept(tt_emb_plan_t plan, uint64_t kept_token, const float* g1,
                               const float* g2, const float* g3, const float* grad_out,
                               float* dg1, float* dg2, float* dg3, void* stream);

/* Backward fused with the SGD step: G_k <- G_k - lr * dG_k in place, for
 * the slices that some lookup of the batch touches (the others are neither
 * read nor written), without writing the gradients out. The result is bit
 * for bit that of the backward followed by tt_emb_sgd (untouched slices
 * have zero gradients, so the plain step leaves them unchanged too).
 *   kept_token  a token from tt_emb_forward_train to reuse its prefix
 *               products (rules as for tt_emb_backward_kept), or 0 to form
 *               them again
 *   g1, g2, g3  the cores, read and then updated in place
 * Returns TT_ERR_UNSUPPORTED for plans whose backward takes the generic
 * kernels (tt_emb_query_paths), TT_ERR_STALE for a token that does not name
 * the plan's kept products. Ends the validity of any kept token. */
tt_status tt_emb_backward_sgd(tt_emb_plan_t plan, uint64_t kept_token, float* g1, float* g2,
                              float* g3, const float* grad_out, float lr, void* stream);

/* SGD step on every core element: G <- G - lr * dG (device buffers). */
tt_status tt_emb_sgd(tt_emb_plan_t plan, float* g1, float* g2, float* g3, const float* dg1,
                     const float* dg2, const float* dg3, float lr, void* stream);

/* Synchronises `stream` and reads the device error flag of the plan into
 * *flag_out (0, or TT_FLAG_* bits). Returns TT_OK when the flag is clear and
 * TT_ERR_DEVICE_FLAG when it is set. */
tt_status tt_emb_get_error(tt_emb_plan_t plan, int32_t* flag_out, void* stream);

/* Device pointers to the planner's tables inside the workspace (no copy). */
typedef struct {
    const int32_t* key;          /* [L] original lookup order                  */
    const int32_t* i3;           /* [L]                                        */
    const int32_t* bag_of;       /* [L]                                        */
    const int32_t* perm;         /* [L] sorted position -> lookup              */
    const int32_t* sorted_i3;    /* [L] i3[perm[s]]                            */
    const int32_t* sorted_bag;   /* [L] bag_of[perm[s]]                        */
    const int32_t* group_key;    /* [num_groups]                               */
    const int32_t* group_start;  /* [num_groups + 1]                           */
    const int32_t* chunk_group;  /* [num_chunks]                               */
    const int32_t* chunk_begin;  /* [num_chunks] sorted positions              */
    const int32_t* chunk_end;    /* [num_chunks]                               */
    int64_t max_groups;          /* capacity of the group arrays               */
    int64_t max_chunks;          /* capacity of the chunk arrays               */
} tt_emb_plan_view;

tt_status tt_emb_plan_get_view(tt_emb_plan_t plan, tt_emb_plan_view* view);

/* Synchronises `stream` and reads the number of groups and chunks. */
tt_status tt_emb_plan_counts(tt_emb_plan_t plan, int64_t* num_groups, int64_t* num_chunks,
                             void* stream);

/* Frees the host handle (the workspace stays the caller's). NULL is a no-op.
 * Kernels of the plan that are already enqueued run to completion: they use
 * their launch arguments and caller-owned buffers only, not the handle. */
tt_status tt_emb_plan_destroy(tt_emb_plan_t plan);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation): plans the batch and runs the forward in one call, with the
 * same kernels and the same result as tt_emb_plan + tt_emb_forward, using a
 * static device buffer of the library's own instead of a caller workspace.
 * Arguments as for tt_emb_plan (tables, T, indices, offsets, L, B, chunk) and
 * tt_emb_forward (cores, out, stream); tables is read during the call only.
 * The buffer holds tt_emb_scratch_capacity() bytes (64 MiB) per device,
 * taken when the library is loaded and held until the process ends; a
 * forward-only plan of the 11M-row table (dim 128) fits about 100,000
 * lookups. A batch that needs more returns TT_ERR_SCRATCH before any device
 * work. Calls no allocator (device or host). All calls on one device share
 * its buffer: calls that overlap in time on one device (different streams,
 * different host threads) race and give undefined results; calls on one
 * stream are ordered and safe. Device-found data errors (bad index or
 * offsets) leave the output unspecified and are not reported (there is no
 * plan to query): validate inputs with tt_emb_plan first where that
 * matters. */
tt_status tt_emb_forward_scratch(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                                 const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                                 const float* g1, const float* g2, const float* g3, float* out,
                                 void* stream);

/* Bytes of the static device buffer tt_emb_forward_scratch uses. */
size_t tt_emb_scratch_capacity(void);

/* Which kernels a call on this plan runs (pure host query, no launch).
 * The matrix-core path serves plans whose tables all share one shape
 * (n1, n2, n3, R) among those the library is built for, with G1 and G2
 * offsets that are multiples of 4 floats, 16-byte aligned g1 and g2, and
 * m3 <= 1024. Forward shapes: (4,8,4,32), (4,4,4,32), (4,4,4,16),
 * (2,8,4,32), (8,4,4,32), (4,4,4,64), (4,4,8,32), (4,4,2,32), (4,4,1,32);
 * the backward's matrix-core kernels serve the first six (n3 = 4) for tables
 * that do not share a G2 core. Other plans take the generic kernels (scalar
 * FMA, one workgroup per chunk, fp32 atomics whose summation order varies
 * from run to run). */
#define TT_PATH_MATRIX_CORE 1
#define TT_PATH_GENERIC 2
typedef struct {
    int32_t forward_path;     /* TT_PATH_* of tt_emb_forward / _forward_train        */
    int32_t backward_path;    /* TT_PATH_* of tt_emb_backward / _backward_kept       */
    int32_t keeps_prefix;     /* 1: tt_emb_forward_train keeps P (nonzero token)     */
    int32_t dg3_by_rows;      /* 1: dG3 reduced per G3 row from per-run terms;       */
                              /* 0: fp64 device atomics (G3 rows not aligned, or     */
                              /* more than 8192 G3 rows in all)                      */
    uint64_t workspace_bytes; /* the plan's workspace size (tt_emb_workspace_bytes)  */
} tt_emb_path_info;

tt_status tt_emb_query_paths(tt_emb_plan_t plan, const float* g1, const float* g2,
                             tt_emb_path_info* info);

/* Kernel timing, for measurement. With timing on, every kernel that a call
 * on this plan enqueues is bracketed by two HIP events recorded on that
 * call's stream (the first 1024 launches since the last read are kept).
 * tt_emb_kernel_times synchronises `stream`, writes up to `max` records in
 * launch order (kernel name, static storage; milliseconds between the two
 * events), sets *count, and clears the records. Timing adds two event
 * records per launch; it is off unless enabled. tt_emb_set_timing(NULL, on)
 * sets it for every plan created afterwards (from its planning kernels on). */
typedef struct {
    const char* kernel;
    float ms;
} tt_emb_kernel_time;

tt_status tt_emb_set_timing(tt_emb_plan_t plan, int32_t enable);
tt_status tt_emb_kernel_times(tt_emb_plan_t plan, tt_emb_kernel_time* out, int32_t max,
                              int32_t* count, void* stream);

/* Hot-row cache. TT-Rec pairs the TT table with caching for the lookups
 * (TT-Rec abstract: caching strategies; news article, method paragraph: a
 * cache structure that exploits the skewed sparse-feature distribution and
 * changes accuracy). Here a set of hot rows is kept uncompressed, as
 * trainable fp32 vectors: hot entry s is the pair (hot_table[s],
 * hot_row[s]) with its vector W[s] (D floats, a caller buffer [n_hot][D]).
 * A lookup of a hot row takes W[s] in place of the TT contraction; in the
 * backward its grad row goes to dW[s], and the cores get gradients from the
 * other lookups only. A pair listed twice is served by its first slot (the
 * later slot gets no lookups); a pair naming no valid row matches nothing.
 * Which rows are hot, and how W[s] starts (for instance the row's TT value,
 * from a forward of one-lookup bags), is the caller's choice.
 *
 * The cache is a device hash table in caller memory: tt_emb_cache_bytes(n)
 * bytes (256-byte aligned), filled by tt_emb_cache_build from device arrays
 * hot_table (int32 [n_hot]) and hot_row (int64 [n_hot]) on `stream`; it is
 * read by tt_emb_plan_cached (and must stay unchanged while plans made with
 * it are used). A plan made with a cache takes only the _cached compute calls
 * (the others return TT_ERR_CACHE), and only shapes with the matrix-core
 * kernels in both directions (tt_emb_query_paths; else TT_ERR_UNSUPPORTED at
 * the compute call). n_hot = 0 is allowed and changes nothing. */
size_t tt_emb_cache_bytes(int64_t n_hot);
tt_status tt_emb_cache_build(const int32_t* hot_table, const int64_t* hot_row, int64_t n_hot,
                             void* cache, size_t cache_bytes, void* stream);

/* As tt_emb_plan, for a batch served with the hot-row cache `cache` of
 * n_hot entries (built by tt_emb_cache_build with the same n_hot). */
tt_status tt_emb_plan_cached(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                             const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                             const void* cache, int64_t n_hot, void* workspace,
                             size_t workspace_bytes, void* stream, tt_emb_plan_t* plan_out);

/* Forward with the hot rows W (fp32 [n_hot][D], read only). kept_token NULL:
 * as tt_emb_forward; non-NULL: as tt_emb_forward_train (the token names the
 * kept products). */
tt_status tt_emb_forward_cached(tt_emb_plan_t plan, const float* g1, const float* g2,
                                const float* g3, const float* hot_w, float* out,
                                uint64_t* kept_token, void* stream);

/* Backward: dG1..dG3 as tt_emb_backward (from the lookups of rows outside
 * the hot set) and dW (fp32 [n_hot][D], every row written: zero for hot rows
 * the batch does not look up). kept_token 0: P is formed again; otherwise
 * as tt_emb_backward_kept (TT_ERR_STALE for a stale token). */
tt_status tt_emb_backward_cached(tt_emb_plan_t plan, uint64_t kept_token, const float* g1,
                                 const float* g2, const float* g3, const float* grad_out,
                                 float* dg1, float* dg2, float* dg3, float* hot_dw, void* stream);

/* Backward fused with the SGD step on the cores and on W (in place, W[s]
 * updated only for hot rows the batch looks up), as tt_emb_backward_sgd. */
tt_status tt_emb_backward_sgd_cached(tt_emb_plan_t plan, uint64_t kept_token, float* g1, float* g2,
                                     float* g3, float* hot_w, const float* grad_out, float lr,
                                     void* stream);

/* Human-readable name of a status code (static storage). */
const char* tt_emb_status_string(tt_status s);

#ifdef __cplusplus
}
#endif

#endif /* TT_EMB_H */
