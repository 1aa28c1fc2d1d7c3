// Internal definitions shared by the HIP sources of libtt_emb.so (not part of
// the C ABI). Written for gfx950 (CDNA4): wave64, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "tt_emb.h"

namespace tt {

// Per-table descriptor as the kernels read it (device copy in the workspace).
struct alignas(16) TabDev {
    int32_t N, m1, m2, m3;      // rows and radices
    int32_t n1, n2, n3, R;      // dim factors and rank
    int64_t o1, o2, o3;         // element offsets of this table's G1/G2/G3
    int32_t key_base;           // first prefix key of this table
    int32_t i2_base;            // first (table, i2) slice index of this table
    int32_t fb_base;            // first forward batch (kFwdBatch groups of one slice) of this table
    int32_t pad_;
    int64_t g3_base;            // first element of this table's G3 in a walk over every table's G3
};
static_assert(sizeof(TabDev) == 80, "TabDev layout");

// Control words at the head of the workspace (int32 slots).
enum CtrlSlot : int {
    CTRL_FLAG = 0,        // TT_FLAG_* bits
    CTRL_NUM_GROUPS = 1,
    CTRL_NUM_CHUNKS = 2,
    CTRL_NUM_RUNS = 4,    // row runs
    CTRL_NUM_XPIECES = 5, // backward: extra run pieces of the groups split over several waves
    CTRL_NUM_BATCHES = 6, // forward batches that hold a group (the compacted batch list's length)
    CTRL_CLASS_BASE = 8,  // 8 words: start of each XCD class's part of the batch list (class c:
                          //     slices with global index = c mod 8); the list's length after them
    CTRL_SCAN_CTR = 24,   // tile counters of the single-pass scans, one per scan of a plan
    CTRL_SCAN_MAX = 16,   //   (at most this many scans per plan)
    CTRL_WORDS = 64
};

constexpr int kXcds = 8;
// Table shapes (n1, n2, n3, R) the matrix-core kernels are built for, every
// table of a plan having the same one; the last field says whether the
// backward's matrix-core kernels serve the shape too (they need n3 = 4 and
// a dim that is a multiple of 64). Other shapes take the generic kernels.
#define TT_MFMA_SHAPES(X)                                                                         \
    X(4, 8, 4, 32, true) X(4, 4, 4, 32, true) X(4, 4, 4, 16, true) X(2, 8, 4, 32, true)           \
    X(8, 4, 4, 32, true) X(4, 4, 4, 64, true) X(4, 4, 8, 32, false) X(4, 4, 2, 32, false)         \
    X(4, 4, 1, 32, false)

// Forward work unit: up to this many prefix groups of one (table, i2) slice.
constexpr int kFwdBatch = 8;
// Spare stage rows after the L run rows (targets of inactive lanes' stores).
constexpr int kStageSpare = 16;
// Workgroups (four waves each) of the persistent forward batch kernel: three
// per CU (the kernel's registers and LDS allow no more).
constexpr int kFwdPersistBlocks = 3 * 256;
// The backward's run kernel hands out row runs in ranges of about this many
// (a group of more runs is split; smaller groups are never split).
constexpr int kRunRange = 32;
// At most this many pieces of split groups are listed (each has an fp64 dP
// slot in the workspace); the groups that would exceed it run whole, one
// wave each.
constexpr int64_t kMaxXPieces = 8192;
// The run kernel's waves claim their units from this many counters (each on a
// 128-byte line of its own; counter c hands out units c, c + kRunCounters,
// ...), the waves of workgroup b from counter b mod kRunCounters.
constexpr int kRunCounters = 32;
// The forward batch kernel's workgroups claim their batches from this many
// counters (after the run kernel's in the same array): workgroup b from
// counter b mod kFwdCounters, whose XCD class is b mod kXcds.
constexpr int kFwdCounters = 32;
static_assert(kFwdCounters % kXcds == 0, "each counter serves one XCD class");
// With at most this many G3 rows in all (any number of tables, each table's
// G3 offset a whole number of R*n3 rows), dG3 is reduced per G3 row from
// per-run terms (one workgroup per row sums its bucket) instead of with
// device atomics.
constexpr int kMaxBuckets3 = 8192;   // G3 rows whose runs the planner counts (see Layout::i3cnt)
constexpr int kI3Pad = 32;   // int32 words per i3 counter (one 128-byte line each)
// LDS the batch kernels may spend on the run i3 list of one batch
// (kFwdBatch * largest m3 int32 values); larger m3 takes the generic kernels.
constexpr int kMaxBatchI3Bytes = 32768;

// One forward batch as the planner describes it to the batch kernels: up to
// kFwdBatch groups of one (table, i2) slice, consecutive in key order. Slot j
// of slice i2 of table t is batch slot fb_base_t + j*m2_t + i2 (layer-major:
// the first kFwdBatch groups of every slice, then the next ones, ...). The
// planner keeps the slots that hold a group as the batch list, in 8 parts by
// XCD class (the slice's global index mod 8), each part in slot order (under
// skew the first layer holds the low i1 and the heaviest groups, so each
// part starts with its heaviest batches). Workgroups run on XCD blockIdx mod
// 8, so a workgroup that walks the part of its own class reads the G2 slices
// that its XCD's L2 already holds.
struct alignas(16) BatchRec {
    int32_t ng;                    // groups in the batch (0: nothing to do)
    int32_t g0;                    // first group
    int32_t i2;                    // slice index inside the table
    int32_t rb0;                   // first row run of the batch
    int32_t nr;                    // row runs of the batch
    int32_t pad0[3];
    int64_t o1, o2, o3;            // the table's core offsets
    int32_t pad1[2];
    int32_t i1[kFwdBatch];         // i1 of each group (0 past ng)
    int32_t rbase[kFwdBatch + 1];  // first row run of each group, relative to rb0; then nr
    int32_t pad2[7];
};
static_assert(sizeof(BatchRec) == 160, "BatchRec layout");

constexpr int kSlotTile = 256;   // batch slots per workgroup of the planner's batch-list kernel

constexpr int kRadixBits = 8;
constexpr int kRadixBins = 1 << kRadixBits;
constexpr int kSortThreads = 1024;                       // 16 waves
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 4;                            // per thread
constexpr int kSortTile = kSortThreads * kSortItems;     // 4096 lookups per tile
// Up to this many tiles, each scatter workgroup sums the per-tile digit counts
// it needs itself; beyond, a device-wide scan of the counts runs between the
// two kernels of a pass.
constexpr int64_t kDirectTiles = 512;
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanThreads * kScanItems;     // 4096 per scan tile

// Limits (mirrored in the public header's comment).
constexpr int kMaxR = 64;
constexpr int kMaxN12 = 64;
constexpr int kMaxN3 = 16;
constexpr int kMaxD = 1024;
constexpr int kMaxTables = 4096;
constexpr int64_t kMaxKeys = int64_t(1) << 30;

// Tile status of the single-pass scans: flag = (epoch << 2) | state, state 1
// when `agg` (the tile's total) is published, 2 when `incl` (the sum through
// the tile) is.
struct alignas(32) ScanTileStatus {
    uint32_t flag;
    uint32_t pad_;
    uint64_t agg;
    uint64_t incl;
};

// Carving of the caller's workspace. Every array starts on a 256-byte boundary.
struct Layout {
    size_t ctrl, scan_st, desc;               // scan_st: tile status words of the single-pass
                                             //     scans, right after ctrl (cleared with it)
    size_t key, i3, bag_of;                  // [L]
    size_t ckey;                             // [L] sort key = key * M3 + i3
    size_t cslot;                            // [L] int32: each lookup's hot-row slot (-1: not hot),
                                             //     cached plans only (full layouts)
    size_t run_cslot;                        // [L] int32: each row run's hot-row slot (-1: not hot)
    size_t bag_start;                        // [TB+1] int32 copy of the offsets
    size_t rid;                              // [L] int32, sorted order: number of row-run heads before s
    size_t run_i3;                           // [L] int32: i3 of each run
    size_t run_of;                           // [L] int32, input order: run id of each lookup
    size_t run_start;                        // [L] int32: first sorted position of each row run
    size_t run_bag1;                         // [L] int32 (plans with the backward): the bag of a run
                                             //     of one lookup (its S is that grad row), else -1
    size_t xpiece;                           // [xcap] int32 pairs: (group, piece) (backward)
    size_t dpart;                            // [xcap][n1*n2*R] double: dP of each listed piece
    size_t group_rbase;                      // [Gmax+1] int32: first row run of each group
    size_t stage;                            // [L + kStageSpare][D] float, one row per row run: forward, the
                                             //     run's embedding row; backward, its grad-row sum S,
                                             //     then (bucketed dG3) its dG3 term P^T S over S
    size_t perm, sorted_i3, sorted_bag;      // [L]
    size_t skey, sort_k0, sort_v0, sort_b0, sort_k1, sort_v1, sort_b1;  // [L] radix ping-pong
    size_t hist;                             // [kRadixBins][hstride] uint32: digit counts per tile
    size_t key_start, key_end;               // [K] int32
    size_t key_scan;                         // [K] uint64
    size_t run_tiles;                        // [n_tiles] uint32: row-run heads per tile of sorted positions
    size_t key_tiles;                        // [n_ktiles] uint64: key words per tile of keys
    size_t group_key, group_start, group_cbase;   // [Gmax], [Gmax+1], [Gmax+1]
    size_t chunk_group, chunk_begin, chunk_end;   // [Cmax]
    size_t gdone;                            // [Gmax] int32: pieces of a split group finished (backward);
                                             //     -1: a group too large for the piece list, run whole
    size_t pbuf;                             // [Gmax][n1*n2*R] float: P per group, in the lane order of the
                                             //     matrix-core operands; the backward's run kernel then
                                             //     writes each group's dL/dP over it (row-major)
    size_t g3t;                              // [extent of G3] float: each G3 slice transposed to [n3][R]
                                             //     (the forward's suffix operand, written per forward call)
    size_t c3;                               // [L][R*n3] float, only when R*n3 > D (and dG3 is bucketed):
                                             //     each run's dG3 term P^T S (else written over its S row)
    size_t acc1, acc3;                       // [extent of G1], [extent of G3] double: dG1 and
                                             //     dG3 accumulated in fp64 by the backward
    size_t acc2;                             // [extent of G2] double: dG2 of the generic backward
    size_t xsum;                             // [2*ceil(L/64)][D] double: pieces of the row runs
                                             //     cut by the backward's windows
    size_t xcnt;                             // [ceil(L/64)] int32: spans done per long cut run
    size_t claims;                           // [kRunCounters + kFwdCounters][32] int32: the run kernel's and
                                             //     the forward batch kernel's claim counters
    // the backward's c3 rows, bucketed by G3 row (table's G3 offset / (R*n3) + i3),
    // when every table's G3 offset is a whole number of rows and there are at
    // most kMaxBuckets3 rows (NB3 of them; else NB3 = 0 and dG3 takes atomics)
    size_t i3cnt;                            // [NB3][kI3Pad] int32: runs per bucket (one counter per line)
    size_t i3start;                          // [NB3 + 1] int32: exclusive scan of the counts
    size_t run_rank;                         // [L] int32: rank of each run inside its bucket
    size_t run_bkt;                          // [L] int32: bucket (G3 row) of each run
    size_t bucket_runs;                      // [L] int32: backward: the runs of each bucket, in rank order
    size_t batch_tiles;                      // [ceil(NFB/kSlotTile)][kXcds] uint32: slots holding a group
                                             //     per tile of kSlotTile batch slots and XCD class
    size_t batch_place;                      // [NFB] int32: each slot's place in the batch list (-1: none),
                                             //     indexed slice-major (fb_base + i2*ceil(m1/kFwdBatch) + jb)
    size_t batch;                            // [NFB] BatchRec: the batches that hold a group,
                                             //     compacted (CTRL_NUM_BATCHES of them)
    size_t total;
    int64_t n_tiles, hstride, n_ktiles, K, Gmax, Cmax, NFB, scan_tiles, NB3, xcap;
    int passes;
};

Layout make_layout(int32_t T, int64_t L, int64_t B, int32_t chunk, int64_t K, int32_t D,
                   int64_t M3, int64_t PR, int64_t CN, int64_t E1, int64_t E2, int64_t E3, int64_t NFB,
                   int64_t NB3, bool fwd_only);

// Kernel timing of a plan (tt_emb_set_timing): a start and an end event per
// launch, recorded on the launch's stream, read back by tt_emb_kernel_times.
struct Timing {
    static constexpr int kCap = 1024;
    const char* name[kCap];
    hipEvent_t ev[kCap][2];
    int n = 0;         // launches recorded since the last read
    int created = 0;   // event pairs created so far (slots [0, created))
};
void timing_free(Timing* t);

}  // namespace tt

// Host-side plan handle.
struct tt_emb_plan_s {
    int32_t T;
    int64_t L, B, TB;
    int32_t chunk;
    int32_t D;
    int64_t K;
    int32_t M3;               // largest m3 over the tables
    int32_t nb3;              // G3 rows of the dG3 buckets (0: dG3 by device atomics)
    int64_t cn;               // R*n3 (the G3 row length) when nb3 > 0
    int64_t n_i2;             // sum over tables of m2 (number of (table, i2) slices)
    int64_t n_fb;             // forward batches: sum over tables of m2 * ceil(m1 / kFwdBatch)
    bool uniform;             // all tables share (n1, n2, n3, R)
    int32_t n1, n2, n3, R;    // the shared shape when uniform
    int64_t extent[3];        // elements of the packed G1/G2/G3 buffers in use
    int64_t g3_total;         // sum over tables of m3*R*n3 (the G3 elements the tables use)
    bool packed;              // tables' cores sit back to back from offset 0 (no gaps)
    bool off4;                // every table's G1 and G2 offsets are multiples of 4 floats
    bool g2_overlap;          // two tables' G2 ranges overlap (a shared core)
    uint64_t kept_token;      // nonzero: pbuf holds P of every group for kept_g1/kept_g2, kept by
                              //     the tt_emb_forward_train call that returned this token
    uint64_t next_token;      // last token handed out on this plan
    const float* kept_g1;
    const float* kept_g2;
    bool fwd_only;            // the layout holds no backward buffers (forward calls only)
    bool cached = false;      // planned with a hot-row cache (tt_emb_plan_cached)
    int64_t n_hot = 0;        // the cache's entries
    const int64_t* hot_keys = nullptr;    // the cache's hash table (device): keys, then slots
    const int32_t* hot_slots = nullptr;
    int32_t hot_lg = 0;       // log2 of the table's capacity
    char* ws;                 // workspace base (device)
    tt::Layout lay;
    const tt_emb_table* tables = nullptr;     // T descriptors (owned_tables, or the caller's
    tt_emb_table* owned_tables = nullptr;     //     array for the length of one call)
    tt::Timing* timing = nullptr;             // non-null while kernel timing is on

    ~tt_emb_plan_s() {
        delete[] owned_tables;
        tt::timing_free(timing);
    }

    template <class P>
    P* at(size_t off) const { return reinterpret_cast<P*>(ws + off); }
    int32_t* ctrl() const { return at<int32_t>(lay.ctrl); }
    const tt::TabDev* desc() const { return at<tt::TabDev>(lay.desc); }
};

#define TT_HIP_CHECK(expr)                                  \
    do {                                                    \
        hipError_t _e = (expr);                             \
        if (_e != hipSuccess) return TT_ERR_HIP;            \
    } while (0)

#define TT_LAUNCH_CHECK()                                   \
    do {                                                    \
        hipError_t _e = hipGetLastError();                  \
        if (_e != hipSuccess) return TT_ERR_HIP;            \
    } while (0)

namespace tt {
// Waits until every memory access this wave has issued has completed (for
// device-scope stores and atomics: performed at the level all XCDs share).
// Used before a completion count or a ready flag is published, in place of a
// device-scope release fence, which on this chip also writes back the whole
// L2 of the XCD.
__device__ __forceinline__ void wait_vmem_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Plans into *p without allocating (plan.hip); the workspace size of a layout.
tt_status plan_into(tt_emb_plan_s* p, const tt_emb_table* tables, int32_t T, const int64_t* indices,
                    const int64_t* offsets, int64_t L, int64_t B, int32_t chunk, void* workspace,
                    size_t workspace_bytes, bool fwd_only, hipStream_t s, const void* cache = nullptr,
                    int64_t n_hot = 0);
size_t workspace_bytes_for(const tt_emb_table* tables, int32_t T, int64_t L, int64_t B, int32_t chunk,
                           bool fwd_only);
// The forward on a plan (forward.hip); keep: also keep P (needs a full layout).
tt_status forward_run(tt_emb_plan_s* p, const float* g1, const float* g2, const float* g3, float* out,
                      bool keep, uint64_t* token, hipStream_t s, const float* hot_w = nullptr);

// Whether the plan's calls take the matrix-core kernels with these cores
// (forward.hip, backward.hip).
bool mfma_shape(int n1, int n2, int n3, int R, bool backward);
bool fwd_mfma_ok(const tt_emb_plan_s* p, const float* g1, const float* g2);
bool bwd_mfma_ok(const tt_emb_plan_s* p, const float* g1, const float* g2);

// Kernel timing hooks around one launch (no-ops unless the plan times its
// kernels): kt_begin records the start event and returns the record's slot
// (-1: not recorded), kt_end records the end event.
int kt_begin(const tt_emb_plan_s* p, const char* name, hipStream_t s);
void kt_end(const tt_emb_plan_s* p, int slot, hipStream_t s);

inline unsigned grid_for(int64_t n, int threads) {
    int64_t g = (n + threads - 1) / threads;
    return (unsigned)(g < 1 ? 1 : g);
}
// Fill `n` 32-bit words at `ptr` with `v` (stream-ordered, capture-safe).
tt_status fill32(const tt_emb_plan_s* p, void* ptr, uint32_t v, int64_t n, hipStream_t s);

// Hot-row cache: an open-addressing hash table (linear probing, at most half
// full) of 2^lg int64 keys (table << 40 | row; -1: empty) and int32 slots,
// after a 256-byte header, in caller memory.
constexpr int64_t kHotEmpty = -1;
constexpr int kHotHeader = 256;
inline int cache_lg(int64_t n_hot) {
    int lg = 6;
    while ((int64_t(1) << lg) < 2 * n_hot) ++lg;
    return lg;
}
inline size_t cache_bytes_lg(int lg) {
    const size_t c = size_t(1) << lg;
    return (size_t)kHotHeader + ((8 * c + 255) & ~size_t(255)) + ((4 * c + 255) & ~size_t(255));
}
__host__ __device__ inline size_t cache_slots_offset(int lg) {
    return (size_t)kHotHeader + ((8 * (size_t(1) << lg) + 255) & ~size_t(255));
}
__device__ __forceinline__ uint64_t cache_hash(int64_t key, int lg) {
    return ((uint64_t)key * 0x9E3779B97F4A7C15ull) >> (64 - lg);
}
// Slot of `key` in the table, or -1 (the probe ends at the first empty entry;
// the table always has one).
__device__ __forceinline__ int32_t cache_probe(const int64_t* __restrict__ keys, const int32_t* __restrict__ slots,
                                               int lg, int64_t key) {
    const uint64_t mask = (uint64_t(1) << lg) - 1;
    uint64_t h = cache_hash(key, lg);
    for (uint64_t n = 0; n <= mask; ++n) {
        const int64_t k = keys[h];
        if (k == key) return slots[h];
        if (k == kHotEmpty) return -1;
        h = (h + 1) & mask;
    }
    return -1;
}
}  // namespace tt

// A kernel launch on stream `s` for plan `p`, bracketed by the plan's timing
// events when timing is on.
#define TT_LAUNCH(p, name, s, ...)                              \
    do {                                                        \
        const int _kt_slot = tt::kt_begin((p), (name), (s));    \
        hipLaunchKernelGGL(__VA_ARGS__);                        \
        tt::kt_end((p), _kt_slot, (s));                         \
    } while (0)
