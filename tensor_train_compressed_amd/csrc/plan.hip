// Planning pass of the TT-EmbeddingBag library: index split, prefix grouping
// and chunking, all on the GPU.
//
// The pages' task-formation step groups lookups that share high-order TT core
// indices so that the shared part of the contraction chain is done once per
// group, and cuts skewed groups into chunks for load balance ("FlowTT:
// Exploiting Computation Flow Reuse in Irregular Tensor-Train Embedding":
// summary card, key innovations; abstract). The pages fix which
// lookups share a group; the order and chunk shape used here are this
// library's (see include/tt_emb.h): groups are ordered by key
// base_t + i2*m1 + i1, so that groups that read the same G2 slice are
// adjacent; inside a group lookups are ordered by i3 (ties in input order), so
// repeats of one table row are adjacent and that row is contracted once.
//
// Kernels, in stream order:
//   k_init            clears the control words, writes the table descriptors
//   k_split           offsets check, bag labels, digit split, prefix key; marks keys absent
//   k_radix_hist      \  stable LSD radix sort of key*M3 + i3, 8 bits per pass:
//   k_radix_scatter   /  per-tile digit counts, then wave-ballot stable ranks inside a
//                        tile, staged in LDS and written out in digit runs
//   k_gather          sorted i3, first and last position of each key, row-run heads
//                     per tile (the sorted bags come out of the sort)
//   k_key_tiles       present keys and chunks per tile of keys
//   k_groups          key scan (group id and first chunk of every key), group tables
//   k_runs            row-run ids and tables, chunk table; runs per G3 row
//   k_runs            (also counts the forward batch slots that hold a group, per tile)
//   k_batches         the records of the batch slots (kFwdBatch groups of one slice) that
//                     hold a group, compacted into the batch list
// A device-wide scan of the tile totals runs before k_radix_scatter, k_groups
// or k_runs only when there are more than kDirectTiles tiles.
#include "tt_internal.h"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>

namespace tt {

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int32_t T, int64_t L, int64_t B, int32_t chunk, int64_t K, int32_t D,
                   int64_t M3, int64_t PR, int64_t CN, int64_t E1, int64_t E2, int64_t E3, int64_t NFB,
                   int64_t NB3, bool fwd_only) {
    Layout y{};
    // a forward-only plan carries none of the backward's buffers
    const int64_t LB = fwd_only ? 0 : L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + (bytes ? bytes : 1)); return o; };
    y.K = K;
    y.n_tiles = (L + kSortTile - 1) / kSortTile;
    y.hstride = (y.n_tiles + 15) & ~int64_t(15);   // rows of whole 64-byte lines (padding kept zero)
    y.Gmax = std::min<int64_t>(L, K);
    y.Cmax = L == 0 ? 0 : std::min<int64_t>(L, y.Gmax + (L + chunk - 1) / chunk);
    int bits = 0;
    while ((int64_t(1) << bits) < K * M3) ++bits;
    y.passes = std::max(1, (bits + kRadixBits - 1) / kRadixBits);
    y.ctrl = take(sizeof(int32_t) * CTRL_WORDS);
    {
        const int64_t nh = (int64_t)kRadixBins * y.hstride;
        const int64_t nscan = std::max<int64_t>(std::max<int64_t>(nh, K), L);
        y.scan_tiles = (nscan + kScanTile - 1) / kScanTile + 1;
        y.scan_st = take(sizeof(ScanTileStatus) * (size_t)y.scan_tiles);
    }
    y.desc = take(sizeof(TabDev) * (size_t)T);
    const size_t l4 = sizeof(int32_t) * (size_t)L;
    y.key = take(l4); y.i3 = take(l4); y.bag_of = take(l4);
    y.ckey = take(l4);
    // hot-row slots (plans with a hot-row cache; always carved in full layouts)
    y.cslot = take(sizeof(int32_t) * (size_t)LB);
    y.run_cslot = take(sizeof(int32_t) * (size_t)LB);
    y.bag_start = take(sizeof(int32_t) * (size_t)((int64_t)T * B + 1));
    y.rid = take(l4);
    y.run_i3 = take(l4);
    y.run_of = take(l4);
    y.run_start = take(l4);
    y.run_bag1 = take(sizeof(int32_t) * (size_t)LB);
    // pieces of the groups with more than kRunRange row runs: a group of n > W
    // runs has ceil(n / W) < 2n / W of them, so fewer than 2L / W in all; at
    // most kMaxXPieces are listed (the groups past that run whole)
    y.xcap = fwd_only ? 0 : std::min<int64_t>(2 * (L / kRunRange) + 1, kMaxXPieces);
    const size_t xcap = (size_t)y.xcap;
    y.xpiece = take(sizeof(int32_t) * 2 * xcap);
    y.dpart = take(sizeof(double) * xcap * (size_t)PR);
    // one row per row run, plus kStageSpare rows that take the writes of
    // inactive lanes (kept branch-free) in the forward
    y.stage = take(sizeof(float) * ((size_t)L + kStageSpare) * (size_t)D);
    y.perm = take(l4); y.sorted_i3 = take(l4); y.sorted_bag = take(l4);
    y.skey = take(l4);
    // The radix passes move (sort key, lookup, bag) and ping-pong between
    // (skey, perm, sorted_bag) and a temporary triple that reuses sorted_i3,
    // rid and run_start, which are written only after the sort.
    y.sort_k0 = y.sorted_i3; y.sort_v0 = y.rid; y.sort_b0 = y.run_start;
    y.sort_k1 = y.skey; y.sort_v1 = y.perm; y.sort_b1 = y.sorted_bag;
    const int64_t nhist = (int64_t)kRadixBins * y.hstride;
    y.hist = take(sizeof(uint32_t) * (size_t)nhist);
    y.key_start = take(sizeof(int32_t) * (size_t)K);
    y.key_end = take(sizeof(int32_t) * (size_t)K);
    y.key_scan = take(sizeof(uint64_t) * (size_t)K);
    y.n_ktiles = (K + kSortTile - 1) / kSortTile;
    y.run_tiles = take(sizeof(uint32_t) * (size_t)y.n_tiles);
    y.key_tiles = take(sizeof(uint64_t) * (size_t)y.n_ktiles);
    y.group_key = take(sizeof(int32_t) * (size_t)y.Gmax);
    y.group_start = take(sizeof(int32_t) * (size_t)(y.Gmax + 1));
    y.group_cbase = take(sizeof(int32_t) * (size_t)(y.Gmax + 1));
    y.group_rbase = take(sizeof(int32_t) * (size_t)(y.Gmax + 1));
    y.chunk_group = take(sizeof(int32_t) * (size_t)y.Cmax);
    y.chunk_begin = take(sizeof(int32_t) * (size_t)y.Cmax);
    y.chunk_end = take(sizeof(int32_t) * (size_t)y.Cmax);
    const int64_t GB = fwd_only ? 0 : y.Gmax;
    y.gdone = take(sizeof(int32_t) * (size_t)GB);
    // P per group (kept from the training forward, or formed by the
    // backward), then dL/dP per group written over it by the run kernel
    y.pbuf = take(sizeof(float) * (size_t)GB * (size_t)PR);
    y.g3t = take(sizeof(float) * (size_t)E3);
    y.acc1 = take(fwd_only ? 0 : sizeof(double) * (size_t)E1);
    y.acc2 = take(fwd_only ? 0 : sizeof(double) * (size_t)E2);   // the generic backward only
    y.acc3 = take(fwd_only ? 0 : sizeof(double) * (size_t)E3);
    // each run's dG3 term P^T S (R*n3 floats) goes over the run's S row when
    // that row is long enough, else into a buffer of its own
    y.c3 = take(NB3 > 0 && CN > D ? sizeof(float) * (size_t)L * (size_t)CN : 0);
    // fp64 pieces of the row runs cut by the backward's 64-position windows:
    // two slots per window (its start piece and its end piece)
    y.xsum = take(sizeof(double) * 2 * (size_t)((LB + 63) / 64) * (size_t)D);
    y.xcnt = take(sizeof(int32_t) * (size_t)((LB + 63) / 64));
    y.claims = take(sizeof(int32_t) * 32 * (kRunCounters + kFwdCounters));
    y.NB3 = NB3;
    y.i3cnt = take(sizeof(int32_t) * (size_t)NB3 * kI3Pad);
    y.i3start = take(sizeof(int32_t) * (size_t)(NB3 + 1));
    y.run_rank = take(sizeof(int32_t) * (size_t)LB);
    y.run_bkt = take(NB3 > 0 ? sizeof(int32_t) * (size_t)L : 0);
    y.bucket_runs = take(NB3 > 0 ? sizeof(int32_t) * (size_t)L : 0);
    y.NFB = NFB;
    y.batch_tiles = take(sizeof(uint32_t) * kXcds * (size_t)((NFB + kSlotTile - 1) / kSlotTile));
    y.batch_place = take(sizeof(int32_t) * (size_t)NFB);
    y.batch = take(sizeof(BatchRec) * (size_t)NFB);
    y.total = off;
    return y;
}

// ---------------------------------------------------------------------------
// small utilities

__global__ void k_fill32(uint32_t* p, uint32_t v, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

tt_status fill32(const tt_emb_plan_s* p, void* ptr, uint32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return TT_OK;
    unsigned g = std::min<unsigned>(grid_for(n, 256), 4096u);
    TT_LAUNCH(p, "k_fill32", s, k_fill32, dim3(g), dim3(256), 0, s, (uint32_t*)ptr, v, n);
    TT_LAUNCH_CHECK();
    return TT_OK;
}

// ---------------------------------------------------------------------------
// kernel timing

void timing_free(Timing* t) {
    if (!t) return;
    for (int i = 0; i < t->created; ++i) {
        (void)hipEventDestroy(t->ev[i][0]);
        (void)hipEventDestroy(t->ev[i][1]);
    }
    delete t;
}

int kt_begin(const tt_emb_plan_s* p, const char* name, hipStream_t s) {
    Timing* t = p ? p->timing : nullptr;
    if (!t || t->n >= Timing::kCap) return -1;
    const int i = t->n;
    if (i >= t->created) {
        if (hipEventCreate(&t->ev[i][0]) != hipSuccess) return -1;
        if (hipEventCreate(&t->ev[i][1]) != hipSuccess) {
            (void)hipEventDestroy(t->ev[i][0]);
            return -1;
        }
        t->created = i + 1;
    }
    if (hipEventRecord(t->ev[i][0], s) != hipSuccess) return -1;
    t->name[i] = name;
    return i;
}

void kt_end(const tt_emb_plan_s* p, int slot, hipStream_t s) {
    if (slot < 0) return;
    Timing* t = p->timing;
    if (hipEventRecord(t->ev[slot][1], s) == hipSuccess) t->n = slot + 1;
}

struct DescBatch {
    int32_t first, count;
    TabDev d[16];
};

__global__ void k_write_desc(TabDev* out, DescBatch b) {
    int i = threadIdx.x;
    if (i < b.count) out[b.first + i] = b.d[i];
}

// Clears `nzero` words from `zero` (the control words and the scans' status
// words) and writes the first batch of table descriptors.
__global__ __launch_bounds__(256) void k_init(uint32_t* __restrict__ zero, int64_t nzero,
                                              TabDev* __restrict__ out, DescBatch b) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = t; i < nzero; i += (int64_t)gridDim.x * blockDim.x) zero[i] = 0u;
    if (t < b.count) out[b.first + t] = b.d[t];
}

// 64-lane match: mask of valid lanes whose digit equals this lane's.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, uint64_t valid) {
    uint64_t peers = valid;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
        const uint64_t bal = __ballot((d >> b) & 1u);
        peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    return peers;
}

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---------------------------------------------------------------------------
// split
//
// Workgroups 0 .. n_tiles-1 take one tile of kSortTile lookups each (the
// sort's tiles), kSortItems per thread: each lookup's table, digits and
// prefix key, and the tile's counts of the sort key's lowest digit (the
// first radix pass's histogram, as k_radix_hist writes it for the later
// passes). The workgroups after them, running alongside, take kSortThreads
// offsets, kSortTile keys and kSortTile G3 buckets each: bag_start and the
// offsets check; every wave labels the lookups of its 64 bags, consecutive
// lanes on consecutive lookups (lane j holds bag j's offset; a lookup's bag is
// the last lane whose offset is not past it, found by a binary search over
// the lanes); keys marked absent; bucket run counters cleared.

__device__ __forceinline__ uint32_t sort_digit(int32_t k, int shift) {
    return ((uint32_t)k >> shift) & (kRadixBins - 1);
}

__global__ __launch_bounds__(kSortThreads) void k_split(const int64_t* __restrict__ idx,
                                                        const int64_t* __restrict__ off, int64_t L,
                                                        int64_t TB, int64_t B,
                                                        const TabDev* __restrict__ desc,
                                                        int32_t* __restrict__ key, int32_t* __restrict__ i3o,
                                                        int32_t* __restrict__ bag_of,
                                                        int32_t* __restrict__ bag_start,
                                                        int32_t* __restrict__ ckey, int32_t M3,
                                                        int32_t* ctrl, int32_t* __restrict__ key_start,
                                                        int64_t K, int32_t* __restrict__ i3cnt, int32_t n3cnt,
                                                        int64_t n_tiles, int64_t hstride,
                                                        uint32_t* __restrict__ hist,
                                                        const int64_t* __restrict__ hot_keys,
                                                        const int32_t* __restrict__ hot_slots, int hot_lg,
                                                        int32_t* __restrict__ cslot) {
    __shared__ uint32_t cnt[kSortWaves][kRadixBins];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int64_t)blockIdx.x >= n_tiles) {
        const int64_t x = blockIdx.x - n_tiles;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const int64_t i = x * kSortTile + j * kSortThreads + threadIdx.x;
            if (i < K) key_start[i] = -1;              // k_gather records each present key's first position
            if (i < n3cnt) i3cnt[i * kI3Pad] = 0;       // k_runs counts the runs of each bucket
        }
        const int64_t q0 = x * kSortThreads + 64 * w;   // this wave's bags q0 .. q0+63
        if (q0 > TB) return;   // wave-uniform
        const int64_t i = q0 + lane;
        const int64_t x0 = off[i < TB ? i : TB], x1 = off[i < TB ? i + 1 : TB];
        int64_t a = L, an = L;   // bag i's offset and the next one, clamped into [0, L]
        if (i <= TB) {
            a = x0 < 0 ? 0 : (x0 > L ? L : x0);
            bag_start[i] = (int32_t)a;
            const int64_t xn = i < TB ? x1 : L;
            an = xn < 0 ? 0 : (xn > L ? L : xn);
            const bool bad = (i == 0 && x0 != 0) || (i == TB && x0 != L) || (i < TB && xn < x0);
            if (bad) atomicOr(&ctrl[CTRL_FLAG], TT_FLAG_BAD_OFFSETS);
        }
        if (q0 >= TB) return;
        // lookups [lo, hi) belong to these bags (bags past TB start at L)
        const int32_t o = (int32_t)a;
        const int32_t lo = __builtin_amdgcn_readfirstlane(o);
        const int32_t hi = __builtin_amdgcn_readlane((int32_t)an, 63);
        for (int32_t l0 = lo; l0 < hi; l0 += 64) {
            const int32_t l = l0 + lane;
            int jj = 0;   // last lane whose offset is <= l (lane 0's is lo <= l)
#pragma unroll
            for (int st = 32; st >= 1; st >>= 1) {
                const int32_t y = __shfl(o, jj + st);
                if (y <= l) jj += st;
            }
            if (l < hi) bag_of[l] = (int32_t)(q0 + jj);
        }
        return;
    }
    const int64_t tile = blockIdx.x;
    for (int i = lane; i < kRadixBins; i += 64) cnt[w][i] = 0;   // own row, so no barrier
    // lookups: wave w takes the w-th sixteenth of the tile, 64 at a time;
    // every index load is issued before the first is used
    const int64_t T = TB / B;
    const int64_t base = tile * kSortTile + (int64_t)w * (kSortTile / kSortWaves);
    int64_t xv[kSortItems];
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const int64_t e = base + slot * 64 + lane;
        xv[slot] = idx[e < L ? e : L - 1];   // L > 0: there is a lookup tile
    }

    // one lookup: its key, sort key and i3 (a bad index reads as row 0), and
    // with a hot-row cache its row's slot
    auto split_one = [&](int64_t e, int64_t x, const TabDev& dd, int64_t t) {
        if (x < 0 || x >= dd.N) {
            atomicOr(&ctrl[CTRL_FLAG], TT_FLAG_BAD_INDEX);
            x = 0;
        }
        if (cslot) cslot[e] = cache_probe(hot_keys, hot_slots, hot_lg, (t << 40) | x);
        const uint32_t xi = (uint32_t)x;
        const uint32_t r3 = xi % (uint32_t)dd.m3;
        const uint32_t p = xi / (uint32_t)dd.m3;
        const uint32_t r2 = p % (uint32_t)dd.m2;
        const uint32_t r1 = p / (uint32_t)dd.m2;
        const int32_t k = dd.key_base + (int32_t)(r2 * (uint32_t)dd.m1 + r1);
        const int32_t ck = k * M3 + (int32_t)r3;
        key[e] = k;
        ckey[e] = ck;
        i3o[e] = (int32_t)r3;
        return sort_digit(ck, 0);
    };
    uint32_t dg[kSortItems];
    // the tables of the tile's first and last lookups: the number of table
    // starts (tables 1 .. T-1) at or before each (every thread counts a
    // share, added across the block); when they agree, every lookup of the
    // tile is in that table
    int64_t tu = 0;   // the tile's table, or -1: the tile spans tables
    if (T > 1) {
        __shared__ int32_t sTab[2];
        if (threadIdx.x == 0) { sTab[0] = 0; sTab[1] = 0; }
        __syncthreads();
        const int64_t ef = tile * kSortTile, el = min<int64_t>(L, ef + kSortTile) - 1;
        int32_t cf = 0, cl = 0;
        for (int64_t t = 1 + threadIdx.x; t < T; t += kSortThreads) {
            const int64_t st = off[t * B];
            cf += st <= ef ? 1 : 0;
            cl += st <= el ? 1 : 0;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            cf += __shfl_xor(cf, m);
            cl += __shfl_xor(cl, m);
        }
        if (lane == 0 && (cf | cl)) { atomicAdd(&sTab[0], cf); atomicAdd(&sTab[1], cl); }
        __syncthreads();
        tu = sTab[0] == sTab[1] ? sTab[0] : -1;
    }
    if (tu >= 0) {   // one table for the whole tile: its descriptor read once (uniform)
        const TabDev d0 = desc[tu];
#pragma unroll
        for (int slot = 0; slot < kSortItems; ++slot) {
            const int64_t e = base + slot * 64 + lane;
            dg[slot] = e < L ? split_one(e, xv[slot], d0, tu) : 0u;
        }
    } else {
#pragma unroll
        for (int slot = 0; slot < kSortItems; ++slot) {
            const int64_t e = base + slot * 64 + lane;
            dg[slot] = 0u;
            if (e < L) {
                // table of lookup e: last t with off[t*B] <= e (in range for any offsets)
                int64_t lo = 0, hi = T;
                while (hi - lo > 1) {
                    const int64_t mid = (lo + hi) >> 1;
                    if (off[mid * B] <= e) lo = mid; else hi = mid;
                }
                dg[slot] = split_one(e, xv[slot], desc[lo], lo);
            }
        }
    }
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const bool valid = base + slot * 64 + lane < L;
        const uint64_t peers = match_digit(dg[slot], __ballot(valid));
        if (valid && popc_below(peers) == 0) cnt[w][dg[slot]] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kRadixBins; i += kSortThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) c += cnt[ww][i];
        hist[(int64_t)i * hstride + tile] = c;
    }
    if (tile == n_tiles - 1) {
        const int64_t pad = hstride - n_tiles;
        for (int64_t i = threadIdx.x; i < pad * kRadixBins; i += kSortThreads)
            hist[(i / pad) * hstride + n_tiles + i % pad] = 0u;
    }
}

// ---------------------------------------------------------------------------
// stable LSD radix sort
//
// A tile is kSortTile consecutive elements; wave w of its workgroup takes the
// w-th sixteenth, 64 at a time, so ranks in (wave, slot, lane) order are ranks
// in sequence order. Digit counts are kept per wave (no LDS atomics: in a
// slot, one leader lane per distinct digit adds its peers' count).

// Per-tile digit counts: hist[d * hstride + tile]; the last tile also zeroes
// the padding columns [n_tiles, hstride).
__global__ __launch_bounds__(kSortThreads) void k_radix_hist(const int32_t* __restrict__ keys,
                                                             int64_t L, int shift, int64_t n_tiles,
                                                             int64_t hstride, uint32_t* __restrict__ hist) {
    __shared__ uint32_t cnt[kSortWaves][kRadixBins];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = lane; i < kRadixBins; i += 64) cnt[w][i] = 0;   // own row, so no barrier
    const int64_t tile = blockIdx.x;
    const int64_t base = tile * kSortTile + (int64_t)w * (kSortTile / kSortWaves);
    uint32_t d[kSortItems];
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const int64_t e = base + slot * 64 + lane;
        d[slot] = e < L ? sort_digit(keys[e], shift) : 0u;
    }
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const bool valid = base + slot * 64 + lane < L;
        const uint64_t peers = match_digit(d[slot], __ballot(valid));
        if (valid && popc_below(peers) == 0) cnt[w][d[slot]] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kRadixBins; i += kSortThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) c += cnt[ww][i];
        hist[(int64_t)i * hstride + tile] = c;
    }
    if (tile == n_tiles - 1) {
        const int64_t pad = hstride - n_tiles;
        for (int64_t i = threadIdx.x; i < pad * kRadixBins; i += kSortThreads)
            hist[(i / pad) * hstride + n_tiles + i % pad] = 0u;
    }
}

// Scatter of one tile. The tile's elements are first placed in LDS in their
// output order (by digit, stable), then written out with consecutive threads
// on consecutive output positions, so each digit's run is one coalesced
// stretch. DIRECT: the workgroup forms its digits' global bases from the raw
// per-tile counts (digit start = counts of all smaller digits, plus this
// digit's counts in earlier tiles); otherwise hist holds the exclusive scan of
// the counts in digit-major order.
//
// Each element carries its lookup and its bag. The first pass (vin null)
// takes the lookup from the position and the bag from bin = bag_of, clamped
// into [0, TB) (bad offsets can leave lookups unlabelled).
template <bool DIRECT>
__global__ __launch_bounds__(kSortThreads) void k_radix_scatter(
    const int32_t* __restrict__ kin, const int32_t* __restrict__ vin, const int32_t* __restrict__ bin,
    int64_t L, int32_t TB, int shift, int64_t hstride, const uint32_t* __restrict__ hist,
    int32_t* __restrict__ kout, int32_t* __restrict__ vout, int32_t* __restrict__ bout) {
    __shared__ uint32_t cnt[kSortWaves][kRadixBins];
    __shared__ int32_t sk[kSortTile], sv[kSortTile], sb[kSortTile];
    __shared__ uint32_t gpre[kRadixBins];    // digit's count in earlier tiles (DIRECT) or global base
    __shared__ uint32_t gtot[kRadixBins];    // digit's count in all tiles (DIRECT)
    __shared__ uint32_t lbase[kRadixBins];   // digit's first position in the tile's output order
    __shared__ int32_t delta[kRadixBins];    // global position - tile position, per digit
    __shared__ uint32_t wsum[2][kRadixBins / 64];
    const int64_t tile = blockIdx.x;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = lane; i < kRadixBins; i += 64) cnt[w][i] = 0;
    // this tile's elements, all loads in flight at once
    const int64_t base = tile * kSortTile + (int64_t)w * (kSortTile / kSortWaves);
    int32_t kk[kSortItems], vv[kSortItems], bb[kSortItems];
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const int64_t e = base + slot * 64 + lane;
        const bool valid = e < L;
        kk[slot] = valid ? kin[e] : 0;
        vv[slot] = valid ? (vin ? vin[e] : (int32_t)e) : 0;
        bb[slot] = valid ? bin[e] : 0;
        if (!vin) bb[slot] = min(max(bb[slot], 0), TB - 1);
    }
    if (DIRECT) {
        // LPD lanes per digit, each sums every LPD-th 16-byte piece of the
        // digit's row
        constexpr int LPD = kSortThreads / kRadixBins;
        static_assert(LPD >= 1 && (LPD & (LPD - 1)) == 0 && LPD <= 64, "lanes per digit");
        const int dg = threadIdx.x / LPD, part = threadIdx.x % LPD;
        const uint4* row = reinterpret_cast<const uint4*>(hist + (int64_t)dg * hstride);
        const int64_t n4 = hstride / 4;
        uint32_t pre = 0, tot = 0;
        for (int64_t v0 = part; v0 < n4; v0 += 8 * LPD) {   // eight loads in flight per lane
            uint4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = v0 + LPD * u < n4 ? row[v0 + LPD * u] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t t0 = 4 * (v0 + LPD * u);
                const uint32_t c[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    tot += c[j];
                    if (t0 + j < tile) pre += c[j];
                }
            }
        }
#pragma unroll
        for (int o = 1; o < LPD; o <<= 1) {
            pre += __shfl_xor(pre, o);
            tot += __shfl_xor(tot, o);
        }
        if (part == 0) {
            gpre[dg] = pre;
            gtot[dg] = tot;
        }
    } else {
        for (int i = threadIdx.x; i < kRadixBins; i += kSortThreads) gpre[i] = hist[(int64_t)i * hstride + tile];
    }
    // stable ranks inside the tile, per wave
    uint32_t rk[kSortItems];
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const bool valid = base + slot * 64 + lane < L;
        const uint32_t d = sort_digit(kk[slot], shift);
        const uint64_t peers = match_digit(d, __ballot(valid));
        const uint32_t below = popc_below(peers);
        uint32_t pre = 0;
        if (valid) pre = cnt[w][d];
        if (valid && below == 0) cnt[w][d] = pre + (uint32_t)__popcll(peers);
        rk[slot] = pre + below;
    }
    __syncthreads();
    // per digit (threads 0..255, waves 0..3): exclusive prefix over the waves,
    // then exclusive scans over the digits of the tile counts and (DIRECT) of
    // the all-tile counts
    uint32_t linc = 0, lcnt = 0, tinc = 0, tcnt = 0;
    if (threadIdx.x < kRadixBins) {
        const int dg = threadIdx.x;
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) {
            const uint32_t c = cnt[ww][dg];
            cnt[ww][dg] = lcnt;
            lcnt += c;
        }
        linc = lcnt;
        if (DIRECT) tinc = tcnt = gtot[dg];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(linc, o, 64);
            const uint32_t z = __shfl_up(tinc, o, 64);
            if (lane >= o) {
                linc += y;
                tinc += z;
            }
        }
        if (lane == 63) {
            wsum[0][w] = linc;
            wsum[1][w] = tinc;
        }
    }
    __syncthreads();
    if (threadIdx.x < kRadixBins) {
        uint32_t lo = 0, to = 0;
        for (int ww = 0; ww < w; ++ww) {
            lo += wsum[0][ww];
            to += wsum[1][ww];
        }
        const uint32_t lb = lo + linc - lcnt;
        const uint32_t gb = DIRECT ? to + tinc - tcnt + gpre[threadIdx.x] : gpre[threadIdx.x];
        lbase[threadIdx.x] = lb;
        delta[threadIdx.x] = (int32_t)(gb - lb);
    }
    __syncthreads();
    // place in output order inside the tile
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        if (base + slot * 64 + lane < L) {
            const uint32_t d = sort_digit(kk[slot], shift);
            const uint32_t lp = lbase[d] + cnt[w][d] + rk[slot];
            if (lp < (uint32_t)kSortTile) {   // always, as above
                sk[lp] = kk[slot];
                sv[lp] = vv[slot];
                sb[lp] = bb[slot];
            }
        }
    }
    __syncthreads();
    const int64_t nt = min<int64_t>(kSortTile, L - tile * kSortTile);
    for (int i = threadIdx.x; i < nt; i += kSortThreads) {
        const int32_t k = sk[i];
        const int64_t pos = (int64_t)delta[sort_digit(k, shift)] + i;
        if (pos >= 0 && pos < L) {   // always, when the counts are consistent
            kout[pos] = k;
            vout[pos] = sv[i];
            bout[pos] = sb[i];
        }
    }
}

// ---------------------------------------------------------------------------
// device-wide exclusive scan (single block for short arrays, else single-pass look-back)

template <class V>
__device__ V block_exclusive_scan(V x, V* wsum, V* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    V inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const V y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    if (w == 0) {
        const V v = lane < nw ? wsum[lane] : V(0);
        V s = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const V y = __shfl_up(s, o, 64);
            if (lane >= o) s += y;
        }
        if (lane < nw) wsum[lane] = s - v;
        if (lane == nw - 1) wsum[16] = s;
    }
    __syncthreads();
    const V r = wsum[w] + inc - x;
    *total = wsum[16];
    __syncthreads();
    return r;
}

template <class V>
__global__ __launch_bounds__(kScanThreads) void k_scan_single(V* data, int64_t n, V* total_out) {
    __shared__ V wsum[17];
    V carry = 0;
    for (int64_t base = 0; base < n; base += kScanTile) {
        const int64_t i0 = base + (int64_t)threadIdx.x * kScanItems;
        V v[kScanItems];
        V s = 0;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            v[k] = (i0 + k < n) ? data[i0 + k] : V(0);
            s += v[k];
        }
        V tot;
        V run = carry + block_exclusive_scan<V>(s, wsum, &tot);
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            if (i0 + k < n) data[i0 + k] = run;
            run += v[k];
        }
        carry += tot;
    }
    if (threadIdx.x == 0 && total_out) *total_out = carry;
}

// Single-pass scan of arrays longer than one block's share: decoupled look-back
// (Merrill and Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back"). A workgroup claims the next tile from a counter, scans it,
// publishes the tile's total, then walks back over the earlier tiles' status
// words 64 at a time (one wave, one word per lane), adding totals until it
// meets a tile whose inclusive prefix is known, and publishes its own
// inclusive prefix. Status words carry the scan's epoch
// (one per scan of a plan) so they need no clearing between scans; the plan's
// control-word fill clears them once. Each wait is bounded: past the bound the
// workgroup raises TT_FLAG_INTERNAL and goes on (wrong sums, never a hang).
constexpr int kLookbackSpins = 1 << 20;

template <class V>
__global__ __launch_bounds__(kScanThreads) void k_scan_lookback(V* data, int64_t n, ScanTileStatus* st,
                                                                uint32_t* tile_ctr, uint32_t epoch,
                                                                V* total_out, int32_t* ctrl) {
    __shared__ V wsum[17];
    __shared__ uint32_t s_tile;
    __shared__ V s_prefix;
    if (threadIdx.x == 0) s_tile = atomicAdd(tile_ctr, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const int64_t i0 = (int64_t)tile * kScanTile + (int64_t)threadIdx.x * kScanItems;
    V v[kScanItems];
    V sum = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        v[k] = (i0 + k < n) ? data[i0 + k] : V(0);
        sum += v[k];
    }
    V tot;
    V run = block_exclusive_scan<V>(sum, wsum, &tot);
    if (threadIdx.x < 64) {
        // wave 0: publish the tile's total, then look back 64 tiles at a time
        const int lane = threadIdx.x;
        // the value goes out as a device-scope store and has completed before
        // the flag does (a wait, not a device-scope release fence, which
        // would write back the whole L2)
        auto publish = [&](uint32_t state, V x) {
            __hip_atomic_store(state == 2u ? &st[tile].incl : &st[tile].agg, (uint64_t)x, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            wait_vmem_done();
            __hip_atomic_store(&st[tile].flag, (epoch << 2) | state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        V prefix = 0;
        if (tile > 0) {
            if (lane == 0) publish(1u, tot);
            int64_t top = (int64_t)tile - 1;   // nearest tile of the window
            int spins = 0;
            while (true) {
                const int64_t j = top - lane;
                uint32_t f = 0;
                if (j >= 0) f = __hip_atomic_load(&st[j].flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const bool mine = (f >> 2) == epoch;
                const uint32_t state = mine ? (f & 3u) : 0u;
                const uint64_t incl = __ballot(j >= 0 && state == 2u);
                const int first = incl ? __ffsll((unsigned long long)incl) - 1 : 64;   // nearest inclusive
                const uint64_t need = first == 64 ? ~0ull : ((1ull << first) - 1ull);
                const uint64_t waiting = __ballot(j >= 0 && state == 0u) & need;
                if (waiting) {
                    if (++spins > kLookbackSpins) {
                        if (lane == 0) atomicOr(ctrl + CTRL_FLAG, TT_FLAG_INTERNAL);
                        break;
                    }
                    continue;
                }
                // values read after their flags (device-scope loads)
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                V c = 0;
                if (j >= 0 && lane < first)
                    c = (V)__hip_atomic_load(&st[j].agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (lane == first) c = (V)__hip_atomic_load(&st[j].incl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
                prefix += c;
                if (first < 64 || top < 64) break;
                top -= 64;
            }
        }
        if (lane == 0) {
            publish(2u, prefix + tot);
            s_prefix = prefix;
            if (total_out && (int64_t)(tile + 1) * kScanTile >= n) *total_out = prefix + tot;
        }
    }
    __syncthreads();
    run += s_prefix;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        if (i0 + k < n) data[i0 + k] = run;
        run += v[k];
    }
}

// Exclusive scan in place, one launch: one workgroup for short arrays, the
// single-pass scan otherwise. `seq` numbers the plan's scans from 1.
template <class V>
static tt_status scan_exclusive(const tt_emb_plan_s* p, int seq, V* data, int64_t n, V* total_out,
                                hipStream_t s) {
    if (n <= 4 * (int64_t)kScanTile) {
        TT_LAUNCH(p, "k_scan_single", s, k_scan_single<V>, dim3(1), dim3(kScanThreads), 0, s, data, n, total_out);
        TT_LAUNCH_CHECK();
        return TT_OK;
    }
    const int64_t nb = (n + kScanTile - 1) / kScanTile;
    if (seq < 1 || seq >= CTRL_SCAN_MAX || nb > p->lay.scan_tiles) return TT_ERR_UNSUPPORTED;
    TT_LAUNCH(p, "k_scan_lookback", s, k_scan_lookback<V>, dim3((unsigned)nb), dim3(kScanThreads), 0, s, data, n,
                       p->at<ScanTileStatus>(p->lay.scan_st),
                       reinterpret_cast<uint32_t*>(p->ctrl() + CTRL_SCAN_CTR + seq), (uint32_t)seq,
                       total_out, p->ctrl());
    TT_LAUNCH_CHECK();
    return TT_OK;
}

// ---------------------------------------------------------------------------
// groups and chunks
//
// The position-indexed passes below work on tiles of kSortTile sorted
// positions (one workgroup each) and the key-indexed ones on tiles of
// kSortTile keys. A counting pass leaves one total per tile; the pass that
// needs the exclusive scan adds up the earlier tiles' totals itself (DIRECT,
// up to kDirectTiles tiles) or reads them from a device-wide scan of the
// tile totals, and scans inside its tile.

// Sum of tsum[0, tile) (DIRECT, tile <= kDirectTiles) or the scanned tsum[tile],
// by wave 0, into *out (LDS); the caller synchronises before reading it.
template <bool DIRECT, class V>
__device__ __forceinline__ void tile_base(const V* __restrict__ tsum, int64_t tile, V* out) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    V x = 0;
    if (DIRECT) {
#pragma unroll
        for (int j = 0; j < (int)(kDirectTiles / 64); ++j) {
            const int64_t u = lane + 64 * j;
            if (u < tile) x += tsum[u];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    } else {
        x = tsum[tile];
    }
    if (lane == 0) *out = x;
}

// Per sorted position: sorted i3 (from the sort key), first and last
// position of each key; per tile: the number of row-run heads (a row run is a
// maximal stretch of one (key, i3) row in sorted order).
__global__ __launch_bounds__(kSortThreads) void k_gather(const int32_t* __restrict__ skey, int64_t L,
                                                         int32_t M3, int32_t* __restrict__ sorted_i3,
                                                         int32_t* __restrict__ key_start,
                                                         int32_t* __restrict__ key_end,
                                                         uint32_t* __restrict__ run_tiles) {
    __shared__ uint32_t wc[kSortWaves];
    const int64_t tile = blockIdx.x;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t heads = 0;
#pragma unroll
    for (int slot = 0; slot < kSortItems; ++slot) {
        const int64_t s = tile * kSortTile + slot * kSortThreads + threadIdx.x;
        if (s < L) {
            const int32_t ck = skey[s];
            const int32_t prev = s > 0 ? skey[s - 1] : -1;
            const int32_t next = s + 1 < L ? skey[s + 1] : -1;
            const int32_t k = ck / M3;
            sorted_i3[s] = ck - k * M3;
            heads += (s == 0 || prev != ck) ? 1u : 0u;
            if (s == 0 || prev / M3 != k) key_start[k] = (int32_t)s;
            if (s + 1 == L || next / M3 != k) key_end[k] = (int32_t)(s + 1);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) heads += __shfl_xor(heads, o);
    if (lane == 0) wc[w] = heads;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kSortWaves; ++i) t += wc[i];
        run_tiles[tile] = t;
    }
}

// Per key: (present << 32) | number of chunks (0 when absent).
__device__ __forceinline__ uint64_t key_word(const int32_t* __restrict__ key_start,
                                             const int32_t* __restrict__ key_end, int64_t k, int64_t K,
                                             int32_t chunk) {
    if (k >= K) return 0;
    const int32_t st = key_start[k];
    if (st < 0) return 0;
    return (uint64_t(1) << 32) | (uint32_t)((key_end[k] - st + chunk - 1) / chunk);
}

// Per tile of keys: the sum of the key words (present keys, chunks).
__global__ __launch_bounds__(kSortThreads) void k_key_tiles(const int32_t* __restrict__ key_start,
                                                            const int32_t* __restrict__ key_end, int64_t K,
                                                            int32_t chunk, uint64_t* __restrict__ key_tiles) {
    __shared__ uint64_t wc[kSortWaves];
    const int64_t tile = blockIdx.x;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint64_t v = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j)
        v += key_word(key_start, key_end, tile * kSortTile + j * kSortThreads + threadIdx.x, K, chunk);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) wc[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int i = 0; i < kSortWaves; ++i) t += wc[i];
        key_tiles[tile] = t;
    }
}

// Per key: key_scan[k] = exclusive scan of the key words (group id << 32 |
// first chunk); group tables for the present keys; the last tile writes the
// totals (groups, chunks) and the closing entries of the group tables.
template <bool DIRECT>
__global__ __launch_bounds__(kSortThreads) void k_groups(const int32_t* __restrict__ key_start,
                                                         const int32_t* __restrict__ key_end, int64_t K,
                                                         int64_t L, int32_t chunk,
                                                         const uint64_t* __restrict__ key_tiles,
                                                         uint64_t* __restrict__ key_scan,
                                                         int32_t* __restrict__ group_key,
                                                         int32_t* __restrict__ group_start,
                                                         int32_t* __restrict__ group_cbase, int32_t* ctrl) {
    __shared__ uint64_t wsum[17];
    __shared__ uint64_t sbase;
    const int64_t tile = blockIdx.x;
    tile_base<DIRECT, uint64_t>(key_tiles, tile, &sbase);
    // thread t takes keys 4t .. 4t+3 of the tile
    const int64_t k0 = tile * kSortTile + (int64_t)threadIdx.x * kSortItems;
    uint64_t v[kSortItems];
    uint64_t sum = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        v[j] = key_word(key_start, key_end, k0 + j, K, chunk);
        sum += v[j];
    }
    uint64_t tot;
    uint64_t run = block_exclusive_scan<uint64_t>(sum, wsum, &tot);   // synchronises
    run += sbase;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t k = k0 + j;
        if (k < K) {
            key_scan[k] = run;
            if (v[j]) {
                const int32_t g = (int32_t)(run >> 32);
                const int32_t c0 = (int32_t)(run & 0xffffffffu);
                group_key[g] = (int32_t)k;
                group_start[g] = key_start[k];
                group_cbase[g] = c0;
            }
        }
        run += v[j];
    }
    if (tile == (int64_t)gridDim.x - 1 && threadIdx.x == 0) {
        const uint64_t all = sbase + tot;
        const int32_t U = (int32_t)(all >> 32), NC = (int32_t)(all & 0xffffffffu);
        ctrl[CTRL_NUM_GROUPS] = U;
        ctrl[CTRL_NUM_CHUNKS] = NC;
        group_start[U] = (int32_t)L;
        group_cbase[U] = NC;
    }
}

// The table holding both `first` and `last`, values of a per-table start
// field that grows with the table index (key_base, fb_base), or -1 when they
// lie in different tables: the number of starts of tables 1 .. T-1 at or
// before each, counted by every thread of the block (the block's threads all
// call it; it synchronises the block).
template <class Start>
__device__ int32_t block_table_of(const TabDev* __restrict__ desc, int32_t T, int64_t first, int64_t last,
                                  Start start) {
    if (T <= 1) return 0;
    __shared__ int32_t sTab[2];
    if (threadIdx.x == 0) { sTab[0] = 0; sTab[1] = 0; }
    __syncthreads();
    int32_t cf = 0, cl = 0;
    for (int64_t t = 1 + threadIdx.x; t < T; t += blockDim.x) {
        const int64_t st = start(desc[t]);
        cf += st <= first ? 1 : 0;
        cl += st <= last ? 1 : 0;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        cf += __shfl_xor(cf, m);
        cl += __shfl_xor(cl, m);
    }
    if ((threadIdx.x & 63) == 0 && (cf | cl)) { atomicAdd(&sTab[0], cf); atomicAdd(&sTab[1], cl); }
    __syncthreads();
    const int32_t a = sTab[0], b = sTab[1];
    __syncthreads();   // sTab is free for the next call
    return a == b ? a : -1;
}

// G3 row of a run of key k and digit i3: its table's first G3 row plus i3
// (tu >= 0: the caller knows the table).
__device__ __forceinline__ int32_t bucket3(const TabDev* __restrict__ desc, int32_t T, int32_t CN, int32_t k,
                                           int32_t i3, int32_t tu = -1) {
    int lo = tu;
    if (lo < 0) {
        lo = 0;
        int hi = T;   // last table with key_base <= k
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (desc[mid].key_base <= k) lo = mid; else hi = mid;
        }
    }
    return (int32_t)(desc[lo].o3 / CN) + i3;
}

// Row-run ids and tables over one tile of sorted positions (rid[s] = number
// of row-run heads before s), and the chunk table: position s opens a chunk
// when it lies a multiple of `chunk` past its group's start (chunk c of group
// g starts `chunk` lookups after the previous one of g).
// Forward batch slot b (layer-major): its table, slice and layer, and the
// slice's groups [gs0, gs1).
struct SlotOf {
    TabDev d;
    int32_t i2, jb, gs0, gs1;
    int32_t cls;   // XCD class: the slice's global index mod kXcds
    int64_t kb;
};
__device__ __forceinline__ SlotOf slot_of(const TabDev* __restrict__ desc, int32_t T, int64_t K, int64_t b,
                                          const uint64_t* __restrict__ key_scan, const int32_t* __restrict__ ctrl,
                                          int32_t tu = -1) {
    int lo = tu;
    if (lo < 0) {
        lo = 0;
        int hi = T;   // last table with fb_base <= b
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (desc[mid].fb_base <= b) lo = mid; else hi = mid;
        }
    }
    SlotOf o;
    o.d = desc[lo];
    o.i2 = (int32_t)((b - o.d.fb_base) % o.d.m2);
    o.jb = (int32_t)((b - o.d.fb_base) / o.d.m2);
    o.kb = (int64_t)o.d.key_base + (int64_t)o.i2 * o.d.m1;
    const int64_t ke = o.kb + o.d.m1;
    o.gs0 = (int32_t)(key_scan[o.kb] >> 32);
    o.gs1 = ke < K ? (int32_t)(key_scan[ke] >> 32) : ctrl[CTRL_NUM_GROUPS];
    o.cls = (o.d.i2_base + o.i2) % kXcds;
    return o;
}

template <bool DIRECT>
__global__ __launch_bounds__(kSortThreads) void k_runs(const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ skey,
                                                       const uint64_t* __restrict__ key_scan,
                                                       const int32_t* __restrict__ key_start,
                                                       const int32_t* __restrict__ key_end,
                                                       const uint32_t* __restrict__ run_tiles,
                                                       int64_t L, int32_t M3, int32_t chunk, int32_t* ctrl,
                                                       int32_t* __restrict__ rid,
                                                       int32_t* __restrict__ run_i3,
                                                       int32_t* __restrict__ run_of,
                                                       int32_t* __restrict__ run_start,
                                                       int32_t* __restrict__ group_rbase,
                                                       int32_t* __restrict__ chunk_group,
                                                       int32_t* __restrict__ chunk_begin,
                                                       int32_t* __restrict__ chunk_end,
                                                       int32_t* __restrict__ i3cnt, int32_t n3cnt,
                                                       int32_t* __restrict__ run_rank,
                                                       int32_t* __restrict__ run_bkt,
                                                       const TabDev* __restrict__ desc, int32_t T, int32_t CN,
                                                       int64_t K, int64_t NFB,
                                                       uint32_t* __restrict__ batch_tiles,
                                                       const int32_t* __restrict__ cslot,
                                                       int32_t* __restrict__ run_cslot,
                                                       const int32_t* __restrict__ sorted_bag,
                                                       int32_t* __restrict__ run_bag1) {
    __shared__ uint32_t sh3[kMaxBuckets3];
    for (int i = threadIdx.x; i < n3cnt; i += kSortThreads) sh3[i] = 0u;   // ordered by the scan's barriers
    const int64_t tile = blockIdx.x;
    __shared__ uint32_t wsum[17];
    __shared__ uint32_t sbase;
    tile_base<DIRECT, uint32_t>(run_tiles, tile, &sbase);
    // thread t takes positions 4t .. 4t+3 of the tile
    const int64_t s0 = tile * kSortTile + (int64_t)threadIdx.x * kSortItems;
    // ck[j + 1] = key at position s0 + j, ck[0] the one before, ck[kSortItems + 1]
    // the one after (-1 outside [0, L))
    int32_t ck[kSortItems + 2];
    ck[0] = s0 > 0 && s0 <= L ? skey[s0 - 1] : -1;
#pragma unroll
    for (int j = 0; j <= kSortItems; ++j) ck[j + 1] = s0 + j < L ? skey[s0 + j] : -1;
    uint32_t hr[kSortItems], sum = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        hr[j] = (s0 + j < L && (s0 + j == 0 || ck[j] != ck[j + 1])) ? 1u : 0u;
        sum += hr[j];
    }
    // the tile's keys lie in one table (usually): its index for the G3 rows
    const int32_t tuk = n3cnt ? block_table_of(desc, T, skey[tile * kSortTile] / M3,
                                               skey[min<int64_t>(L, (tile + 1) * kSortTile) - 1] / M3,
                                               [](const TabDev& d) { return (int64_t)d.key_base; })
                              : -1;
    // every per-position load goes out before the scan's barriers: the
    // lookup, its key's first and last position and scan word (a position
    // past L reads key 0's), and with a hot-row cache the lookup's slot
    int32_t pl[kSortItems], kst[kSortItems], kend[kSortItems], csv[kSortItems];
    uint64_t ksc[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t s = min(s0 + j, L - 1);
        const int32_t k = max(ck[j + 1], 0) / M3;
        pl[j] = perm[s];
        kst[j] = key_start[k];
        kend[j] = key_end[k];
        ksc[j] = key_scan[k];
    }
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) csv[j] = cslot ? cslot[pl[j]] : -1;
    int32_t sbg[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) sbg[j] = run_bag1 ? sorted_bag[min(s0 + j, L - 1)] : 0;
    uint32_t tot;
    uint32_t run = block_exclusive_scan<uint32_t>(sum, wsum, &tot) + sbase;   // synchronises
    uint32_t lrank[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t s = s0 + j;
        if (s < L) {
            const int32_t rr = (int32_t)run;   // heads before s
            rid[s] = rr;
            const int32_t k = ck[j + 1] / M3;
            if (hr[j]) {
                const int32_t r3 = ck[j + 1] - k * M3;
                run_i3[rr] = r3;
                run_start[rr] = (int32_t)s;
                if (run_bag1) run_bag1[rr] = ck[j + 2] != ck[j + 1] ? sbg[j] : -1;   // one lookup: its bag
                if (n3cnt) lrank[j] = atomicAdd(&sh3[bucket3(desc, T, CN, k, r3, tuk)], 1u);   // rank in the tile
            }
            int32_t ro = rr + (int32_t)hr[j] - 1;
            if (cslot) {   // a hot row's lookups: -(slot + 1), its run: the slot
                if (hr[j]) run_cslot[rr] = csv[j];
                if (csv[j] >= 0) ro = -(csv[j] + 1);
            }
            run_of[pl[j]] = ro;
            const int32_t off = (int32_t)s - kst[j];
            if (off % chunk == 0) {
                const uint64_t ks = ksc[j];
                const int32_t g = (int32_t)(ks >> 32);
                const int32_t c = (int32_t)(ks & 0xffffffffu) + off / chunk;
                chunk_group[c] = g;
                chunk_begin[c] = (int32_t)s;
                chunk_end[c] = min((int32_t)s + chunk, kend[j]);
                if (off == 0) group_rbase[g] = rr;
            }
            if (s == L - 1) {
                ctrl[CTRL_NUM_RUNS] = rr + (int32_t)hr[j];
                group_rbase[ctrl[CTRL_NUM_GROUPS]] = rr + (int32_t)hr[j];
            }
        }
        run += hr[j];
    }
    if (n3cnt) {
        // one counter claim per (tile, i3): the tile's runs of i3 take the
        // next sh3[i3] ranks of the bucket (buckets fill in any tile order)
        __syncthreads();
        for (int i = threadIdx.x; i < n3cnt; i += kSortThreads)
            if (sh3[i]) sh3[i] = (uint32_t)atomicAdd(i3cnt + (int64_t)i * kI3Pad, (int32_t)sh3[i]);
        __syncthreads();
        uint32_t r = run - sum;   // heads before this thread's first position
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            if (s0 + j < L && hr[j]) {
                const int32_t k = ck[j + 1] / M3;
                const int32_t b = bucket3(desc, T, CN, k, ck[j + 1] - k * M3, tuk);
                run_rank[r] = (int32_t)(sh3[b] + lrank[j]);
                run_bkt[r] = b;
            }
            r += hr[j];
        }
    }
    // forward batch slots holding a group, per tile of kSlotTile slots and
    // XCD class (the group tables are complete: k_groups ran before);
    // kSortThreads slots per round, counted in LDS
    constexpr int TPR = kSortThreads / kSlotTile;
    static_assert(kSortThreads % kSlotTile == 0, "slot tiles");
    __shared__ uint32_t ccnt[TPR][kXcds];
    const int64_t nst = (NFB + kSlotTile - 1) / kSlotTile;
    for (int64_t jt0 = (int64_t)blockIdx.x * TPR; jt0 < nst; jt0 += (int64_t)gridDim.x * TPR) {
        if (threadIdx.x < TPR * kXcds) ccnt[threadIdx.x / kXcds][threadIdx.x % kXcds] = 0u;
        const int64_t b = jt0 * kSlotTile + threadIdx.x;
        const int32_t tus = block_table_of(desc, T, jt0 * kSlotTile, min<int64_t>(NFB, (jt0 + TPR) * kSlotTile) - 1,
                                           [](const TabDev& d) { return (int64_t)d.fb_base; });
        __syncthreads();   // ccnt cleared
        if (b < NFB) {
            const SlotOf o = slot_of(desc, T, K, b, key_scan, ctrl, tus);
            if (o.gs1 - (o.gs0 + kFwdBatch * o.jb) > 0) atomicAdd(&ccnt[threadIdx.x / kSlotTile][o.cls], 1u);
        }
        __syncthreads();
        if (threadIdx.x < TPR * kXcds && jt0 + threadIdx.x / kXcds < nst)
            batch_tiles[(jt0 + threadIdx.x / kXcds) * kXcds + threadIdx.x % kXcds] =
                ccnt[threadIdx.x / kXcds][threadIdx.x % kXcds];
        __syncthreads();   // ccnt is reused by the next round
    }
}

// One workgroup per tile of kSlotTile batch slots, one slot per thread: the
// record of a slot that holds a group (the jb-th run of kFwdBatch groups
// among its slice's groups, consecutive in key order), written at the slot's
// place in the batch list: its class's part starts after the parts of the
// lower classes, and inside it come the class's slots holding a group in
// earlier tiles and then those before it in the tile (the workgroup adds up
// k_runs' per-tile, per-class counts itself). The record's loads are issued
// first. Every slot's place (-1: no group) goes to `place`, indexed
// slice-major (fb_base + i2*ceil(m1/kFwdBatch) + jb); workgroup 0 writes the
// parts' starts and the list's length.
__global__ __launch_bounds__(kSlotTile) void k_batches(const TabDev* __restrict__ desc, int32_t T, int64_t K,
                                                       int64_t NFB, const uint64_t* __restrict__ key_scan,
                                                       const int32_t* __restrict__ group_key,
                                                       const int32_t* __restrict__ group_rbase,
                                                       int32_t* __restrict__ ctrl,
                                                       const uint32_t* __restrict__ batch_tiles,
                                                       int32_t* __restrict__ place,
                                                       BatchRec* __restrict__ rec,
                                                       int32_t* __restrict__ fwd_claims) {
    __shared__ uint32_t sbase[kXcds], stot[kXcds];
    if (blockIdx.x == 0 && threadIdx.x < kFwdCounters) fwd_claims[threadIdx.x * 32] = 0;   // the forward's counters
    __shared__ uint32_t wc[kSlotTile / 64][kXcds];
    const int64_t jt = blockIdx.x;
    const int64_t b = jt * kSlotTile + threadIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    BatchRec r;
    memset(&r, 0, sizeof(r));
    SlotOf o{};
    const int32_t tus = block_table_of(desc, T, jt * kSlotTile, min<int64_t>(NFB, (jt + 1) * kSlotTile) - 1,
                                       [](const TabDev& d) { return (int64_t)d.fb_base; });
    if (b < NFB) {
        o = slot_of(desc, T, K, b, key_scan, ctrl, tus);
        r.g0 = o.gs0 + kFwdBatch * o.jb;
        r.ng = max(0, min(kFwdBatch, o.gs1 - r.g0));
        if (r.ng > 0) {
            r.i2 = o.i2;
            r.o1 = o.d.o1; r.o2 = o.d.o2; r.o3 = o.d.o3;
            r.rb0 = group_rbase[r.g0];
            for (int j = 0; j < kFwdBatch; ++j) {
                if (j < r.ng) r.i1[j] = (int32_t)(group_key[r.g0 + j] - o.kb);
                r.rbase[j] = group_rbase[r.g0 + min(j, r.ng)] - r.rb0;
            }
            r.nr = group_rbase[r.g0 + r.ng] - r.rb0;
            r.rbase[kFwdBatch] = r.nr;
        }
    }
    if (threadIdx.x < kXcds) { sbase[threadIdx.x] = 0u; stot[threadIdx.x] = 0u; }
    __syncthreads();
    // per class: the counts of the earlier tiles, and the total of all tiles
    const int64_t nst = (NFB + kSlotTile - 1) / kSlotTile;
    for (int64_t i = threadIdx.x; i < nst * kXcds; i += kSlotTile) {
        const uint32_t c = batch_tiles[i];
        if (c) {
            atomicAdd(&stot[i % kXcds], c);
            if (i / kXcds < jt) atomicAdd(&sbase[i % kXcds], c);
        }
    }
    // rank of the slot among the tile's slots of its class that hold a group
    const bool live = r.ng > 0;
    uint32_t rank = 0;
#pragma unroll
    for (int c = 0; c < kXcds; ++c) {
        const uint64_t m = __ballot(live && o.cls == c);
        if (lane == 0) wc[w][c] = (uint32_t)__popcll(m);
        if (live && o.cls == c) rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    }
    __syncthreads();
    if (live) {
        for (int ww = 0; ww < w; ++ww) rank += wc[ww][o.cls];
        uint32_t start = 0;
        for (int c = 0; c < o.cls; ++c) start += stot[c];
        const uint32_t pos = start + sbase[o.cls] + rank;
        rec[pos] = r;
        place[o.d.fb_base + (int64_t)o.i2 * ((o.d.m1 + kFwdBatch - 1) / kFwdBatch) + o.jb] = (int32_t)pos;
    } else if (b < NFB) {
        place[o.d.fb_base + (int64_t)o.i2 * ((o.d.m1 + kFwdBatch - 1) / kFwdBatch) + o.jb] = -1;
    }
    if (jt == 0 && threadIdx.x <= kXcds) {
        uint32_t start = 0;
        for (int c = 0; c < (int)threadIdx.x; ++c) start += stot[c];
        ctrl[CTRL_CLASS_BASE + threadIdx.x] = (int32_t)start;   // the last one: the list's length
        if (threadIdx.x == kXcds) ctrl[CTRL_NUM_BATCHES] = (int32_t)start;
    }
}

}  // namespace tt

using namespace tt;

// ---------------------------------------------------------------------------
// host side

// Plans created while this is set time their kernels from the start.
static std::atomic<int> g_timing_default{0};

static tt_status check_tables(const tt_emb_table* tables, int32_t T, int64_t* K_out, int32_t* D_out,
                              int32_t* M3_out, int64_t* PR_out, int64_t* CN_out, int64_t* E1_out,
                              int64_t* E2_out, int64_t* E3_out, int64_t* NFB_out, int64_t* NB3_out) {
    if (!tables || T < 1) return TT_ERR_INVALID_ARG;
    if (T > kMaxTables) return TT_ERR_UNSUPPORTED;
    int64_t K = 0, PR = 1, CN = 1, E1 = 0, E2 = 0, E3 = 0, NFB = 0;
    int32_t D = -1, M3 = 1;
    for (int32_t t = 0; t < T; ++t) {
        const tt_emb_table& x = tables[t];
        if (x.reserved != 0) return TT_ERR_INVALID_ARG;
        if (x.num_rows < 1 || x.rank < 1) return TT_ERR_INVALID_ARG;
        for (int k = 0; k < 3; ++k)
            if (x.m[k] < 1 || x.n[k] < 1 || x.g_offset[k] < 0) return TT_ERR_INVALID_ARG;
        const int64_t rows = (int64_t)x.m[0] * x.m[1] * x.m[2];
        if (rows < x.num_rows) return TT_ERR_INVALID_ARG;
        if (x.num_rows >= (int64_t(1) << 31)) return TT_ERR_UNSUPPORTED;
        const int64_t d = (int64_t)x.n[0] * x.n[1] * x.n[2];
        if (D >= 0 && d != D) return TT_ERR_INVALID_ARG;
        if (x.rank > kMaxR || (int64_t)x.n[0] * x.n[1] > kMaxN12 || x.n[2] > kMaxN3 || d > kMaxD)
            return TT_ERR_UNSUPPORTED;
        D = (int32_t)d;
        K += (int64_t)x.m[0] * x.m[1];
        if (K >= kMaxKeys) return TT_ERR_UNSUPPORTED;
        M3 = std::max(M3, x.m[2]);
        NFB += (int64_t)x.m[1] * ((x.m[0] + kFwdBatch - 1) / kFwdBatch);
        PR = std::max<int64_t>(PR, (int64_t)x.n[0] * x.n[1] * x.rank);
        CN = std::max<int64_t>(CN, (int64_t)x.rank * x.n[2]);
        E1 = std::max<int64_t>(E1, x.g_offset[0] + (int64_t)x.m[0] * x.n[0] * x.rank);
        E2 = std::max<int64_t>(E2, x.g_offset[1] + (int64_t)x.m[1] * x.rank * x.n[1] * x.rank);
        E3 = std::max<int64_t>(E3, x.g_offset[2] + (int64_t)x.m[2] * x.rank * x.n[2]);
    }
    if (K * M3 >= (int64_t(1) << 31)) return TT_ERR_UNSUPPORTED;
    // dG3 buckets: every table's G3 rows R*n3 long and aligned to that length
    bool rows3 = E3 % CN == 0 && E3 / CN <= kMaxBuckets3;
    for (int32_t t = 0; t < T && rows3; ++t)
        rows3 = (int64_t)tables[t].rank * tables[t].n[2] == CN && tables[t].g_offset[2] % CN == 0;
    *NB3_out = rows3 ? E3 / CN : 0;
    *K_out = K;
    *D_out = D;
    *M3_out = M3;
    *PR_out = PR;
    *CN_out = CN;
    *E1_out = E1;
    *E2_out = E2;
    *E3_out = E3;
    *NFB_out = NFB;
    return TT_OK;
}

static tt_status check_sizes(int32_t T, int64_t L, int64_t B, int32_t chunk) {
    if (L < 0 || B < 0 || chunk < 1) return TT_ERR_INVALID_ARG;
    if (L >= (int64_t(1) << 31) - 1) return TT_ERR_UNSUPPORTED;
    if ((int64_t)T * B >= (int64_t(1) << 31) - 1) return TT_ERR_UNSUPPORTED;
    if ((int64_t)T * B == 0 && L != 0) return TT_ERR_INVALID_ARG;
    return TT_OK;
}

namespace tt {
size_t workspace_bytes_for(const tt_emb_table* tables, int32_t T, int64_t L, int64_t B, int32_t chunk,
                           bool fwd_only) {
    int64_t K = 0, PR = 1, CN = 1, E1 = 0, E2 = 0, E3 = 0, NFB = 0, NB3 = 0;
    int32_t D = 0, M3 = 1;
    if (check_tables(tables, T, &K, &D, &M3, &PR, &CN, &E1, &E2, &E3, &NFB, &NB3) != TT_OK) return 0;
    if (check_sizes(T, L, B, chunk) != TT_OK) return 0;
    return make_layout(T, L, B, chunk, K, D, M3, PR, CN, E1, E2, E3, NFB, NB3, fwd_only).total;
}
}  // namespace tt

extern "C" size_t tt_emb_workspace_bytes(const tt_emb_table* tables, int32_t T, int64_t L,
                                         int64_t B, int32_t chunk) {
    return workspace_bytes_for(tables, T, L, B, chunk, false);
}

// Plans into the host object *p (filled here; nothing is allocated). The
// caller keeps `tables` alive as long as p uses it.
tt_status tt::plan_into(tt_emb_plan_s* p, const tt_emb_table* tables, int32_t T, const int64_t* indices,
                        const int64_t* offsets, int64_t L, int64_t B, int32_t chunk, void* workspace,
                        size_t workspace_bytes, bool fwd_only, hipStream_t s, const void* cache,
                        int64_t n_hot) {
    int64_t K = 0, PR = 1, CN = 1, E1 = 0, E2 = 0, E3 = 0, NFB = 0, NB3 = 0;
    int32_t D = 0, M3 = 1;
    tt_status st = check_tables(tables, T, &K, &D, &M3, &PR, &CN, &E1, &E2, &E3, &NFB, &NB3);
    if (st != TT_OK) return st;
    st = check_sizes(T, L, B, chunk);
    if (st != TT_OK) return st;
    if (!offsets || !workspace || (L > 0 && !indices)) return TT_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255) != 0) return TT_ERR_INVALID_ARG;
    if (cache && (fwd_only || n_hot < 0 || ((uintptr_t)cache & 255) != 0)) return TT_ERR_INVALID_ARG;
    if (fwd_only) NB3 = 0;
    const Layout lay = make_layout(T, L, B, chunk, K, D, M3, PR, CN, E1, E2, E3, NFB, NB3, fwd_only);
    if (workspace_bytes < lay.total) return TT_ERR_WORKSPACE;

    p->T = T; p->L = L; p->B = B; p->TB = (int64_t)T * B; p->chunk = chunk; p->D = D; p->K = K;
    p->M3 = M3;
    p->nb3 = (int32_t)NB3;
    p->cn = CN;
    p->n_i2 = 0;
    p->n_fb = 0;
    for (int32_t t = 0; t < T; ++t) {
        p->n_i2 += tables[t].m[1];
        p->n_fb += (int64_t)tables[t].m[1] * ((tables[t].m[0] + kFwdBatch - 1) / kFwdBatch);
    }
    p->ws = (char*)workspace;
    p->lay = lay;
    p->cached = cache != nullptr;
    p->n_hot = cache ? n_hot : 0;
    p->hot_lg = cache ? cache_lg(n_hot) : 0;
    p->hot_keys = cache ? reinterpret_cast<const int64_t*>((const char*)cache + kHotHeader) : nullptr;
    p->hot_slots = cache ? reinterpret_cast<const int32_t*>((const char*)cache + cache_slots_offset(p->hot_lg))
                         : nullptr;
    p->tables = tables;
    p->fwd_only = fwd_only;
    p->uniform = true;
    p->n1 = tables[0].n[0]; p->n2 = tables[0].n[1]; p->n3 = tables[0].n[2]; p->R = tables[0].rank;
    for (int k = 0; k < 3; ++k) p->extent[k] = 0;
    p->packed = true;
    p->kept_token = 0;
    p->next_token = 0;
    p->kept_g1 = nullptr;
    p->kept_g2 = nullptr;
    p->off4 = true;
    p->g3_total = 0;
    for (int32_t t = 0; t < T; ++t) {
        if (tables[t].g_offset[0] % 4 != 0 || tables[t].g_offset[1] % 4 != 0 || tables[t].g_offset[2] % 4 != 0)
            p->off4 = false;
        p->g3_total += (int64_t)tables[t].m[2] * tables[t].rank * tables[t].n[2];
        const tt_emb_table& x = tables[t];
        if (x.n[0] != p->n1 || x.n[1] != p->n2 || x.n[2] != p->n3 || x.rank != p->R) p->uniform = false;
        const int64_t R = x.rank;
        const int64_t sz[3] = {(int64_t)x.m[0] * x.n[0] * R, (int64_t)x.m[1] * R * x.n[1] * R,
                               (int64_t)x.m[2] * R * x.n[2]};
        for (int k = 0; k < 3; ++k) {
            if (x.g_offset[k] != p->extent[k]) p->packed = false;
            p->extent[k] = std::max(p->extent[k], x.g_offset[k] + sz[k]);
        }
    }
    // tables may share a core; a shared G2 needs a backward that adds the
    // tables' dG2 terms (the matrix-core dG2 kernel stores each slice once)
    p->g2_overlap = false;
    for (int32_t a = 0; a < T && !p->g2_overlap; ++a)
        for (int32_t b = a + 1; b < T; ++b) {
            const tt_emb_table& x = tables[a];
            const tt_emb_table& y = tables[b];
            const int64_t xe = x.g_offset[1] + (int64_t)x.m[1] * x.rank * x.n[1] * x.rank;
            const int64_t ye = y.g_offset[1] + (int64_t)y.m[1] * y.rank * y.n[1] * y.rank;
            if (x.g_offset[1] < ye && y.g_offset[1] < xe) { p->g2_overlap = true; break; }
        }
    // control words and descriptors
    // control words and the scans' tile status words (adjacent in the workspace)
    // are cleared by the launch that writes the first descriptors
    const int64_t nzero = (int64_t)((lay.scan_st - lay.ctrl) + sizeof(ScanTileStatus) * lay.scan_tiles) / 4;
    int nscan = 0;   // scans issued so far (each gets its own epoch and tile counter)
    int32_t kb = 0, i2b = 0, fbb = 0;
    int64_t g3b = 0;
    for (int32_t first = 0; first < T; first += 16) {
        DescBatch b{};
        b.first = first;
        b.count = std::min<int32_t>(16, T - first);
        for (int i = 0; i < b.count; ++i) {
            const tt_emb_table& x = tables[first + i];
            TabDev& d = b.d[i];
            d.N = (int32_t)x.num_rows;
            d.m1 = x.m[0]; d.m2 = x.m[1]; d.m3 = x.m[2];
            d.n1 = x.n[0]; d.n2 = x.n[1]; d.n3 = x.n[2]; d.R = x.rank;
            d.o1 = x.g_offset[0]; d.o2 = x.g_offset[1]; d.o3 = x.g_offset[2];
            d.key_base = kb;
            d.i2_base = i2b;
            i2b += x.m[1];
            d.fb_base = fbb;
            fbb += x.m[1] * ((x.m[0] + kFwdBatch - 1) / kFwdBatch);
            d.g3_base = g3b;
            g3b += (int64_t)x.m[2] * x.rank * x.n[2];
            kb += x.m[0] * x.m[1];
        }
        if (first == 0)
            TT_LAUNCH(p, "k_init", s, k_init, dim3(std::min<unsigned>(grid_for(nzero, 256), 64u)), dim3(256), 0, s,
                               reinterpret_cast<uint32_t*>(p->ctrl()), nzero, p->at<TabDev>(lay.desc), b);
        else
            TT_LAUNCH(p, "k_write_desc", s, k_write_desc, dim3(1), dim3(16), 0, s, p->at<TabDev>(lay.desc), b);
        if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
    }

    int32_t* ctrl = p->ctrl();
    // runs per G3 row are counted for the backward's dG3 reduction
    const int32_t n3cnt = (int32_t)NB3;
    int32_t* key = p->at<int32_t>(lay.key);
    int32_t* i3 = p->at<int32_t>(lay.i3);
    int32_t* bag = p->at<int32_t>(lay.bag_of);
    // split (also checks the offsets, labels the bags, marks every key absent
    // and counts the first radix pass's digits per tile)
    {
        const int64_t nx = std::max<int64_t>(std::max<int64_t>((p->TB + 1 + kSortThreads - 1) / kSortThreads,
                                                               (K + kSortTile - 1) / kSortTile),
                                             ((int64_t)n3cnt + kSortTile - 1) / kSortTile);
        TT_LAUNCH(p, "k_split", s, k_split, dim3((unsigned)(lay.n_tiles + nx)), dim3(kSortThreads), 0,
                  s, indices, offsets, L, p->TB, B > 0 ? B : 1, p->desc(), key, i3, bag,
                  p->at<int32_t>(lay.bag_start), p->at<int32_t>(lay.ckey), p->M3, ctrl,
                  p->at<int32_t>(lay.key_start), K, p->at<int32_t>(lay.i3cnt), n3cnt, lay.n_tiles, lay.hstride,
                  p->at<uint32_t>(lay.hist), p->hot_keys, p->hot_slots, p->hot_lg,
                  p->cached ? p->at<int32_t>(lay.cslot) : nullptr);
        if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
    }
    // stable radix sort: key -> (skey, perm)
    if (L > 0) {
        const int P = lay.passes;
        uint32_t* hist = p->at<uint32_t>(lay.hist);
        const int32_t* kin = p->at<int32_t>(lay.ckey);
        const int32_t* vin = nullptr;
        const int32_t* bin = bag;
        for (int pass = 0; pass < P; ++pass) {
            // the last pass lands in (skey, perm); earlier passes alternate so that it does
            const bool to_final = ((P - 1 - pass) % 2) == 0;
            int32_t* kout = p->at<int32_t>(to_final ? lay.sort_k1 : lay.sort_k0);
            int32_t* vout = p->at<int32_t>(to_final ? lay.sort_v1 : lay.sort_v0);
            int32_t* bout = p->at<int32_t>(to_final ? lay.sort_b1 : lay.sort_b0);
            const int shift = pass * kRadixBits;
            if (pass > 0) {   // the first pass's counts come from k_split
                TT_LAUNCH(p, "k_radix_hist", s, k_radix_hist, dim3((unsigned)lay.n_tiles), dim3(kSortThreads), 0, s,
                          kin, L, shift, lay.n_tiles, lay.hstride, hist);
                if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
            }
            if (lay.n_tiles <= kDirectTiles) {
                TT_LAUNCH(p, "k_radix_scatter", s, k_radix_scatter<true>, dim3((unsigned)lay.n_tiles), dim3(kSortThreads), 0,
                                   s, kin, vin, bin, L, (int32_t)p->TB, shift, lay.hstride, hist, kout, vout, bout);
            } else {
                if (scan_exclusive<uint32_t>(p, ++nscan, hist, (int64_t)kRadixBins * lay.hstride, nullptr, s) !=
                    TT_OK)
                    return TT_ERR_HIP;
                TT_LAUNCH(p, "k_radix_scatter", s, k_radix_scatter<false>, dim3((unsigned)lay.n_tiles), dim3(kSortThreads), 0,
                                   s, kin, vin, bin, L, (int32_t)p->TB, shift, lay.hstride, hist, kout, vout, bout);
            }
            if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
            kin = kout;
            vin = vout;
            bin = bout;
        }
    }
    // groups and chunks
    {
        int32_t* key_start = p->at<int32_t>(lay.key_start);
        int32_t* key_end = p->at<int32_t>(lay.key_end);
        uint64_t* kscan = p->at<uint64_t>(lay.key_scan);
        uint32_t* run_tiles = p->at<uint32_t>(lay.run_tiles);
        uint64_t* key_tiles = p->at<uint64_t>(lay.key_tiles);
        if (L > 0) {
            TT_LAUNCH(p, "k_gather", s, k_gather, dim3((unsigned)lay.n_tiles), dim3(kSortThreads), 0, s,
                               p->at<int32_t>(lay.skey), L, p->M3, p->at<int32_t>(lay.sorted_i3), key_start,
                               key_end, run_tiles);
            if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
        }
        TT_LAUNCH(p, "k_key_tiles", s, k_key_tiles, dim3((unsigned)lay.n_ktiles), dim3(kSortThreads), 0, s, key_start,
                           key_end, K, chunk, key_tiles);
        if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
        const bool kdirect = lay.n_ktiles <= kDirectTiles;
        if (!kdirect && scan_exclusive<uint64_t>(p, ++nscan, key_tiles, lay.n_ktiles, nullptr, s) != TT_OK)
            return TT_ERR_HIP;
        TT_LAUNCH(p, "k_groups", s, kdirect ? k_groups<true> : k_groups<false>, dim3((unsigned)lay.n_ktiles),
                           dim3(kSortThreads), 0, s, key_start, key_end, K, L, chunk, key_tiles, kscan,
                           p->at<int32_t>(lay.group_key), p->at<int32_t>(lay.group_start),
                           p->at<int32_t>(lay.group_cbase), ctrl);
        if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
        if (L > 0) {
            const bool rdirect = lay.n_tiles <= kDirectTiles;
            if (!rdirect && scan_exclusive<uint32_t>(p, ++nscan, run_tiles, lay.n_tiles, nullptr, s) != TT_OK)
                return TT_ERR_HIP;
            TT_LAUNCH(p, "k_runs", s, rdirect ? k_runs<true> : k_runs<false>, dim3((unsigned)lay.n_tiles),
                               dim3(kSortThreads), 0, s, p->at<int32_t>(lay.perm), p->at<int32_t>(lay.skey),
                               p->at<uint64_t>(lay.key_scan), key_start, key_end, run_tiles, L, p->M3, chunk,
                               ctrl, p->at<int32_t>(lay.rid), p->at<int32_t>(lay.run_i3),
                               p->at<int32_t>(lay.run_of), p->at<int32_t>(lay.run_start),
                               p->at<int32_t>(lay.group_rbase), p->at<int32_t>(lay.chunk_group),
                               p->at<int32_t>(lay.chunk_begin), p->at<int32_t>(lay.chunk_end),
                               p->at<int32_t>(lay.i3cnt), n3cnt, p->at<int32_t>(lay.run_rank),
                               p->at<int32_t>(lay.run_bkt), p->desc(), T, (int32_t)CN, K, lay.NFB,
                               p->at<uint32_t>(lay.batch_tiles), p->cached ? p->at<int32_t>(lay.cslot) : nullptr,
                               p->cached ? p->at<int32_t>(lay.run_cslot) : nullptr, p->at<int32_t>(lay.sorted_bag),
                               p->fwd_only ? nullptr : p->at<int32_t>(lay.run_bag1));
            if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
        }
        if (lay.NFB > 0 && L > 0) {   // (no lookups: the list stays empty, its length 0 from k_init)
            // the batch list: slots that hold a group, compacted in slot order
            TT_LAUNCH(p, "k_batches", s, k_batches, dim3((unsigned)((lay.NFB + kSlotTile - 1) / kSlotTile)),
                      dim3(kSlotTile), 0, s, p->desc(), T, K, lay.NFB, kscan, p->at<int32_t>(lay.group_key),
                      p->at<int32_t>(lay.group_rbase), ctrl, p->at<uint32_t>(lay.batch_tiles),
                      p->at<int32_t>(lay.batch_place), p->at<BatchRec>(lay.batch),
                      p->at<int32_t>(lay.claims) + 32 * kRunCounters);
            if (hipGetLastError() != hipSuccess) return TT_ERR_HIP;
        }
    }
    return TT_OK;
}

static tt_status plan_new(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                          const int64_t* offsets, int64_t L, int64_t B, int32_t chunk, void* workspace,
                          size_t workspace_bytes, void* stream, tt_emb_plan_t* plan_out, const void* cache,
                          int64_t n_hot);

extern "C" tt_status tt_emb_plan(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                                 const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 tt_emb_plan_t* plan_out) {
    return plan_new(tables, T, indices, offsets, L, B, chunk, workspace, workspace_bytes, stream, plan_out,
                    nullptr, 0);
}

extern "C" tt_status tt_emb_plan_cached(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                                        const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                                        const void* cache, int64_t n_hot, void* workspace,
                                        size_t workspace_bytes, void* stream, tt_emb_plan_t* plan_out) {
    if (plan_out) *plan_out = nullptr;
    if (!cache || n_hot < 0) return TT_ERR_INVALID_ARG;
    return plan_new(tables, T, indices, offsets, L, B, chunk, workspace, workspace_bytes, stream, plan_out,
                    cache, n_hot);
}

static tt_status plan_new(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                          const int64_t* offsets, int64_t L, int64_t B, int32_t chunk, void* workspace,
                          size_t workspace_bytes, void* stream, tt_emb_plan_t* plan_out, const void* cache,
                          int64_t n_hot) {
    if (!plan_out) return TT_ERR_INVALID_ARG;
    *plan_out = nullptr;
    if (!tables || T < 1) return TT_ERR_INVALID_ARG;
    if (T > kMaxTables) return TT_ERR_UNSUPPORTED;
    tt_emb_plan_s* p = new (std::nothrow) tt_emb_plan_s();
    if (!p) return TT_ERR_INVALID_ARG;
    p->owned_tables = new (std::nothrow) tt_emb_table[T];
    if (!p->owned_tables) { delete p; return TT_ERR_INVALID_ARG; }
    if (g_timing_default.load()) p->timing = new (std::nothrow) Timing();
    std::memcpy(p->owned_tables, tables, sizeof(tt_emb_table) * (size_t)T);
    const tt_status st = plan_into(p, p->owned_tables, T, indices, offsets, L, B, chunk, workspace,
                                   workspace_bytes, false, (hipStream_t)stream, cache, n_hot);
    if (st != TT_OK) { delete p; return st; }
    *plan_out = p;
    return TT_OK;
}

extern "C" tt_status tt_emb_get_error(tt_emb_plan_t p, int32_t* flag_out, void* stream) {
    if (!p || !flag_out) return TT_ERR_INVALID_ARG;
    int32_t f = 0;
    hipStream_t s = (hipStream_t)stream;
    TT_HIP_CHECK(hipMemcpyAsync(&f, p->ctrl() + CTRL_FLAG, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    TT_HIP_CHECK(hipStreamSynchronize(s));
    *flag_out = f;
    return f ? TT_ERR_DEVICE_FLAG : TT_OK;
}

extern "C" tt_status tt_emb_plan_get_view(tt_emb_plan_t p, tt_emb_plan_view* v) {
    if (!p || !v) return TT_ERR_INVALID_ARG;
    const Layout& y = p->lay;
    v->key = p->at<int32_t>(y.key);
    v->i3 = p->at<int32_t>(y.i3);
    v->bag_of = p->at<int32_t>(y.bag_of);
    v->perm = p->at<int32_t>(y.perm);
    v->sorted_i3 = p->at<int32_t>(y.sorted_i3);
    v->sorted_bag = p->at<int32_t>(y.sorted_bag);
    v->group_key = p->at<int32_t>(y.group_key);
    v->group_start = p->at<int32_t>(y.group_start);
    v->chunk_group = p->at<int32_t>(y.chunk_group);
    v->chunk_begin = p->at<int32_t>(y.chunk_begin);
    v->chunk_end = p->at<int32_t>(y.chunk_end);
    v->max_groups = y.Gmax;
    v->max_chunks = y.Cmax;
    return TT_OK;
}

extern "C" tt_status tt_emb_plan_counts(tt_emb_plan_t p, int64_t* num_groups, int64_t* num_chunks,
                                        void* stream) {
    if (!p || !num_groups || !num_chunks) return TT_ERR_INVALID_ARG;
    int32_t c[3] = {0, 0, 0};
    hipStream_t s = (hipStream_t)stream;
    TT_HIP_CHECK(hipMemcpyAsync(c, p->ctrl(), sizeof(c), hipMemcpyDeviceToHost, s));
    TT_HIP_CHECK(hipStreamSynchronize(s));
    *num_groups = c[CTRL_NUM_GROUPS];
    *num_chunks = c[CTRL_NUM_CHUNKS];
    return TT_OK;
}

extern "C" tt_status tt_emb_query_paths(tt_emb_plan_t p, const float* g1, const float* g2,
                                        tt_emb_path_info* info) {
    if (!p || !info) return TT_ERR_INVALID_ARG;
    const bool f = fwd_mfma_ok(p, g1, g2), b = bwd_mfma_ok(p, g1, g2);
    info->forward_path = f ? TT_PATH_MATRIX_CORE : TT_PATH_GENERIC;
    info->backward_path = b ? TT_PATH_MATRIX_CORE : TT_PATH_GENERIC;
    info->keeps_prefix = (f && b) ? 1 : 0;
    info->dg3_by_rows = (b && p->nb3 > 0) ? 1 : 0;
    info->workspace_bytes = (uint64_t)p->lay.total;
    return TT_OK;
}

extern "C" tt_status tt_emb_set_timing(tt_emb_plan_t p, int32_t enable) {
    if (!p) {
        g_timing_default.store(enable ? 1 : 0);
        return TT_OK;
    }
    if (enable && !p->timing) {
        p->timing = new (std::nothrow) Timing();
        if (!p->timing) return TT_ERR_INVALID_ARG;
    } else if (!enable && p->timing) {
        timing_free(p->timing);
        p->timing = nullptr;
    }
    return TT_OK;
}

extern "C" tt_status tt_emb_kernel_times(tt_emb_plan_t p, tt_emb_kernel_time* out, int32_t max,
                                         int32_t* count, void* stream) {
    if (!p || !count || (max > 0 && !out) || max < 0) return TT_ERR_INVALID_ARG;
    *count = 0;
    Timing* t = p->timing;
    if (!t) return TT_OK;
    TT_HIP_CHECK(hipStreamSynchronize((hipStream_t)stream));
    const int n = std::min<int>(t->n, max);
    for (int i = 0; i < n; ++i) {
        float ms = 0.f;
        TT_HIP_CHECK(hipEventElapsedTime(&ms, t->ev[i][0], t->ev[i][1]));
        out[i].kernel = t->name[i];
        out[i].ms = ms;
    }
    *count = n;
    t->n = 0;
    return TT_OK;
}

extern "C" tt_status tt_emb_plan_destroy(tt_emb_plan_t p) {
    delete p;
    return TT_OK;
}

extern "C" const char* tt_emb_status_string(tt_status s) {
    switch (s) {
        case TT_OK: return "ok";
        case TT_ERR_INVALID_ARG: return "invalid argument";
        case TT_ERR_UNSUPPORTED: return "unsupported (outside the library's limits)";
        case TT_ERR_WORKSPACE: return "workspace too small";
        case TT_ERR_HIP: return "HIP runtime error";
        case TT_ERR_DEVICE_FLAG: return "device error flag set (bad index or offsets)";
        case TT_ERR_STALE: return "kept prefix products are stale (token does not match the plan)";
        case TT_ERR_SCRATCH: return "batch needs more than the library's static scratch buffer holds";
        case TT_ERR_CACHE: return "hot-row cache mismatch (a plan with a cache takes only the _cached calls, which need one)";
    }
    return "unknown status";
}
