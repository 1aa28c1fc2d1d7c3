// Hot-row cache of the TT-EmbeddingBag library: the hash table that maps a
// (table, row) pair to its slot among the rows kept uncompressed (TT-Rec
// abstract: caching strategies for the lookups; TT-Rec news article, method
// paragraph: a cache structure for the skewed sparse-feature distribution).
#include "tt_internal.h"

#include <climits>

namespace tt {

// One thread per hot entry: insert (table << 40 | row) by linear probing.
// Entries naming no row (negative, or a row past 2^40) are skipped. A pair
// listed more than once keeps its smallest slot (every copy takes the
// minimum); keys start at kHotEmpty and slots at INT_MAX.
__global__ __launch_bounds__(256) void k_cache_build(const int32_t* __restrict__ hot_table,
                                                     const int64_t* __restrict__ hot_row, int64_t n,
                                                     int lg, int64_t* __restrict__ keys,
                                                     int32_t* __restrict__ slots) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    const int64_t t = hot_table[s], r = hot_row[s];
    if (t < 0 || r < 0 || r >= (int64_t(1) << 40)) return;
    const int64_t key = (t << 40) | r;
    const uint64_t mask = (uint64_t(1) << lg) - 1;
    uint64_t h = cache_hash(key, lg);
    for (uint64_t k = 0; k <= mask; ++k) {   // at most half full: an empty entry is always found
        const unsigned long long prev = atomicCAS(reinterpret_cast<unsigned long long*>(keys + h),
                                                  (unsigned long long)kHotEmpty, (unsigned long long)key);
        if ((int64_t)prev == kHotEmpty || (int64_t)prev == key) {
            atomicMin(slots + h, (int32_t)s);
            return;
        }
        h = (h + 1) & mask;
    }
}

}  // namespace tt

using namespace tt;

extern "C" size_t tt_emb_cache_bytes(int64_t n_hot) {
    if (n_hot < 0 || n_hot > (int64_t(1) << 30)) return 0;
    return cache_bytes_lg(cache_lg(n_hot));
}

extern "C" tt_status tt_emb_cache_build(const int32_t* hot_table, const int64_t* hot_row, int64_t n_hot,
                                        void* cache, size_t cache_bytes, void* stream) {
    if (!cache || n_hot < 0 || (n_hot > 0 && (!hot_table || !hot_row))) return TT_ERR_INVALID_ARG;
    if (((uintptr_t)cache & 255) != 0) return TT_ERR_INVALID_ARG;
    const size_t need = tt_emb_cache_bytes(n_hot);
    if (need == 0) return TT_ERR_UNSUPPORTED;
    if (cache_bytes < need) return TT_ERR_WORKSPACE;
    const int lg = cache_lg(n_hot);
    const int64_t cap = int64_t(1) << lg;
    hipStream_t s = (hipStream_t)stream;
    int64_t* keys = reinterpret_cast<int64_t*>((char*)cache + kHotHeader);
    int32_t* slots = reinterpret_cast<int32_t*>((char*)cache + cache_slots_offset(lg));
    tt_status st = fill32(nullptr, keys, 0xFFFFFFFFu, 2 * cap, s);   // kHotEmpty
    if (st != TT_OK) return st;
    if ((st = fill32(nullptr, slots, (uint32_t)INT_MAX, cap, s)) != TT_OK) return st;
    if (n_hot > 0) {
        TT_LAUNCH(nullptr, "k_cache_build", s, k_cache_build, dim3(grid_for(n_hot, 256)), dim3(256), 0, s,
                  hot_table, hot_row, n_hot, lg, keys, slots);
        TT_LAUNCH_CHECK();
    }
    return TT_OK;
}
