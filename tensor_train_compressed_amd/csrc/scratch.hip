// Allocation-free forward of the TT-EmbeddingBag library: planning and the
// forward of one batch in a static device buffer of the library's own, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid allocation). Same kernels as
// tt_emb_plan + tt_emb_forward, with a forward-only workspace layout.
#include "tt_internal.h"

#include <mutex>

// The scratch buffer: one per device, held from the library's load until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory; kernels get the address hipGetSymbolAddress returns.
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, null until looked up

// The device address of the current device's scratch array, looked up once
// per device (with that device current).
tt_status scratch_address(void** out) {
    int dev = -1;
    TT_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return TT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_lock);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TT_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TT_OK;
}

}  // namespace

extern "C" size_t tt_emb_scratch_capacity(void) { return kScratchBytes; }

extern "C" tt_status tt_emb_forward_scratch(const tt_emb_table* tables, int32_t T, const int64_t* indices,
                                            const int64_t* offsets, int64_t L, int64_t B, int32_t chunk,
                                            const float* g1, const float* g2, const float* g3, float* out,
                                            void* stream) {
    // the size check comes first and needs no device: a batch too large for
    // the buffer is refused before any HIP call
    const size_t need = tt::workspace_bytes_for(tables, T, L, B, chunk, true);
    if (need > kScratchBytes) return TT_ERR_SCRATCH;
    if (!g1 || !g2 || !g3) return TT_ERR_INVALID_ARG;
    void* ws = nullptr;
    tt_status st = scratch_address(&ws);
    if (st != TT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    tt_emb_plan_s p{};   // host object on the stack: the kernels take their arguments by value
    st = tt::plan_into(&p, tables, T, indices, offsets, L, B, chunk, ws, kScratchBytes, true, s);
    if (st != TT_OK) return st;
    return tt::forward_run(&p, g1, g2, g3, out, false, nullptr, s);
}
