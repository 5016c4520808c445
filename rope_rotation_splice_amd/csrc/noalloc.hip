// The in-place splice for callers that cannot allocate device memory (code
// under graph capture, tight serving loops): leyline_splice with its
// workspace taken from a file-scope device array instead of the caller.
//
// The array belongs to the loaded library and exists once per GPU the
// library runs on, until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is a host-side stand-in): its
// device address is taken with hipGetSymbolAddress once per device, on the
// first call with that device current, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kvreloc.h"
#include "kvr_internal.h"

namespace {

constexpr size_t kScratchBytes = KVR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];              // device address of `scratch`, per device

kvr_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return kvr::record_hip_error(e);
    if (dev < 0 || dev >= kMaxDevices) return KVR_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return kvr::record_hip_error(e);
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return KVR_E_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KVR_OK;
}

}  // namespace

extern "C" kvr_status leyline_splice_noalloc(const kvr_cache* cache, const int32_t* d_block_tables,
                                             int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                                             const kvr_directive* dirs, const kvr_rows* stubs, int64_t* new_lens,
                                             hipStream_t stream) {
    void* ws = nullptr;
    kvr_status st = scratch_on_current_device(&ws);
    if (st != KVR_OK) return st;
    // the plan's ticket counters and flags, as a caller's workspace would hold them
    const size_t need = kvr_splice_workspace_bytes(cache, n_seq, seq_lens, dirs);
    if (need > kScratchBytes) return KVR_E_SCRATCH;
    if (need > 0) {
        // the array keeps the previous call's contents: start from zero
        st = kvr_workspace_clear(ws, need, stream);
        if (st != KVR_OK) return st;
    }
    return leyline_splice(cache, d_block_tables, bt_stride, n_seq, seq_lens, dirs, stubs, new_lens, ws,
                          kScratchBytes, stream);
}

extern "C" size_t kvr_noalloc_scratch_bytes(void) { return kScratchBytes; }
