// Block-aligned splice as an edit of the block table and of the per-block
// pending rotary shifts (Leyline, sections 2.2-2.3: downstream slots are
// re-indexed and owe R(Delta); since R(a) R(b) = R(a + b) the shift is added
// to the block's pending delta and applied once when the key is read,
// Irminsul, sections 2.2 and 4).  No KV byte moves.
//
// Splice: one workgroup per sequence; the old table row and shift row are
// staged in LDS first, so the in-place rewrite may shift entries either way.
// Gather by reference: one workgroup per entry.
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_lazy;

namespace {

__global__ __launch_bounds__(kThreads) void lazy_kernel(const LazyArgs A) {
    __shared__ int32_t s_bt[kLazyMaxBlocks], s_pd[kLazyMaxBlocks];
    const LazySeq& S = A.seqs[blockIdx.x];
    const int tid = threadIdx.x;
    int32_t* bt = A.bt + (int64_t)S.row * A.bt_stride;
    int32_t* pd = A.pend + (int64_t)S.row * A.bt_stride;
    for (int k = tid; k < S.n_old; k += kThreads) {
        s_bt[k] = bt[k];
        s_pd[k] = pd[k];
    }
    __syncthreads();
    const int db = S.delta / A.block_size;
    const int kmax = max(S.n_old, S.n_new);
    for (int k = S.s0b + tid; k < kmax; k += kThreads) {
        if (k < S.s0b + S.rb) {
            bt[k] = A.stubs[S.stub_off + k - S.s0b];
            pd[k] = 0;
        } else if (k < S.n_new) {
            const int src = k - db;
            const int64_t v = (int64_t)s_pd[src] + S.delta;
            int32_t nv = (int32_t)v;
            if (v != (int64_t)nv) {
                __hip_atomic_fetch_or(&g_errors_lazy, KVR_DEV_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                nv = s_pd[src];
            }
            bt[k] = s_bt[src];
            pd[k] = nv;
        } else {
            bt[k] = -1;
            pd[k] = 0;
        }
    }
    for (int k = S.s0b + tid; k < S.s1b; k += kThreads) A.freed[S.free_off + k - S.s0b] = s_bt[k];
}

// Registry entries placed by reference (Irminsul, section 2.2: the entry
// owes R(p_target - p_source)): the destination's logical blocks take the
// entry's block ids, each with the entry block's own pending shift plus the
// entry's delta.  Entries of one launch never share a table slot.
__global__ __launch_bounds__(kThreads) void lazy_gather_kernel(const LazyGatherArgs A) {
    const LazyEntry& E = A.ents[blockIdx.x];
    int32_t* bt = A.bt + (int64_t)E.row * A.bt_stride + E.slot0;
    int32_t* pd = A.pend + (int64_t)E.row * A.bt_stride + E.slot0;
    for (int k = threadIdx.x; k < E.nb; k += kThreads) {
        const int32_t own = E.pend ? E.pend[k] : 0;
        const int64_t v = (int64_t)own + E.delta;
        int32_t nv = (int32_t)v;
        if (v != (int64_t)nv) {
            __hip_atomic_fetch_or(&g_errors_lazy, KVR_DEV_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nv = own;
        }
        if (A.replaced) A.replaced[E.rep_off + k] = bt[k];
        bt[k] = E.blocks[k];
        pd[k] = nv;
    }
}

}  // namespace

hipError_t launch_lazy_gather(const LazyGatherArgs& a, hipStream_t s) {
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(lazy_gather_kernel, dim3(a.n), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_lazy(const LazyArgs& a, hipStream_t s) {
    if (a.n_seq <= 0) return hipSuccess;
    hipLaunchKernelGGL(lazy_kernel, dim3(a.n_seq), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_lazy() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_lazy), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_lazy), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
