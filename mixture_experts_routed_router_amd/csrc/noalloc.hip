// noalloc.hip -- moe_expert_ffn_gather without a caller-provided workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The FFN's scratch (its tile schedule and work counters) lives in a file-scope
// device array instead; each GPU holds its own copy of it until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever passed to a kernel.  The entry point allocates and frees nothing.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's contents: the
// schedule kernel at the start of each call rewrites the tile records and clears the GEMMs'
// counters (by kernel stores, no memset), so nothing needs clearing here.  Calls that overlap
// on one GPU (two streams, two host threads) race on the array.
#include <mutex>

#include "moe_launch.h"

namespace {

// Room for the workspace of a table of up to MOE_FFN_NOALLOC_MAX_BLOCKS blocks.
constexpr int64_t kScratchElems = 32 + 15 * (int64_t)MOE_FFN_NOALLOC_MAX_BLOCKS;

__device__ __attribute__((aligned(256))) int32_t scratch[kScratchElems];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int32_t* g_ptr[kMaxDevices] = {};

// This device's address of `scratch` (nullptr on failure); looked up once per device.
int32_t* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = static_cast<int32_t*>(p);
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

moe_status_t moe_expert_ffn_gather_noalloc(const void* x, const int32_t* row_token, int T,
                                           const void* w1, const void* w2, moe_dtype_t dt,
                                           int H, int I, int E_loc, const int32_t* blocks,
                                           const int32_t* n_blocks, int max_blocks, void* act,
                                           void* yp, int64_t max_rows, hipStream_t stream) {
    if (max_blocks < 1) return MOE_ERR_INVALID;
    if (max_blocks > MOE_FFN_NOALLOC_MAX_BLOCKS) return MOE_ERR_UNSUPPORTED;
    const int64_t need = moe_ffn_workspace_elems(max_blocks);
    if (need < 1 || need > kScratchElems) return MOE_ERR_UNSUPPORTED;
    int32_t* ws = scratch_on_current_device();
    if (!ws) return MOE_ERR_LAUNCH;
    return moe_expert_ffn_gather(x, row_token, T, w1, w2, dt, H, I, E_loc, blocks, n_blocks,
                                 max_blocks, act, yp, max_rows, ws, need, stream);
}

}  // extern "C"
