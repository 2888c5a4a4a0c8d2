// moe_layer_forward_noalloc: moe_layer_forward on a scratch buffer the
// library holds itself, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, hosts that forbid
// allocation in the hot path).
//
// The buffer is one file-scope device array of MOE_NOALLOC_SCRATCH_BYTES per
// GPU, alive until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol): the
// first call on a device looks up that device's copy with
// hipGetSymbolAddress, and every later call on the device passes that
// address as the layer's workspace.  The layer needs no zeroed workspace, so
// nothing is cleared between calls.
#include "moe_internal.h"

#include <atomic>
#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_lookup;

// the current device's copy of the array (looked up once per device)
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_EHIP;
    if (dev >= kMaxDevices) return MOE_EUNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return MOE_EHIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

} // namespace

extern "C" int moe_layer_forward_noalloc(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
                                         const float *bias, const moe_weights_t *routed,
                                         const moe_weights_t *shared, float *y, int32_t *idx_out, float *w_out,
                                         uint32_t flags, hipStream_t stream)
{
    // a call the fixed buffer cannot hold is refused before anything runs
    // (0 means the arguments are invalid: moe_layer_forward reports which)
    const size_t need = moe_workspace_bytes(shape, T, flags);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
    void *ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return moe_layer_forward(shape, x, T, gate_w, bias, routed, shared, y, idx_out, w_out, flags, ws,
                             (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
