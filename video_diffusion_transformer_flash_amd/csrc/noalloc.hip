// dit_block_forward_noalloc: the Flash DiT block on a static per-device
// scratch array instead of a caller workspace, for callers that cannot
// allocate (code under graph capture, serving loops, harnesses that forbid
// allocation). Same kernels and launch sequence as dit_block_forward.
#include <mutex>

#include "common.h"
#include "kernels.h"

// The block's workspace, one copy per device the library runs on, held until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress once per
// device (scratch_ptr below), and only that address reaches the kernels.
static constexpr size_t SCRATCH_BYTES = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

namespace {

std::mutex g_mu;
void* g_dev_ptr[64] = {};

// device address of `scratch` on the current device
int scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        dit::set_last_hip((int)e);
        return DIT_EHIP;
    }
    if (dev < 0 || dev >= 64) return DIT_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_dev_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p || ((uintptr_t)p & 255)) {
            dit::set_last_hip(e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol);
            return DIT_EHIP;
        }
        g_dev_ptr[dev] = p;
    }
    *out = g_dev_ptr[dev];
    return DIT_OK;
}

}  // namespace

extern "C" int32_t dit_block_forward_noalloc(const dit_dims* dims, const void* x_text, const void* x_video,
                                             const void* x_audio, const dit_block_weights* weights, int32_t compress_on,
                                             const int32_t* keep, const int32_t* nk, void* y_text, void* y_video,
                                             void* y_audio, void* stream) {
    size_t need = 0;
    int r = dit_block_workspace_size(dims, compress_on, &need);   // validates dims
    if (r) return r;
    if (dims->n_ctrl != 0) return DIT_EINVAL;
    if (need > SCRATCH_BYTES) return DIT_EWORKSPACE;
    void* ws = nullptr;
    if ((r = scratch_ptr(&ws))) return r;
    return dit::block_forward_impl(dims, x_text, x_video, nullptr, nullptr, 0, x_audio, weights, compress_on, keep, nk,
                                   y_text, y_video, nullptr, y_audio, ws, SCRATCH_BYTES, stream);
}
