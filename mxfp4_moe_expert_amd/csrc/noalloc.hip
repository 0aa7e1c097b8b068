// noalloc.hip -- k3g_moe_layer_static: the MoE layer on a library-owned,
// statically sized device scratch array, for callers that cannot allocate
// (code under HIP graph capture, serving loops that forbid hipMalloc).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, from module load to process end.
// Host code never passes the array's name to a kernel (on the host that name
// is a stand-in, not a device address); it asks the runtime for the current
// device's address once, keeps it per device, and hands that pointer to
// k3g_moe_layer as its workspace. Nothing here allocates.
#include <mutex>

#include "k3g_common.h"

static __device__ __align__(256) unsigned char scratch[K3G_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // per device: the array's device address, once looked up

// The current device's copy of `scratch`, looked up on the first call on that
// device (with it current). Returns K3G_OK and *out, or K3G_EHIP.
int scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return K3G_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return K3G_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return K3G_EHIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return K3G_OK;
}

}  // namespace

extern "C" {

size_t k3g_static_scratch_bytes(void) { return (size_t)K3G_STATIC_SCRATCH_BYTES; }

int k3g_moe_layer_static(float *y, const float *x, const int32_t *idx, const float *wts,
                         const k3g_expert_bank *bank, int n_tokens, int top_k, int mode, void *stream) {
    if (!bank || n_tokens < 0) return K3G_EINVAL;
    const k3g_shape s = {n_tokens, top_k, bank->n_experts, bank->latent, bank->inter, 0, 0, mode};
    const size_t need = k3g_workspace_bytes(K3G_OP_MOE_LAYER, &s);
    if (need == 0) return K3G_EINVAL;
    if (need > (size_t)K3G_STATIC_SCRATCH_BYTES) return K3G_ENOSPACE;  // beyond the array: refused
    if (n_tokens == 0)  // an empty batch enqueues nothing (validated as k3g_moe_layer does)
        return k3g_moe_layer(y, x, idx, wts, bank, 0, top_k, mode, nullptr, 0, stream);
    void *ws = nullptr;
    const int rc = scratch_ptr(&ws);
    if (rc != K3G_OK) return rc;
    return k3g_moe_layer(y, x, idx, wts, bank, n_tokens, top_k, mode, ws, (size_t)K3G_STATIC_SCRATCH_BYTES,
                         stream);
}

}  // extern "C"
