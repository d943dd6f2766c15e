// Allocation-free forward: cluster_attn_forward_opts with the workspace taken
// from one file-scope device array per GPU instead of from the caller, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this library's code object, so every GPU the library
// runs on holds its own copy of CA_NOALLOC_SCRATCH_BYTES until the process
// ends. Host code never hands the array's name to a kernel: in host code that
// name is a stand-in, not a device address. The device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept; the kernels receive it as their workspace.
#include <mutex>

#include "launch.h"

static __device__ __align__(256) unsigned char scratch[CA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];   // device address of each GPU's copy; null until looked up

// Device address of the current device's copy of scratch.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" ca_status_t cluster_attn_forward_noalloc(const void *Q, const void *K, const void *V,
                                                    int B, int H, int L, int d, int nclust,
                                                    int iters, int W, float alpha,
                                                    const ca_options_t *opts, void *out,
                                                    int32_t *assign_out, ca_dtype_t dt,
                                                    ca_path_t path, hipStream_t stream) {
    // The workspace this call needs (0 on the single-launch paths, and for
    // arguments that the forward itself rejects below).
    const size_t need = cluster_attn_workspace_size_ex(B, H, L, d, nclust, dt, path);
    if (need > (size_t)CA_NOALLOC_SCRATCH_BYTES) return CA_ERR_SCRATCH_TOO_SMALL;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        if (scratch_address(&ws) != hipSuccess) return CA_ERR_HIP;
        ws_bytes = CA_NOALLOC_SCRATCH_BYTES;
    }
    // Nothing in the workspace has to start at zero: every buffer the staged
    // kernels read is written earlier in the same call.
    return cluster_attn_forward_opts(Q, K, V, B, H, L, d, nclust, iters, W, alpha, opts, out,
                                     assign_out, dt, ws, ws_bytes, path, stream);
}
