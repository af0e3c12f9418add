// rn_forward_noalloc: rn_forward_ex with the split-row workspace taken from a static device
// array of the library instead of the caller (include/rownorm.h).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy
// from the first use of the library's code on it until the process ends. In host code its
// name is only a host-side stand-in for the symbol, not a device address; the device address
// comes from hipGetSymbolAddress, once per device, with that device current, and only that
// address is ever passed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/rownorm.h"

namespace {

constexpr size_t kScratchBytes = RN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // the current device's address of `scratch`, once looked up

// The device address of this device's `scratch`, or nullptr on a HIP error.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> g(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int rn_forward_noalloc(
    int op, const void* x, const void* residual, const void* gamma, const void* beta, void* y, void* residual_out,
    float* mean, float* rstd, int64_t rows, int64_t N, float eps, int dtype, const rn_row_strides* strides,
    hipStream_t stream) {
    // the scratch is needed only by the split-row paths; its size follows the shape
    const size_t need = rn_forward_workspace_bytes(op, rows, N, dtype);
    if (need > kScratchBytes) return RN_ERR_SCRATCH;
    // the argument checks first, on the host (planned without a workspace, which only changes
    // the kernel choice), so that a bad call returns before any HIP call
    const int st = rn_plan(op, x, residual, gamma, beta, y, residual_out, mean, rstd, rows, N, eps, dtype,
                           RN_VARIANT_AUTO, strides, nullptr, 0, nullptr);
    if (st != RN_OK && st != RN_ERR_WORKSPACE) return st;
    void* ws = nullptr;
    if (need > 0 && rows > 0) {
        ws = scratch_ptr();
        if (ws == nullptr) return RN_ERR_HIP;
    }
    return rn_forward_ex(op, x, residual, gamma, beta, y, residual_out, mean, rstd, rows, N, eps, dtype, strides,
                         RN_VARIANT_AUTO, ws, need, stream);
}
