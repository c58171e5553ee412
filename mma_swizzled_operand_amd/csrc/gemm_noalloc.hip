// gemm_noalloc.hip — gemm_run_ws for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the split weight-streaming path's fp32 partials go to a
// scratch array the library owns instead of a caller workspace.
//
// The array is a file-scope device variable of kScratchBytes, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// its name to a kernel (on the host the name is only a stand-in, not a device
// address): on the first call on a device, with that device current, its
// device address is looked up with hipGetSymbolAddress and kept per device,
// and that address is what the kernels receive.  Every call on one GPU shares
// that GPU's copy, which keeps the last call's contents; the split path
// writes every partial before reading it, so nothing needs clearing.  Calls
// that overlap on one GPU (different streams, or host threads racing on one
// stream) race on the array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mswz_gemm.h"

namespace {

constexpr int64_t kScratchBytes = int64_t(16) << 20;   // 16 MiB: the 64 x 16384 x 8192 weight-streaming shape
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of the current device's copy of the scratch array.
int scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MSWZ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MSWZ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MSWZ_OK;
}

}  // namespace

extern "C" {

int64_t gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gemm_run_ws_noalloc(const gemm_plan *plan, const void *A, const void *B, void *D, int beta, void *stream)
{
    if (!plan)
        return MSWZ_ERR_INVALID;
    const int64_t need = gemm_plan_workspace_size(plan);
    if (need < 0)
        return int(need);
    if (need > kScratchBytes)
        return MSWZ_ERR_SCRATCH;
    if (need == 0)   // no split path: gemm_run, which uses no scratch
        return gemm_run(plan, A, B, D, beta, stream);
    if (!A || !B || !D)
        return MSWZ_ERR_INVALID;
    void *ptr = nullptr;
    const int rc = scratch_ptr(&ptr);
    if (rc != MSWZ_OK)
        return rc;
    return gemm_run_ws(plan, A, B, D, beta, ptr, kScratchBytes, stream);
}

}  // extern "C"
