// dion_step_batched_noalloc: the Dion step with its scratch in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The step's kernels are those of dion_step_batched;
// only where their workspace comes from differs.
//
// `scratch` below is a file-scope device array of kNoAllocScratchBytes.  Each GPU that loads this
// library holds its own copy until the process ends.  Host code never passes the array's name
// to a kernel (on the host it names a stand-in, not device memory): the device address of each
// GPU's copy is looked up once per device, with that device current, by hipGetSymbolAddress on
// the entry point's first call there, and kept; every later use goes through that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dion.h"
#include "dion_plan.h"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)DION_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch (looked up once per device).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int dion_step_batched_noalloc(void* X, const void* G, float* M, float* Q, int64_t m, int64_t n, int64_t batch,
                              int64_t rank, float mu, float lr, float eps, int x_dtype, int g_dtype,
                              int32_t* flags, uint32_t options, void* stream) {
    dion::Plan p;
    int st = dion::check_step_args(m, n, batch, rank, mu, lr, eps, x_dtype, g_dtype, options, &p);
    if (st != DION_OK) return st;
    // one chunk only: the concurrent chunks run on library streams created on first use
    if (((options >> DION_OPT_CHUNKS_SHIFT) & 15u) > 1u) return DION_ERR_OPTION;
    if (p.total > kNoAllocScratchBytes) return DION_ERR_SCRATCH;
    if (batch == 0) return DION_OK;
    if (!X || !G || !M || (rank > 0 && !Q)) return DION_ERR_NULL;   // before the first HIP call
    void* ws = nullptr;
    const hipError_t he = scratch_address(&ws);
    if (he != hipSuccess) return DION_ERR_HIP - (int)he;
    st = dion::check_step_buffers(p, X, G, M, Q, x_dtype, g_dtype, ws, kNoAllocScratchBytes, flags);
    if (st != DION_OK) return st;
    const int e = dion::run_step(p, X, G, M, Q, mu, lr, eps, x_dtype == DION_BF16, g_dtype == DION_BF16, (char*)ws,
                                 flags, (options & ~(15u << DION_OPT_CHUNKS_SHIFT)) | (1u << DION_OPT_CHUNKS_SHIFT),
                                 stream, nullptr);
    return e ? DION_ERR_HIP - e : DION_OK;
}

}  // extern "C"
