// noalloc.hip -- the fixed device scratch of dg_gemm_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) still need split-K
// scratch: FP32 partial sums and the arrival counters of the kernels that sum
// them.  Here it is one file-scope device array, `scratch`, of a fixed size,
// which every GPU the library runs on holds from module load until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory:
// the array's device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept, and only that address is ever
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace dg {

// [0, NOALLOC_WS_BYTES): FP32 partials; then NOALLOC_COUNTERS ints of counters.
static __device__ __align__(256) char scratch[NOALLOC_WS_BYTES + NOALLOC_COUNTERS * sizeof(int)];

namespace {

struct ScratchTable {
    std::mutex mu;
    char *ptr[64] = {};   // per device id: the device address of `scratch`
};

ScratchTable &scratch_table() {
    static ScratchTable t;
    return t;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, float **ws, int **counters) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    ScratchTable &t = scratch_table();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.ptr[dev]) {
        void *p = nullptr;
        if ((err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        // The counters start at zero (the array is zero-initialized when the
        // module loads); zero them once more, in order on this first call's
        // stream, and every kernel that uses them leaves them at zero.
        if ((err = launch_fill_zero(reinterpret_cast<int *>(static_cast<char *>(p) + NOALLOC_WS_BYTES),
                                    NOALLOC_COUNTERS, stream)) != hipSuccess)
            return err;
        t.ptr[dev] = static_cast<char *>(p);
    }
    *ws = reinterpret_cast<float *>(t.ptr[dev]);
    *counters = reinterpret_cast<int *>(t.ptr[dev] + NOALLOC_WS_BYTES);
    return hipSuccess;
}

}  // namespace dg
