// epilogue.hip -- split-K reduction and the alpha == 0 / K == 0 scaling of C.
//
// Split-K (sheratonhq.com deep dive, section 5.2): partial sums of S slices of K
// arrive in an FP32 workspace [S][M][N]; this kernel adds them in the fixed
// order s = 0..S-1, so a plan always produces the same bits, then applies
// out = act(alpha * sum + beta * C_in + bias) and rounds to the C dtype.
// When alpha == 0 (or K == 0) the product is never formed: C <- act(beta * C +
// bias), and with beta == 0 C is not read (kwkr.cn article, section 4.3,
// records a kernel that skipped the beta scaling when alpha was 0).
#include "device_common.hpp"

namespace dg {
namespace {

constexpr int NT = 256;

__global__ void __launch_bounds__(NT) splitk_reduce(ReduceArgs p) {
    const int64_t total = (int64_t)p.M * p.N;
    const int64_t plane = total;
    for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * NT) {
        const float s = sum_partials(p.S, [&](int z) { return p.ws[idx + z * plane]; });
        const int64_t m = idx / p.N, n = idx - m * p.N;
        epilogue_store(p.epi, m, n, s);
    }
}

__global__ void __launch_bounds__(NT) scale_c(ScaleArgs p) {
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * NT) {
        const int64_t m = idx / p.N, n = idx - m * p.N;
        char *q = p.epi.C + m * p.epi.c_rs + n * p.epi.c_cs;
        float v = (p.epi.beta != 0.0f) ? p.epi.beta * load_out(q, p.epi.out_kind) : 0.0f;
        if (p.epi.bias) v += load_bias(p.epi, n);
        store_out(q, p.epi.out_kind, activate(p.epi.act, v));
    }
}

// n ints <- 0: the split-K arrival counters of a new workspace block (a kernel,
// not hipMemsetAsync, so that a caller may capture the call in a HIP graph).
__global__ void __launch_bounds__(NT) fill_zero(int *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = 0;
}

int blocks_for(int64_t total) {
    int64_t b = (total + NT - 1) / NT;
    if (b > 65536) b = 65536;
    return (int)(b > 0 ? b : 1);
}

}  // namespace

hipError_t launch_fill_zero(int *p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero, dim3(blocks_for(n)), dim3(NT), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs &args, hipStream_t stream) {
    hipLaunchKernelGGL(splitk_reduce, dim3(blocks_for((int64_t)args.M * args.N)), dim3(NT), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_scale(const ScaleArgs &args, hipStream_t stream) {
    hipLaunchKernelGGL(scale_c, dim3(blocks_for((int64_t)args.M * args.N)), dim3(NT), 0, stream, args);
    return hipGetLastError();
}

}  // namespace dg
