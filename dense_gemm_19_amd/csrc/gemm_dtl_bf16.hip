// gemm_dtl_bf16.hip -- the direct-to-LDS matrix-core kernels for bf16 inputs
// (see gemm_dtl.hpp).
#include "gemm_dtl.hpp"

namespace dg {

hipError_t launch_mfma_dtl_bf16(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream) {
    return dtl::launch_tiles<IN_BF16>(tile, a_mode, b_mode, args, stream);
}

hipError_t launch_mfma_dtl_grouped_bf16(int tile, int a_mode, int b_mode, const GroupedMfmaArgs &args, int units,
                                     hipStream_t stream) {
    return dtl::launch_grouped_tiles<IN_BF16>(tile, a_mode, b_mode, args, units, stream);
}

}  // namespace dg
