// gemm_dtl_f8.hip -- the direct-to-LDS matrix-core kernels for f8 inputs
// (see gemm_dtl.hpp).
#include "gemm_dtl.hpp"

namespace dg {

hipError_t launch_mfma_dtl_f8(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream) {
    return dtl::launch_tiles<IN_F8>(tile, a_mode, b_mode, args, stream);
}

}  // namespace dg
