// gemm_dtl_f8s.hip -- the direct-to-LDS matrix-core kernels for f8 inputs with
// deeper rings (128x64, 64x64, 64x128; see gemm_dtl.hpp and gemm_dtl_f8.hip).
#include "gemm_dtl.hpp"

namespace dg {

hipError_t launch_mfma_dtl_f8_deep(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream) {
    return dtl::launch_tiles_part<IN_F8, false>(tile, a_mode, b_mode, args, stream);
}

}  // namespace dg
