// gemm_dtl_f8.hip -- the direct-to-LDS matrix-core kernels for f8 inputs with
// a two-stage ring (256x256, 128x128; see gemm_dtl.hpp).  The other f8 tiles
// are in gemm_dtl_f8s.hip, a translation unit of their own so that the two
// compile side by side.
#include "gemm_dtl.hpp"

namespace dg {

hipError_t launch_mfma_dtl_f8_two_stage(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream) {
    return dtl::launch_tiles_part<IN_F8, true>(tile, a_mode, b_mode, args, stream);
}

}  // namespace dg
