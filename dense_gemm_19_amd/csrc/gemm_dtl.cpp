// gemm_dtl.cpp -- dispatch of the direct-to-LDS matrix-core kernels by input type.
#include "kernels.hpp"

namespace dg {

hipError_t launch_mfma_dtl_f16(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream);
hipError_t launch_mfma_dtl_bf16(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream);
hipError_t launch_mfma_dtl_f8_two_stage(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream);
hipError_t launch_mfma_dtl_f8_deep(int tile, int a_mode, int b_mode, const MfmaArgs &args, hipStream_t stream);

hipError_t launch_mfma_dtl_grouped_f16(int tile, int a_mode, int b_mode, const GroupedMfmaArgs &args, int units,
                                     hipStream_t stream);
hipError_t launch_mfma_dtl_grouped_bf16(int tile, int a_mode, int b_mode, const GroupedMfmaArgs &args, int units,
                                      hipStream_t stream);

bool mfma_dtl_tile(int tile) { return tile >= 0 && tile < NUM_MFMA_TILES; }

hipError_t launch_mfma_dtl(int in_kind, int tile, int a_mode, int b_mode, const MfmaArgs &args,
                           hipStream_t stream) {
    switch (in_kind) {
    case IN_F16: return launch_mfma_dtl_f16(tile, a_mode, b_mode, args, stream);
    case IN_BF16: return launch_mfma_dtl_bf16(tile, a_mode, b_mode, args, stream);
    case IN_F8:   // (256x256 and 128x128, the two-stage tiles, in one unit; the others in another)
        return tile == T256x256 || tile == T128x128 ? launch_mfma_dtl_f8_two_stage(tile, a_mode, b_mode, args, stream)
                                                    : launch_mfma_dtl_f8_deep(tile, a_mode, b_mode, args, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mfma_dtl_grouped(int in_kind, int tile, int a_mode, int b_mode, const GroupedMfmaArgs &args,
                                   int units, hipStream_t stream) {
    switch (in_kind) {
    case IN_F16: return launch_mfma_dtl_grouped_f16(tile, a_mode, b_mode, args, units, stream);
    case IN_BF16: return launch_mfma_dtl_grouped_bf16(tile, a_mode, b_mode, args, units, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
