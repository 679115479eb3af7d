// quant.hpp -- argument block and launcher of the FP8 E4M3 quantizer (host and device).
#pragma once
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace dg {

struct QuantArgs {
    const char *X; int64_t x_rs, x_cs;   // M x K input, byte strides
    char *Q; int64_t q_rs, q_cs;         // M x K E4M3 codes
    float *S; int64_t s_rs, s_cs;        // scales, byte strides
    int M, K;
    int tiles_k;                         // ceil(K / 128): the 128-wide K blocks (scale columns)
    int block;                           // 0: one scale per row and 128 K; 1: per 128 x 128
    int x_vec;                           // X rows K-contiguous, 16-byte aligned 8-element chunks
    int q_vec;                           // Q rows K-contiguous, 8-byte aligned 8-element chunks
};

// x_dtype: DG_F32, DG_F16 or DG_BF16; cus: compute units of the device (sizes
// the persistent grid).
hipError_t launch_quant(int x_dtype, const QuantArgs &args, hipStream_t stream, int cus);

}  // namespace dg
