// quant.hip -- FP8 E4M3 quantizer: per 1 x 128 (token) or 128 x 128 block,
// s = max(amax, 1e-12) / 448 and q = E4M3(clamp(x / s, -448, 448)), rounded to
// nearest with ties to an even code (include/dg.h states the operation and
// cites the pages).
//
// One workgroup of 256 threads owns a 128 x 128 tile of X.  Thread t holds the
// 8-element chunk cc = t % 16 of rows r0 + 16 i, r0 = t / 16, i < 8, so the 16
// lanes of a row block are adjacent: the row maxima come from four shuffle
// steps, the tile maximum from two more and one LDS exchange between the four
// waves.  X is read once (16-byte loads where rows are K-contiguous) and the
// codes of a chunk leave as one 8-byte store.  The work is a stream: 3 bytes
// per element for 16-bit X, 5 for FP32.
#include "dg.h"
#include "device_common.hpp"
#include "quant.hpp"

namespace dg {
namespace {

constexpr float E4M3_MAX = 448.0f;

// E4M3FN code of a finite v with |v| <= 448 (OCP FP8: bias 7, 3 mantissa
// bits, subnormals m * 2^-9, largest finite 448 = 1.75 * 2^8), rounded to
// nearest with ties to even.  Below 2^-6 the value is a multiple of 2^-9;
// above, a 3-bit mantissa at the value's binary exponent.  Scaling by powers
// of two is exact, so the only rounding is the one rint does (ties to even).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8; 8 is 2^-6, code 0x08
    } else {
        int e;
        (void)__builtin_frexpf(a, &e);                  // a = f * 2^e, f in [0.5, 1)
        int ex = e - 1;                                 // a in [2^ex, 2^(ex+1)), ex in [-6, 8]
        uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - ex));   // 8..16
        if (m == 16u) {
            m = 8u;
            ex += 1;
        }
        code = ((uint32_t)(ex + 7) << 3) | (m - 8u);
    }
    return sign | code;
}

template <int XT>
__device__ __forceinline__ float load_x(const char *p) {
    if (XT == DG_F32) return *reinterpret_cast<const float *>(p);
    const uint16_t b = *reinterpret_cast<const uint16_t *>(p);
    return XT == DG_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

template <int XT>
__global__ void __launch_bounds__(256) quant_fp8(QuantArgs p) {
    __shared__ float wave_max[4];
    const int t = threadIdx.x, cc = t & 15, r0 = t >> 4;
    const int mb = blockIdx.x / p.tiles_k, kb = blockIdx.x - mb * p.tiles_k;
    const int c0 = kb * 128 + cc * 8;
    const int nvalid = min(8, p.K - c0);   // columns of this chunk inside X (may be <= 0)

    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = mb * 128 + r0 + 16 * i;
        const char *xr = p.X + (int64_t)row * p.x_rs;
        if (row < p.M && nvalid == 8 && p.x_vec) {
            if (XT == DG_F32) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(xr + (int64_t)c0 * 4);
                const u32x4 b = *reinterpret_cast<const u32x4 *>(xr + (int64_t)c0 * 4 + 16);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // (copy each vector element to a scalar first: a bit cast of
                    // the element expression itself reads element 0 here)
                    const uint32_t wa = a[j], wb = b[j];
                    v[i][j] = __builtin_bit_cast(float, wa);
                    v[i][4 + j] = __builtin_bit_cast(float, wb);
                }
            } else {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(xr + (int64_t)c0 * 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint16_t lo = (uint16_t)(a[j] & 0xffffu), hi = (uint16_t)(a[j] >> 16);
                    v[i][2 * j] = XT == DG_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
                    v[i][2 * j + 1] = XT == DG_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[i][j] = (row < p.M && j < nvalid) ? load_x<XT>(xr + (int64_t)(c0 + j) * p.x_cs) : 0.0f;
        }
    }

    // row maxima over the 16 lanes of each row block (out-of-range elements are 0)
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[i][j]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        s[i] = a;
    }
    if (!p.block) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = fmaxf(s[i], 1e-12f) / E4M3_MAX;
            const int row = mb * 128 + r0 + 16 * i;
            if (cc == 0 && row < p.M)
                *reinterpret_cast<float *>(reinterpret_cast<char *>(p.S) + (int64_t)row * p.s_rs +
                                           (int64_t)kb * p.s_cs) = s[i];
        }
    } else {
        float a = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) a = fmaxf(a, s[i]);
        a = fmaxf(a, __shfl_xor(a, 16));
        a = fmaxf(a, __shfl_xor(a, 32));
        if ((t & 63) == 0) wave_max[t >> 6] = a;
        __syncthreads();
        a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
        const float sc = fmaxf(a, 1e-12f) / E4M3_MAX;
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = sc;
        if (t == 0)
            *reinterpret_cast<float *>(reinterpret_cast<char *>(p.S) + (int64_t)mb * p.s_rs +
                                       (int64_t)kb * p.s_cs) = sc;
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = mb * 128 + r0 + 16 * i;
        if (row >= p.M || nvalid <= 0) continue;
        uint32_t code[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) code[j] = e4m3_code(fminf(fmaxf(v[i][j] / s[i], -E4M3_MAX), E4M3_MAX));
        char *qr = p.Q + (int64_t)row * p.q_rs;
        if (nvalid == 8 && p.q_vec) {
            const uint32_t lo = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
            const uint32_t hi = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
            *reinterpret_cast<uint64_t *>(qr + c0) = (uint64_t)lo | ((uint64_t)hi << 32);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < nvalid) *reinterpret_cast<uint8_t *>(qr + (int64_t)(c0 + j) * p.q_cs) = (uint8_t)code[j];
        }
    }
}

}  // namespace

hipError_t launch_quant(int x_dtype, const QuantArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)((a.M + 127) / 128) * a.tiles_k)), block(256);
    if (x_dtype == DG_F32) hipLaunchKernelGGL(quant_fp8<DG_F32>, grid, block, 0, stream, a);
    else if (x_dtype == DG_F16) hipLaunchKernelGGL(quant_fp8<DG_F16>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(quant_fp8<DG_BF16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace dg
