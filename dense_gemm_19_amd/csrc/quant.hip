// quant.hip -- FP8 E4M3 quantizer: per 1 x 128 (token) or 128 x 128 block,
// s = max(amax, 1e-12) / 448 and q = E4M3(clamp(x / s, -448, 448)), rounded to
// nearest with ties to an even code (include/dg.h states the operation and
// cites the pages).
//
// One workgroup of 256 threads owns a tile of X: 128 x 128 for block scales,
// 16 x 512 (four 128-wide K blocks) for token scales where K >= 512, else
// 64 x 128.  Thread t holds the 8-element chunk cc = t % CPR of rows
// r0 + (256 / CPR) i, r0 = t / CPR, with CPR = 16 chunks per row (128-column
// tiles: each wave load covers 4 rows x 128 columns) or 64 (512-column tiles:
// each wave load covers one row x 512 columns, 1 KB of 16-bit X, the row
// piece width at which a streaming read of this part reaches its peak).  The
// 16 lanes of a 128-wide row block are adjacent either way: the row maxima come
// from four shuffle steps, the block maximum from two more and one LDS
// exchange between the four waves.  X is read once (16-byte loads where rows
// are K-contiguous) and the codes of a chunk leave as one 8-byte store; with
// 512-column tiles a row's four token scales leave from four adjacent lanes.
// The work is a stream: 3 bytes per element for 16-bit X, 5 for FP32.  Both
// the 16-byte loads of X and the 8-byte code stores are nontemporal (neither
// is touched again by this kernel; measured on MI355X: 4096 x 4096 BF16 per
// token 14.55 -> 12.87 us, 4096 x 7168 per block 20.9 -> 18.7 us; nontemporal
// loads alone 14.3 and 19.8 us).
#include "dg.h"
#include "device_common.hpp"
#include "quant.hpp"

namespace dg {
namespace {

constexpr float E4M3_MAX = 448.0f;
// Row steps per thread of the 512-column token tiles (16 x 512 tiles; measured
// on 4096 x 4096 BF16: 8 x 512 15.2 us, 16 x 512 14.5 us, 32 x 512 18.1 us;
// with nontemporal accesses 8 x 512 14.2 us, 16 x 512 13.0 us, 32 x 512 13.8 us).
constexpr int QRT = 4;

// x / s rounded to nearest, given r = RN(1/s): t = RN(x * r) is within one ulp
// of the quotient, the FMA residual x - t * s is exact, and one correction
// t + residual * r rounds to the correctly rounded quotient (Markstein's
// theorem).  Here |x / s| <= 448 (s is the block's amax / 448), so nothing
// overflows; where the quotient would be subnormal, i.e. far below the
// smallest E4M3 step, any residual error cannot change the code.  The sign is
// that of x (s > 0): the correction of x = -0 would otherwise give +0.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
    const float t = x * r;
    const float e = fmaf(-t, s, x);
    return __builtin_copysignf(fmaf(e, r, t), x);
}

// E4M3FN codes (OCP FP8: bias 7, 3 mantissa bits, subnormals m * 2^-9,
// largest finite 448) of four finite values with |v| <= 448, rounded to
// nearest with ties to even: gfx950's packed FP32 -> FP8 conversion, which
// produces exactly these codes (it matched an arithmetic encoder on 7.6 M
// values from 2^-20 to 448, and the parity tests check every E4M3 midpoint).
// Byte j of the result is the code of v[j].
__device__ __forceinline__ uint32_t e4m3_codes4(float v0, float v1, float v2, float v3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    return (uint32_t)w;
}

// An 8-element chunk of X as raw 32-bit words: 8 FP32 values, or 4 pairs of
// 16-bit values (low half first).
template <int XT> struct Chunk { static constexpr int W = XT == DG_F32 ? 8 : 4; uint32_t w[W]; };

template <int XT>
__device__ __forceinline__ uint32_t load_bits(const char *p) {
    if (XT == DG_F32) return *reinterpret_cast<const uint32_t *>(p);
    return *reinterpret_cast<const uint16_t *>(p);
}

template <int XT>
__device__ __forceinline__ float chunk_value(const Chunk<XT> &c, int j) {
    if (XT == DG_F32) return __builtin_bit_cast(float, c.w[j]);
    const uint16_t h = (uint16_t)(j & 1 ? c.w[j >> 1] >> 16 : c.w[j >> 1] & 0xffffu);
    return XT == DG_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// 32 zero bytes in device memory: the source of the vector loads of chunks
// outside X (rows past M, or a tile past the last one).
__device__ __attribute__((aligned(16))) const u32x4 g_qzero[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};

// The thread's RT chunks of tile `tile`: rows r0 + RS i of the tile's RS*RT rows
// (RS = 256 / CPR), columns 8 cc .. 8 cc + 7 of its 8 * CPR; zeros outside X.  VEC (X rows
// K-contiguous with 16-byte aligned chunks, K a multiple of 8): one or two
// 16-byte loads per chunk, every one issued (chunks outside X read the zero
// block), with no branch, so the compiler's wait before the first use of a
// tile counts exactly the loads issued after it.  Otherwise element loads.
template <int XT, int RT, bool VEC, int CPR>
__device__ __forceinline__ void load_tile(const QuantArgs &p, int tile, int r0, int cc, Chunk<XT> (&buf)[RT]) {
    constexpr int RS = 256 / CPR, TC = 8 * CPR;
    const int tiles_kw = (p.K + TC - 1) / TC;
    const int mb = tile / tiles_kw, kw = tile - mb * tiles_kw;
    const int c0 = kw * TC + cc * 8;
    const int nvalid = min(8, p.K - c0);
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int row = mb * RS * RT + r0 + RS * i;
        const char *xr = p.X + (int64_t)row * p.x_rs;
        if constexpr (VEC) {
            const char *src = row < p.M && nvalid > 0 ? xr + (int64_t)c0 * (XT == DG_F32 ? 4 : 2)
                                                      : reinterpret_cast<const char *>(g_qzero);
#pragma unroll
            for (int h = 0; h < Chunk<XT>::W / 4; ++h) {
                const u32x4 q = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(src + 16 * h));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = q[j];   // (an element copied to a scalar before any bit cast)
                    buf[i].w[4 * h + j] = w;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t b = (row < p.M && j < nvalid) ? load_bits<XT>(xr + (int64_t)(c0 + j) * p.x_cs) : 0u;
                if (XT == DG_F32) buf[i].w[j] = b;
                else if (j & 1) buf[i].w[j >> 1] |= b << 16;
                else buf[i].w[j >> 1] = b;
            }
        }
    }
}

// Quantize one tile from the thread's chunks: row maxima, scales, codes, stores.
template <int XT, int RT, int CPR>
__device__ __forceinline__ void quant_tile(const QuantArgs &p, int tile, int t, int r0, int cc,
                                           const Chunk<XT> (&buf)[RT], float *wave_max) {
    constexpr int RS = 256 / CPR, TC = 8 * CPR;
    static_assert(CPR == 16 || CPR == 64, "16 or 64 chunks per row");
    const int tiles_kw = (p.K + TC - 1) / TC;
    const int mb = tile / tiles_kw, kw = tile - mb * tiles_kw;
    const int kb = kw * (CPR / 16) + (cc >> 4);   // this lane's 128-wide K block
    const int c0 = kw * TC + cc * 8;
    const int nvalid = min(8, p.K - c0);
    // row maxima over the 16 lanes of each row block (out-of-range elements are 0)
    float s[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(chunk_value<XT>(buf[i], j)));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        s[i] = a;
    }
    if (!p.block) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            s[i] = fmaxf(s[i], 1e-12f) / E4M3_MAX;
            const int row = mb * RS * RT + r0 + RS * i;
            if ((cc & 15) == 0 && row < p.M && kb * 128 < p.K)
                *reinterpret_cast<float *>(reinterpret_cast<char *>(p.S) + (int64_t)row * p.s_rs +
                                           (int64_t)kb * p.s_cs) = s[i];
        }
    } else {
        float a = s[0];
#pragma unroll
        for (int i = 1; i < RT; ++i) a = fmaxf(a, s[i]);
        a = fmaxf(a, __shfl_xor(a, 16));
        a = fmaxf(a, __shfl_xor(a, 32));
        if ((t & 63) == 0) wave_max[t >> 6] = a;
        __syncthreads();
        a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
        const float sc = fmaxf(a, 1e-12f) / E4M3_MAX;
#pragma unroll
        for (int i = 0; i < RT; ++i) s[i] = sc;
        if (t == 0)
            *reinterpret_cast<float *>(reinterpret_cast<char *>(p.S) + (int64_t)mb * p.s_rs +
                                       (int64_t)kb * p.s_cs) = sc;
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int row = mb * RS * RT + r0 + RS * i;
        if (row >= p.M || nvalid <= 0) continue;
        const float r = 1.0f / s[i];
        float c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c[j] = fminf(fmaxf(div_by_scale(chunk_value<XT>(buf[i], j), s[i], r), -E4M3_MAX), E4M3_MAX);
        const uint32_t lo = e4m3_codes4(c[0], c[1], c[2], c[3]);
        const uint32_t hi = e4m3_codes4(c[4], c[5], c[6], c[7]);
        char *qr = p.Q + (int64_t)row * p.q_rs;
        if (nvalid == 8 && p.q_vec) {
            __builtin_nontemporal_store((uint64_t)lo | ((uint64_t)hi << 32), reinterpret_cast<uint64_t *>(qr + c0));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < nvalid)
                    *reinterpret_cast<uint8_t *>(qr + (int64_t)(c0 + j) * p.q_cs) =
                        (uint8_t)((j < 4 ? lo : hi) >> (8 * (j & 3)));
        }
    }
}

// RT: chunks (row steps) per thread (CPR 16: 8 for 128 x 128 tiles, 4 for
// 64 x 128 token tiles; CPR 64: 4 for 16 x 512 token tiles).  Each workgroup
// walks tiles bid, bid + grid, ... with the next tile's loads in flight while
// it quantizes and stores the current one, so that the reads and writes of the
// whole grid overlap instead of running in two waves.
template <int XT, int RT, bool VEC, int CPR>
__global__ void __launch_bounds__(256) quant_fp8(QuantArgs p, int ntiles) {
    __shared__ float wave_max[2][4];   // (double-buffered: the next tile writes the other half)
    const int t = threadIdx.x, cc = t % CPR, r0 = t / CPR;
    Chunk<XT> b0[RT], b1[RT];
    // The loads of a tile past the last one are issued too: its rows lie past M,
    // so they read nothing and give zeros.  Unconditional loads keep the wait
    // before each quantization exact (a load under a condition makes the
    // compiler wait for every load in flight, the next tile's included).
    int tile = blockIdx.x;
    load_tile<XT, RT, VEC, CPR>(p, tile, r0, cc, b0);
    for (; tile < ntiles; tile += 2 * gridDim.x) {
        const int t1 = tile + gridDim.x, t2 = t1 + gridDim.x;
        load_tile<XT, RT, VEC, CPR>(p, t1, r0, cc, b1);
        quant_tile<XT, RT, CPR>(p, tile, t, r0, cc, b0, wave_max[0]);
        if (t1 >= ntiles) break;
        load_tile<XT, RT, VEC, CPR>(p, t2, r0, cc, b0);
        quant_tile<XT, RT, CPR>(p, t1, t, r0, cc, b1, wave_max[1]);
    }
}

}  // namespace

hipError_t launch_quant(int x_dtype, const QuantArgs &a, hipStream_t stream, int cus) {
    // Token scales: 16 x 512 tiles (64 x 128 where K < 512); block scales need
    // the whole 128 x 128 block in one workgroup.  A persistent grid walks them.
    const bool wide = !a.block && a.K >= 512;
    const int rows = a.block ? 128 : wide ? 4 * QRT : 64, cols = wide ? 512 : 128;
    const int64_t ntiles = (int64_t)((a.M + rows - 1) / rows) * ((a.K + cols - 1) / cols);
    // 4 (token scales) or 2 (block scales) workgroups per CU, each walking its
    // tiles with the next tile's loads in flight (measured with nontemporal
    // accesses: 1, 2, 4 per CU -> A 4096x4096 per token 16.8, 12.9, 12.5 us; B
    // 4096x7168 per block 24.1, 18.7, 20.1 us).
    const int64_t want = (int64_t)(cus > 0 ? cus : 256) * (a.block ? 2 : 4);
    const dim3 grid((unsigned)(ntiles < want ? ntiles : want)), block(256);
    const int n = (int)ntiles;
    const bool vec = a.x_vec && a.K % 8 == 0;
#define DG_QUANT_LAUNCH(XT, RT, CPR)                                                                  \
    do {                                                                                              \
        if (vec) hipLaunchKernelGGL((quant_fp8<XT, RT, true, CPR>), grid, block, 0, stream, a, n);   \
        else hipLaunchKernelGGL((quant_fp8<XT, RT, false, CPR>), grid, block, 0, stream, a, n);      \
    } while (0)
    if (a.block) {
        if (x_dtype == DG_F32) DG_QUANT_LAUNCH(DG_F32, 8, 16);
        else if (x_dtype == DG_F16) DG_QUANT_LAUNCH(DG_F16, 8, 16);
        else DG_QUANT_LAUNCH(DG_BF16, 8, 16);
    } else if (wide) {
        if (x_dtype == DG_F32) DG_QUANT_LAUNCH(DG_F32, QRT, 64);
        else if (x_dtype == DG_F16) DG_QUANT_LAUNCH(DG_F16, QRT, 64);
        else DG_QUANT_LAUNCH(DG_BF16, QRT, 64);
    } else {
        if (x_dtype == DG_F32) DG_QUANT_LAUNCH(DG_F32, 4, 16);
        else if (x_dtype == DG_F16) DG_QUANT_LAUNCH(DG_F16, 4, 16);
        else DG_QUANT_LAUNCH(DG_BF16, 4, 16);
    }
#undef DG_QUANT_LAUNCH
    return hipGetLastError();
}

}  // namespace dg
