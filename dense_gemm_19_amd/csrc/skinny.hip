// skinny.hip -- bandwidth-bound thin GEMM (M <= 8) without matrix cores.
//
// The pages single out thin shapes such as x[1,4096] . W1[4096,14336] (an MoE
// FFN up-projection) and q[1,4096] . K_cache^T (a 128-key cache): with M this
// small the work is one pass over B, so the kernel is built to stream B exactly
// once with 16-byte loads and reduce with cross-lane shuffles instead of
// issuing matrix-core instructions ("DeepGEMM is not a new model" article,
// cf-1.com, sections 2 and 4; sheratonhq.com deep dive, section 5.4).  The
// stores are plain, one writer per output element, with no atomics (cf-1.com
// article, section 4.5).
//
// SK_BN: B is N-contiguous (row-major [K][N], e.g. W1).  A workgroup owns 64
//   columns; each lane owns 8 adjacent columns (one 16-byte load per K row) and
//   every 32nd K row of the workgroup's K slice; the 32 K groups of the
//   workgroup are summed with cross-lane shuffles, then through LDS, always in
//   the same order.  A's K slice is staged in LDS as [k][m] so one LDS read
//   broadcasts A[0..M)[k] to a whole K group.
// SK_BK: B is K-contiguous (B = K_cache^T, each column a contiguous row of the
//   cache).  A wave owns one column; lanes stride K with 16-byte loads of B and
//   A, and the wave reduces with shuffles.
// With grid.y = S > 1 the K range is split and FP32 partials go to a workspace
// that the reduction kernel sums in a fixed order.
#include "device_common.hpp"

namespace dg {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ void unpack8(u32x4 v, int in_kind, float (&f)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = v[q];
        if (in_kind == IN_BF16) {
            f[2 * q] = __builtin_bit_cast(float, w << 16);
            f[2 * q + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
        } else {
            f[2 * q] = f16_bits_to_f32((uint16_t)(w & 0xffff));
            f[2 * q + 1] = f16_bits_to_f32((uint16_t)(w >> 16));
        }
    }
}

__device__ __forceinline__ float load_in(const char *p, int in_kind) {
    const uint16_t b = *reinterpret_cast<const uint16_t *>(p);
    return in_kind == IN_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// ------------------------------------------------------------------ SK_BN

constexpr int BN_COLS = 64;              // columns per workgroup (8 lanes x 8)
constexpr int BN_KG = NT / 8;            // K groups per workgroup
constexpr int BN_UNROLL = 8;             // 16-byte B loads in flight per lane

template <int MMAX, int IN>
__global__ void __launch_bounds__(NT) skinny_bn(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // LDS: A slice as float [k_per_split][MMAX], then the reduction buffer.
    float *la = reinterpret_cast<float *>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tc = tid & 7;              // column group within the workgroup
    const int kg = tid >> 3;             // K group 0..31
    const int n0 = blockIdx.x * BN_COLS + tc * 8;
    const int z = blockIdx.y;
    const int kb = z * p.k_per_split;
    const int ke = min(kb + p.k_per_split, p.K);
    const int klen = ke - kb;

    // Stage A[0..M)[kb..ke) into LDS as [k][m] FP32.
    for (int idx = tid; idx < klen * MMAX; idx += NT) {
        const int k = idx / MMAX, m = idx - k * MMAX;
        float v = 0.f;
        if (m < p.M) v = load_in(p.A + (int64_t)m * p.a_rs + (int64_t)(kb + k) * p.a_cs, IN);
        la[idx] = v;
    }
    __syncthreads();

    float acc[MMAX][8];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[m][c] = 0.f;

    const bool full = n0 + 8 <= p.N;
    const char *bcol = p.B + (int64_t)n0 * p.b_cs;
    if (full) {
        // main stream: rows kb + kg + BN_KG * t
        int k = kg;
        for (; k + BN_KG * (BN_UNROLL - 1) < klen; k += BN_KG * BN_UNROLL) {
            u32x4 v[BN_UNROLL];
#pragma unroll
            for (int u = 0; u < BN_UNROLL; ++u)
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    bcol + (int64_t)(kb + k + BN_KG * u) * p.b_rs));
#pragma unroll
            for (int u = 0; u < BN_UNROLL; ++u) {
                float b[8];
                unpack8(v[u], IN, b);
                const float *ar = la + (k + BN_KG * u) * MMAX;
#pragma unroll
                for (int m = 0; m < MMAX; ++m) {
                    const float a = ar[m];
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[m][c] = fmaf(a, b[c], acc[m][c]);
                }
            }
        }
        for (; k < klen; k += BN_KG) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(bcol + (int64_t)(kb + k) * p.b_rs);
            float b[8];
            unpack8(v, IN, b);
            const float *ar = la + k * MMAX;
#pragma unroll
            for (int m = 0; m < MMAX; ++m)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[m][c] = fmaf(ar[m], b[c], acc[m][c]);
        }
    } else {
        // ragged right edge: element loads, columns beyond N contribute nothing
        for (int k = kg; k < klen; k += BN_KG) {
            const float *ar = la + k * MMAX;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (n0 + c < p.N) {
                    const float b = load_in(p.B + (int64_t)(kb + k) * p.b_rs + (int64_t)(n0 + c) * p.b_cs, IN);
#pragma unroll
                    for (int m = 0; m < MMAX; ++m) acc[m][c] = fmaf(ar[m], b, acc[m][c]);
                }
            }
        }
    }

    // Reduce the 8 K groups of a wave (lanes differing in bits 3..5), fixed order.
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v = acc[m][c];
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[m][c] = v;
        }
    // Then the 4 waves through LDS: red[wave][m][64 columns].
    __syncthreads();   // A slice no longer needed
    float *red = la;
    if (lane < 8) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int c = 0; c < 8; ++c) red[(wave * MMAX + m) * BN_COLS + lane * 8 + c] = acc[m][c];
    }
    __syncthreads();
    for (int idx = tid; idx < MMAX * BN_COLS; idx += NT) {
        const int m = idx / BN_COLS, col = idx - m * BN_COLS;
        const int n = blockIdx.x * BN_COLS + col;
        if (m >= p.M || n >= p.N) continue;
        float s = red[(0 * MMAX + m) * BN_COLS + col];
        s += red[(1 * MMAX + m) * BN_COLS + col];
        s += red[(2 * MMAX + m) * BN_COLS + col];
        s += red[(3 * MMAX + m) * BN_COLS + col];
        if (p.splits > 1) p.ws[((int64_t)z * p.M + m) * p.N + n] = s;
        else epilogue_store(p.epi, m, n, s);
    }
}

// ------------------------------------------------------------------ SK_BK

template <int MMAX, int IN>
__global__ void __launch_bounds__(NT) skinny_bk(SkinnyArgs p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * (NT / 64) + wave;
    const int z = blockIdx.y;
    const int kb = z * p.k_per_split;
    const int ke = min(kb + p.k_per_split, p.K);
    if (n >= p.N) return;   // whole wave leaves together; no barrier follows
    const char *bcol = p.B + (int64_t)n * p.b_cs;
    float acc[MMAX];
#pragma unroll
    for (int m = 0; m < MMAX; ++m) acc[m] = 0.f;
    // vector part: chunks of 8 K values, both A and B K-contiguous and aligned
    const int kv_end = p.a_vec ? kb + ((ke - kb) / 8) * 8 : kb;
    for (int k = kb + lane * 8; k < kv_end; k += 64 * 8) {
        float b[8];
        unpack8(*reinterpret_cast<const u32x4 *>(bcol + (int64_t)k * p.b_rs), IN, b);
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < p.M) {
                float a[8];
                unpack8(*reinterpret_cast<const u32x4 *>(p.A + (int64_t)m * p.a_rs + (int64_t)k * p.a_cs), IN, a);
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[m] = fmaf(a[c], b[c], acc[m]);
            }
        }
    }
    // scalar tail (or everything, if A is not K-contiguous)
    for (int k = kv_end + lane; k < ke; k += 64) {
        const float b = load_in(bcol + (int64_t)k * p.b_rs, IN);
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
            if (m < p.M) acc[m] = fmaf(load_in(p.A + (int64_t)m * p.a_rs + (int64_t)k * p.a_cs, IN), b, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
        float v = acc[m];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        acc[m] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < p.M) {
                if (p.splits > 1) p.ws[((int64_t)z * p.M + m) * p.N + n] = acc[m];
                else epilogue_store(p.epi, m, n, acc[m]);
            }
        }
    }
}

template <int MMAX, int IN>
hipError_t launch_k(int kind, const SkinnyArgs &a, int grid_x, hipStream_t s) {
    dim3 grid(grid_x, a.splits);
    if (kind == SK_BN) {
        const int kmax = a.k_per_split;
        const int lds = max(kmax * MMAX * 4, 4 * MMAX * BN_COLS * 4);
        auto k = skinny_bn<MMAX, IN>;
        static int attr = 0;
        if (lds > attr) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            attr = lds;
        }
        hipLaunchKernelGGL(k, grid, dim3(NT), lds, s, a);
    } else {
        hipLaunchKernelGGL((skinny_bk<MMAX, IN>), grid, dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <int IN>
hipError_t launch_m(int kind, int m_max, const SkinnyArgs &a, int grid_x, hipStream_t s) {
    switch (m_max) {
    case 1: return launch_k<1, IN>(kind, a, grid_x, s);
    case 2: return launch_k<2, IN>(kind, a, grid_x, s);
    case 4: return launch_k<4, IN>(kind, a, grid_x, s);
    case 8: return launch_k<8, IN>(kind, a, grid_x, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_skinny(int kind, int m_max, const SkinnyArgs &args, int grid_x, hipStream_t stream) {
    if (args.in_kind == IN_BF16) return launch_m<IN_BF16>(kind, m_max, args, grid_x, stream);
    return launch_m<IN_F16>(kind, m_max, args, grid_x, stream);
}

}  // namespace dg
