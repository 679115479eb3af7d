// skinny.hip -- bandwidth-bound thin GEMM (M <= 8) without matrix cores.
//
// The articles single out thin shapes such as x[1,4096] . W1[4096,14336] (an MoE
// FFN up-projection) and q[1,4096] . K_cache^T (a 128-key cache): with M this
// small the work is one pass over B, so the kernels stream B exactly once with
// 16-byte loads, multiply on the vector ALUs, and reduce with cross-lane
// shuffles and LDS instead of issuing matrix-core instructions ("DeepGEMM is
// not a new model" article, cf-1.com, sections 2 and 4; sheratonhq.com deep
// dive, section 5.4).  Every output element has one writer and partial sums
// are added in a fixed order, never with floating-point atomics (cf-1.com
// article, section 4.5), so results are reproducible.
//
// SK_BN: B is N-contiguous (row-major [K][N], e.g. W1).  A workgroup of 8 waves
//   owns a slab of p.cols columns and one split of K.  W = 32 lanes cover a row
//   piece (slabs of at most 256 columns): lane (r, c), r = lane/32, c = lane%32,
//   owns columns 8c..8c+7 of the slab and, in each 128-row sweep, the 8
//   consecutive rows 8*(2*wave + r) + u, u < 8, so every load instruction of a
//   wave reads two whole row pieces.  W = 64 (slabs of up to 512 columns, M <= 4):
//   lane c owns columns 8c..8c+7 and the rows 8*wave + u of 64-row sweeps, one
//   row piece of up to 1 KB per load instruction.  Lanes with 8c >= p.cols load
//   nothing of B.  The A values a lane needs are 16-byte LDS reads.  The slab
//   width and the K split are planned together so that slabs x splits fill the
//   CUs once with whole 128-byte lines per row piece (x.W1, N = 14336: 32 slabs
//   of 448 columns x 8 splits = 256 workgroups).
//   A's K slice is staged in LDS as 16-bit values [m][k], with the first
//   sweep's loads of B already in flight.  The two row groups of a wave are
//   summed with a shuffle and the 8 waves through LDS, always in the same
//   order.  K is split so that the grid holds at most one workgroup per CU;
//   the last workgroup of a slab to finish (an arrival counter) adds the S
//   partials in the order s = 0..S-1, so the sum does not depend on timing.
// skinny_bn_grouped runs several SK_BN problems in one grid: the experts of an
//   MoE layer, each a small GEMM such as [1,512] x [512,4096] (cf-1.com
//   article, section 1), whose separate launches would each pay the launch
//   cost (section 5.1 of that article) and leave most CUs idle.
// SK_BK: B is K-contiguous (B = K_cache^T: column n is row n of the cache).  A
//   wave owns one column; lanes take 8 consecutive K values each per 512-wide K
//   step, with up to 8 steps' loads of B and A issued before any is used, then a
//   wave reduction with shuffles.  Workgroups hold 1 wave when N is small (to
//   spread the columns over many compute units) and 4 otherwise.
// SK_BK with grid.y = S > 1 splits K too, and a reduction kernel sums the FP32
// partials in a fixed order.
#include "device_common.hpp"

namespace dg {
namespace {

// 16-byte chunk of 8 bf16/f16 values -> 8 floats.
template <int IN>
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = v[q];
        if (IN == IN_BF16) {
            f[2 * q] = __builtin_bit_cast(float, w << 16);
            f[2 * q + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
        } else {
            f[2 * q] = f16_bits_to_f32((uint16_t)(w & 0xffff));
            f[2 * q + 1] = f16_bits_to_f32((uint16_t)(w >> 16));
        }
    }
}

template <int IN>
__device__ __forceinline__ float to_f32(uint16_t b) {
    return IN == IN_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// ------------------------------------------------------------------ SK_BN

// Global-address-space view of 16 bytes (keeps loads "global", not "flat").
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
// 16 zero bytes in device memory: the source of out-of-range row loads.
__device__ __attribute__((aligned(16))) const u32x4 g_zero16 = {0u, 0u, 0u, 0u};

constexpr int BN_NT = SKINNY_BN_THREADS;        // 8 waves
constexpr int BN_WAVES = BN_NT / 64;
constexpr int BN_U = 8;                         // consecutive rows per lane per sweep
static_assert(SKINNY_BN_SWEEP % (BN_WAVES * BN_U) == 0, "splits and chunks are whole sweeps");

// One workgroup's share of an SK_BN problem: column slab `slab`, K split `z`.
// W lanes cover a row piece of a slab (W * 8 columns at most): W = 32, two row
// pieces of up to 512 bytes per load instruction of a wave; W = 64, one piece
// of up to 1 KB.
template <int MMAX, int IN, int W>
__device__ __forceinline__ void skinny_bn_body(const SkinnyArgs &p, const int slab, const int z) {
    constexpr int BN_W = W;                     // lanes per row
    constexpr int BN_R = 64 / BN_W;             // rows per load instruction of a wave
    constexpr int BN_COLS = BN_W * 8;           // most columns per workgroup
    constexpr int BN_SWEEP = BN_WAVES * BN_R * BN_U;
    static_assert(SKINNY_BN_SWEEP % BN_SWEEP == 0, "planner sweeps are whole kernel sweeps");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // LDS: A chunk as 16-bit values [MMAX][kc] (kc a multiple of BN_SWEEP), later
    // reused for the cross-wave reduction red[wave][m][BN_COLS].
    uint16_t *la = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem);
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % BN_W, r = lane / BN_W;
    const int cols = p.cols;
    const int n0 = slab * cols + c * 8;
    const int kb = z * p.k_per_split;
    const int ke = min(kb + p.k_per_split, p.K);
    // A lane whose 8 columns all lie in the slab and in the matrix streams
    // them with 16-byte loads.  The other lanes run the same code on the
    // 16-byte zero block (row stride 0), so the loop stays uniform: lanes past
    // the slab's width or past N contribute nothing, and the one lane whose
    // columns straddle N (a ragged last slab) adds its columns with element
    // loads after each chunk's sweeps.
    const bool in_slab = c * 8 < cols;
    const bool vec = in_slab && n0 + 8 <= p.N;
    const bool straddle = in_slab && n0 < p.N && n0 + 8 > p.N;
    const char *bcol = vec ? p.B + (int64_t)n0 * p.b_cs : reinterpret_cast<const char *>(&g_zero16);
    const int64_t brs = vec ? p.b_rs : 0;

    float acc[MMAX][8];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

    const int lrow = wave * (BN_R * BN_U) + r * BN_U;   // first of the lane's rows in a sweep

    auto fma_sweep = [&](const u32x4 (&v)[BN_U], int k) {   // k: the lane's first row in the chunk
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            // A[m][k .. k+7]: one 16-byte LDS read (zero beyond the chunk end)
            const u32x4 av = *reinterpret_cast<const u32x4 *>(la + m * p.kc + k);
            float a[8];
            unpack8<IN>(av, a);
#pragma unroll
            for (int u = 0; u < BN_U; ++u) {
                float b[8];
                unpack8<IN>(v[u], b);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(a[u], b[j], acc[m][j]);
            }
        }
    };

    // Split and chunk boundaries are multiples of the sweep, so every sweep is
    // whole except, possibly, the last one of K; only that one needs guards.
    for (int c0 = kb; c0 < ke; c0 += p.kc) {
        const int c1 = min(c0 + p.kc, ke);
        const int clen = c1 - c0;
        const int nfull = clen / BN_SWEEP;   // whole sweeps of this chunk
        // The first sweep's loads of B go out before A is staged.  They are
        // issued unconditionally (from the 16-byte zero block when there is no
        // whole sweep), so the wait for A below is exactly "all but these 8".
        const bool first = nfull > 0;
        const char *fb = first ? bcol + (int64_t)(c0 + lrow) * brs : reinterpret_cast<const char *>(&g_zero16);
        const int64_t fs = first ? brs : 0;
        u32x4 v[BN_U];

        // Stage A[0..MMAX)[c0..c1) in LDS (rows >= M and k >= c1 as zeros).  With
        // A rows K-contiguous and 16-byte aligned and K a multiple of 8 (a_vec;
        // then every chunk length is a multiple of 8 and a 16-byte piece that
        // starts inside the chunk ends inside it), every thread first issues one
        // 16-byte piece of A (threads past the end read the zero block and
        // write a spare LDS slot), then the 8 loads of B, and only then stores A
        // to LDS.
        const int achunks = MMAX * (p.kc / 8);
        auto a_chunk = [&](int idx, int &off) {
            const int m = idx / (p.kc / 8), k = (idx - m * (p.kc / 8)) * 8;
            off = m * p.kc + k;
            const bool in = m < p.M && k < clen;
            const char *q = in ? p.A + (int64_t)m * p.a_rs + (int64_t)(c0 + k) * 2
                               : reinterpret_cast<const char *>(&g_zero16);
            return *(const gu32x4 *)q;
        };
        int a_off = 0;
        u32x4 a_first = u32x4{0u, 0u, 0u, 0u};
        if (p.a_vec) {
            a_first = a_chunk(tid < achunks ? tid : 0, a_off);
            if (tid >= achunks) a_off = MMAX * p.kc;   // the spare slot
        }
#pragma unroll
        for (int u = 0; u < BN_U; ++u)
            v[u] = __builtin_nontemporal_load((const gu32x4 *)(fb + u * fs));
        __builtin_amdgcn_sched_barrier(0);
        if (c0 != kb) __syncthreads();   // the previous chunk's A is no longer read
        if (p.a_vec) {
            *reinterpret_cast<u32x4 *>(la + a_off) = a_first;
            for (int idx = tid + BN_NT; idx < achunks; idx += BN_NT) {
                int off;
                const u32x4 x = a_chunk(idx, off);
                *reinterpret_cast<u32x4 *>(la + off) = x;
            }
        } else {
            for (int idx = tid; idx < MMAX * p.kc; idx += BN_NT) {
                const int m = idx / p.kc, k = idx - m * p.kc;
                uint16_t x = 0;
                if (m < p.M && k < clen)
                    x = *reinterpret_cast<const uint16_t *>(p.A + (int64_t)m * p.a_rs + (int64_t)(c0 + k) * p.a_cs);
                la[idx] = x;
            }
        }
        __syncthreads();

        // whole sweeps: plain loads, then the multiply
        for (int s = 0; s < nfull; ++s) {
            const int k = s * BN_SWEEP + lrow;
            if (s > 0) {
                const char *q = bcol + (int64_t)(c0 + k) * brs;
#pragma unroll
                for (int u = 0; u < BN_U; ++u)
                    v[u] = __builtin_nontemporal_load((const gu32x4 *)(q + u * brs));
            }
            fma_sweep(v, k);
        }
        // the partial last sweep of K (full slab), with per-row guards
        if (nfull * BN_SWEEP < clen) {
            const int k = nfull * BN_SWEEP + lrow;
#pragma unroll
            for (int u = 0; u < BN_U; ++u) {
                v[u] = u32x4{0u, 0u, 0u, 0u};
                if (k + u < clen) v[u] = *(const gu32x4 *)(bcol + (int64_t)(c0 + k + u) * brs);
            }
            fma_sweep(v, k);
        }
        if (straddle) {
            // ragged right edge: element loads; columns beyond N contribute nothing
            for (int k = lrow; k < clen; k += BN_SWEEP) {
                for (int u = 0; u < BN_U && k + u < clen; ++u) {
                    const char *q = p.B + (int64_t)(c0 + k + u) * p.b_rs;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (n0 + j < p.N) {
                            const float b = to_f32<IN>(*reinterpret_cast<const uint16_t *>(q + (int64_t)(n0 + j) * p.b_cs));
#pragma unroll
                            for (int m = 0; m < MMAX; ++m)
                                acc[m][j] = fmaf(to_f32<IN>(la[m * p.kc + k + u]), b, acc[m][j]);
                        }
                    }
                }
            }
        }
    }

    // Sum the two row groups of a wave (W = 32: lanes c and c + 32), then the 8
    // waves through LDS: red[wave][m][BN_COLS], always in the same order.
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (BN_R == 2) acc[m][j] += __shfl_xor(acc[m][j], 32);
    __syncthreads();   // the A chunk is no longer needed
    if (lane < BN_W) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int j = 0; j < 8; ++j) red[(wave * MMAX + m) * BN_COLS + lane * 8 + j] = acc[m][j];
    }
    __syncthreads();
    for (int t = tid; t < MMAX * cols; t += BN_NT) {
        const int m = t / cols, col = t - m * cols;
        const int n = slab * cols + col;
        if (m < p.M && n < p.N) {
            float s = red[m * BN_COLS + col];
#pragma unroll
            for (int w = 1; w < BN_WAVES; ++w) s += red[(w * MMAX + m) * BN_COLS + col];
            if (p.splits > 1)   // agent-scope store: coherent across the XCDs' L2 caches
                __hip_atomic_store(p.ws + ((int64_t)z * p.M + m) * p.N + n, s, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            else epilogue_store(p.epi, m, n, s);
        }
    }
    if (p.splits == 1) return;

    // K was split over grid.y: the last workgroup of this column slab to finish
    // adds the S partials in the order s = 0..S-1 (so the bits do not depend on
    // which workgroup finishes last), applies the epilogue, and re-arms the
    // slab's counter for the next call on this stream.  The partials are
    // written and read with agent-scope atomic accesses; each thread waits
    // until its partial stores have completed, then the workgroup takes its
    // ticket (take_last_ticket states why the workgroup holding the last
    // ticket sees every partial).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) is_last = take_last_ticket(p.counters + slab, p.splits);
    __syncthreads();
    if (!is_last) return;
    const int64_t plane = (int64_t)p.M * p.N;
    for (int t = tid; t < MMAX * cols; t += BN_NT) {
        const int m = t / cols, col = t - m * cols;
        const int n = slab * cols + col;
        if (m < p.M && n < p.N) {
            float *w = p.ws + (int64_t)m * p.N + n;
            const float s = sum_partials(p.splits, [&](int q) {
                return __hip_atomic_load(w + q * plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            });
            epilogue_store(p.epi, m, n, s);
        }
    }
    if (tid == 0) __hip_atomic_store(p.counters + slab, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MMAX, int IN, int W>
__global__ void __launch_bounds__(BN_NT) skinny_bn(SkinnyArgs p) {
    skinny_bn_body<MMAX, IN, W>(p, blockIdx.x, blockIdx.y);
}

// Several SK_BN problems in one grid (the experts of an MoE layer, say): the
// group of this workgroup is found by a scan of at most SKINNY_GROUP_MAX
// uniform values, then the workgroup runs exactly what skinny_bn would.
template <int MMAX, int IN, int W>
__global__ void __launch_bounds__(BN_NT) skinny_bn_grouped(GroupedSkinnyArgs p) {
    const int u = blockIdx.x;
    int g = 0;
    while (g + 1 < p.ngroups && u >= p.unit_begin[g + 1]) ++g;
    const int local = u - p.unit_begin[g];
    skinny_bn_body<MMAX, IN, W>(p.g[g], local % p.slabs[g], local / p.slabs[g]);
}

// ------------------------------------------------------------------ SK_BK

// 512-wide K steps whose loads are in flight together (fewer for larger M, so
// the A chunks still fit in registers)
template <int MMAX> struct BkSteps { static constexpr int v = MMAX == 1 ? 8 : MMAX == 2 ? 4 : 2; };

template <int MMAX, int IN>
__global__ void __launch_bounds__(256) skinny_bk(SkinnyArgs p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * (blockDim.x >> 6) + wave;
    const int z = blockIdx.y;
    const int kb = z * p.k_per_split;
    const int ke = min(kb + p.k_per_split, p.K);
    if (n >= p.N) return;   // whole wave leaves together; no barrier follows
    const char *bcol = p.B + (int64_t)n * p.b_cs;
    float acc[MMAX];
#pragma unroll
    for (int m = 0; m < MMAX; ++m) acc[m] = 0.f;
    // vector part: 16-byte chunks of 8 K values, A and B both K-contiguous and aligned
    const int kv_end = p.a_vec ? kb + ((ke - kb) / 8) * 8 : kb;
    constexpr int BK_STEPS = BkSteps<MMAX>::v;
    for (int k0 = kb; k0 < kv_end; k0 += 512 * BK_STEPS) {
        u32x4 bv[BK_STEPS], av[BK_STEPS][MMAX];
#pragma unroll
        for (int t = 0; t < BK_STEPS; ++t) {
            const int k = k0 + t * 512 + lane * 8;
            if (k < kv_end) {
                bv[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(bcol + (int64_t)k * p.b_rs));
#pragma unroll
                for (int m = 0; m < MMAX; ++m)
                    av[t][m] = (m < p.M) ? *reinterpret_cast<const u32x4 *>(p.A + (int64_t)m * p.a_rs + (int64_t)k * p.a_cs)
                                         : u32x4{0u, 0u, 0u, 0u};
            } else {
                bv[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int m = 0; m < MMAX; ++m) av[t][m] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int t = 0; t < BK_STEPS; ++t) {
            float b[8];
            unpack8<IN>(bv[t], b);
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                float a[8];
                unpack8<IN>(av[t][m], a);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[m] = fmaf(a[j], b[j], acc[m]);
            }
        }
    }
    // scalar tail (or everything, if A is not K-contiguous)
    for (int k = kv_end + lane; k < ke; k += 64) {
        const float b = to_f32<IN>(*reinterpret_cast<const uint16_t *>(bcol + (int64_t)k * p.b_rs));
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
            if (m < p.M)
                acc[m] = fmaf(to_f32<IN>(*reinterpret_cast<const uint16_t *>(p.A + (int64_t)m * p.a_rs + (int64_t)k * p.a_cs)),
                              b, acc[m]);
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

template <int MMAX, int IN, int W>
hipError_t launch_bn(const SkinnyArgs &a, dim3 grid, int lds, hipStream_t s) {
    if (lds > 48 * 1024) {
        static int attr = 0;   // benign race: setting the attribute twice is harmless
        if (lds > attr) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(skinny_bn<MMAX, IN, W>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            attr = lds;
        }
    }
    hipLaunchKernelGGL((skinny_bn<MMAX, IN, W>), grid, dim3(BN_NT), lds, s, a);
    return hipGetLastError();
}

template <int MMAX, int IN>
hipError_t launch_k(int kind, const SkinnyArgs &a, int grid_x, int waves, hipStream_t s) {
    dim3 grid(grid_x, a.splits);
    if (kind == SK_BN) {
        const int lds = skinny_bn_lds(MMAX, a.kc, a.cols);
        if (a.cols > 256) return launch_bn<MMAX, IN, 64>(a, grid, lds, s);
        return launch_bn<MMAX, IN, 32>(a, grid, lds, s);
    } else {
        hipLaunchKernelGGL((skinny_bk<MMAX, IN>), grid, dim3(64 * waves), 0, s, a);
    }
    return hipGetLastError();
}

template <int IN>
hipError_t launch_m(int kind, int m_max, const SkinnyArgs &a, int grid_x, int waves, hipStream_t s) {
    switch (m_max) {
    case 1: return launch_k<1, IN>(kind, a, grid_x, waves, s);
    case 2: return launch_k<2, IN>(kind, a, grid_x, waves, s);
    case 4: return launch_k<4, IN>(kind, a, grid_x, waves, s);
    case 8: return launch_k<8, IN>(kind, a, grid_x, waves, s);
    }
    return hipErrorInvalidValue;
}

template <int MMAX, int IN, int W>
hipError_t launch_grouped_w(const GroupedSkinnyArgs &a, int units, int lds, hipStream_t s) {
    if (lds > 48 * 1024) {
        static int attr = 0;   // benign race: setting the attribute twice is harmless
        if (lds > attr) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(skinny_bn_grouped<MMAX, IN, W>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            attr = lds;
        }
    }
    hipLaunchKernelGGL((skinny_bn_grouped<MMAX, IN, W>), dim3(units), dim3(BN_NT), lds, s, a);
    return hipGetLastError();
}

template <int MMAX, int IN>
hipError_t launch_grouped_k(bool wide, const GroupedSkinnyArgs &a, int units, int lds, hipStream_t s) {
    return wide ? launch_grouped_w<MMAX, IN, 64>(a, units, lds, s) : launch_grouped_w<MMAX, IN, 32>(a, units, lds, s);
}

template <int IN>
hipError_t launch_grouped_m(int m_max, bool wide, const GroupedSkinnyArgs &a, int units, int lds, hipStream_t s) {
    switch (m_max) {
    case 1: return launch_grouped_k<1, IN>(wide, a, units, lds, s);
    case 2: return launch_grouped_k<2, IN>(wide, a, units, lds, s);
    case 4: return launch_grouped_k<4, IN>(wide, a, units, lds, s);
    case 8: return launch_grouped_k<8, IN>(wide, a, units, lds, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_skinny(int kind, int m_max, const SkinnyArgs &args, int grid_x, int waves,
                         hipStream_t stream) {
    if (args.in_kind == IN_BF16) return launch_m<IN_BF16>(kind, m_max, args, grid_x, waves, stream);
    return launch_m<IN_F16>(kind, m_max, args, grid_x, waves, stream);
}

hipError_t launch_skinny_grouped(int in_kind, int m_max, bool wide, const GroupedSkinnyArgs &args, int units,
                                 int lds_bytes, hipStream_t stream) {
    if (in_kind == IN_BF16) return launch_grouped_m<IN_BF16>(m_max, wide, args, units, lds_bytes, stream);
    return launch_grouped_m<IN_F16>(m_max, wide, args, units, lds_bytes, stream);
}

}  // namespace dg
