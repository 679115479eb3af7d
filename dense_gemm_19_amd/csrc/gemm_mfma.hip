// gemm_mfma.hip -- matrix-core (MFMA) GEMM for gfx950.
//
// C = alpha * A * B + beta * C with FP32 accumulation (kwkr.cn view-native GEMM
// article, section 2.3; xdnf.cn methodology, section 3.1), and the FP8 E4M3
// variant whose per-token / per-128x128-block scales are applied in the kernel
// once per 128-wide K block (sheratonhq.com deep dive, section 2.4).
//
// Structure (sheratonhq.com deep dive, sections 2.1-2.3 and 3.3, re-derived for
// CDNA4 with 64-wide waves and 160 KB of LDS):
//  * one workgroup of 4 waves (2 x 2) owns a BM x BN macro tile of C; each wave a
//    (BM/2) x (BN/2) sub-tile of 16x16 MFMA blocks held in FP32 registers;
//  * K is walked in tiles of 128 bytes (64 FP16/BF16 or 128 FP8 elements),
//    staged HBM -> registers -> LDS with 16-byte coalesced loads into a
//    two-stage LDS ring: the next tile's global loads are in flight while the
//    current tile is multiplied; one barrier per K tile;
//  * K-contiguous operands are kept [rows][K] in LDS and read with 16-byte LDS
//    reads; M/N-contiguous operands (row-major B) are copied as they are,
//    [K][rows], and transposed on the way out with the gfx950 LDS transpose
//    reads, so no operand is reshaped in memory;
//  * LDS rows are XOR-swizzled in 16-byte chunks so that the 16 lanes of a
//    fragment read hit distinct banks (the padding/swizzle advice of the
//    sheratonhq.com deep dive, sections 3.4 and 4.3);
//  * a workgroup index -> tile map keeps groups of tiles that share A and B
//    panels on one XCD (blocks are dealt round-robin over the 8 XCDs, each of
//    which has its own L2);
//  * split-K: grid.z slices K and writes FP32 partials that a second kernel sums
//    in a fixed order (sheratonhq.com deep dive, section 5.2), so results are
//    bitwise reproducible (no float atomics).
//
// MFMA operand layouts used (checked on the device):
//  v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[l%16][8*(l/16) + j] and
//    B[8*(l/16) + j][l%16], j = 0..7; D[4*(l/16) + e][l%16], e = 0..3.
//  v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3): lane l holds 32 K values of row
//    (A) / column (B) l%16, the same K set for A and B; D as above.
//  ds_read_b64_tr_b16: within each 16-lane group, result lane j element e comes
//    from the lane (4e + j/4)'s 8-byte address, element j%4.
//  ds_read_b64_tr_b8: result lane j byte e comes from lane (2e + j/8), byte j%8.
#include "device_common.hpp"

namespace dg {
namespace {

constexpr int NT = 256;          // threads per workgroup (4 waves)
constexpr int KBYTES = 128;      // bytes of K per tile

template <int IN> struct InT;
template <> struct InT<IN_F16>  { static constexpr int EB = 2; static constexpr int KSTEPS = 2; };
template <> struct InT<IN_BF16> { static constexpr int EB = 2; static constexpr int KSTEPS = 2; };
template <> struct InT<IN_F8>   { static constexpr int EB = 1; static constexpr int KSTEPS = 1; };

// ------------------------------------------------------------------ LDS layout

// KMAJ: [R][128 B], chunk c of row r stored at chunk c ^ (r & 7).
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * KBYTES + ((c ^ (r & 7)) << 4); }

// MNMAJ: [BK][R * EB bytes]; chunk c of K-row k stored at chunk c ^ swz(k).
// 16-bit: a transpose read touches 4 consecutive K rows x 2 adjacent chunks per
// 16-lane group; the XOR keeps chunk pairs adjacent (even values) and spreads
// the 4 rows, and the 4 groups of a wave (K bits 3-4), over distinct banks.
// 8-bit: a read touches 8 consecutive K rows x 1 chunk per group.
template <int EB, int CPR>
__device__ __forceinline__ int mn_swz(int k) {
    int s;
    // 16-bit rows of 128 bytes (8 chunks): rows k and k + 2 (and k + 8, read by
    // the next lane group) share a bank half; K bits 1 and 3 pick the chunk pair.
    if (EB == 2 && CPR == 8) s = (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1;
    else if (EB == 2) s = ((k & 3) << 1) | (((k >> 3) & 3) << 3);
    else s = (k & 7) | (((k >> 5) & 3) << 3);
    return s & (CPR - 1);
}
template <int EB, int R>
__device__ __forceinline__ int mnmaj_off(int k, int c) {
    constexpr int CPR = R * EB / 16;
    return k * (R * EB) + ((c ^ mn_swz<EB, CPR>(k)) << 4);
}

// ------------------------------------------------------------------ global -> regs -> LDS

// One operand tile: R rows (M for A, N for B) x 128 bytes of K = R*8 chunks of
// 16 bytes; NCH chunks per thread.
//  SLOW == 0: every chunk is either wholly inside the matrix or wholly outside
//             (K % (16/EB) == 0, 16-byte aligned rows); outside chunks load a
//             clamped in-range address and are zeroed with a select, so the
//             loads are branch-free.
//  SLOW == 1: any strides and alignment; element-wise loads with bounds checks.
template <int MODE, int R, int EB, int SLOW>
struct TileIO {
    static constexpr int CHUNKS = R * 8;
    static constexpr int NCH = CHUNKS / NT;
    static constexpr int EPC = 16 / EB;        // elements per chunk
    static constexpr int CPR = R * EB / 16;    // chunks per K row (MNMAJ)
    static_assert(CHUNKS % NT == 0, "tile must give every thread whole chunks");

    // chunk index -> (row within tile, K index within tile) of its first element
    __device__ static void coords(int c, int &r, int &k) {
        if (MODE == KMAJ) { r = c >> 3; k = (c & 7) * EPC; }
        else { k = c / CPR; r = (c % CPR) * EPC; }
    }

    __device__ static void load(u32x4 (&reg)[NCH], const Operand &op, int r0, int k0, int Rlim,
                                int Klim, int tid) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            int r, k;
            coords(tid + i * NT, r, k);
            const int gr = r0 + r, gk = k0 + k;
            if (!SLOW) {
                const bool in = (MODE == KMAJ) ? (gr < Rlim && gk < Klim) : (gk < Klim && gr < Rlim);
                const int cr = in ? gr : 0, ck = in ? gk : 0;
                u32x4 v = *reinterpret_cast<const u32x4 *>(op.ptr + (int64_t)cr * op.r_stride +
                                                           (int64_t)ck * op.k_stride);
                reg[i] = in ? v : u32x4{0u, 0u, 0u, 0u};
            } else {
                uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const int rr = (MODE == KMAJ) ? gr : gr + e;
                    const int kk = (MODE == KMAJ) ? gk + e : gk;
                    if (rr < Rlim && kk < Klim) {
                        const char *p = op.ptr + (int64_t)rr * op.r_stride + (int64_t)kk * op.k_stride;
                        uint32_t v = (EB == 2) ? *reinterpret_cast<const uint16_t *>(p)
                                               : *reinterpret_cast<const uint8_t *>(p);
                        w[(e * EB) >> 2] |= v << (((e * EB) & 3) * 8);
                    }
                }
                reg[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }

    __device__ static void store(char *lds, const u32x4 (&reg)[NCH], int tid) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT;
            const int off = (MODE == KMAJ) ? kmaj_off(c >> 3, c & 7) : mnmaj_off<EB, R>(c / CPR, c % CPR);
            *reinterpret_cast<u32x4 *>(lds + off) = reg[i];
        }
    }
};

// ------------------------------------------------------------------ fragments

// 16-bit fragment (8 elements) of the 16 rows starting at rb, K step ks (32 K).
template <int MODE, int R>
__device__ __forceinline__ u32x4 frag16(const char *lds, int rb, int ks, int lane) {
    if (MODE == KMAJ) {
        const int r = rb + (lane & 15);
        const int c = ks * 4 + (lane >> 4);
        return *reinterpret_cast<const u32x4 *>(lds + kmaj_off(r, c));
    } else {
        const int s = lane & 15, g = lane >> 4;
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = ks * 32 + 8 * g + 4 * q + (s >> 2);
            const int byte = (rb + 4 * (s & 3)) * 2;
            const int off = mnmaj_off<2, R>(k, byte >> 4) + (byte & 15);
            s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<s16x4>(lds + off));
            u32x2 w = __builtin_bit_cast(u32x2, v);
            out[2 * q] = w[0];
            out[2 * q + 1] = w[1];
        }
        return out;
    }
}

// 8-bit fragment (32 elements) of the 16 rows starting at rb.
template <int MODE, int R>
__device__ __forceinline__ i32x8 frag8(const char *lds, int rb, int lane) {
    i32x8 out;
    if (MODE == KMAJ) {
        const int r = rb + (lane & 15), g = lane >> 4;
        u32x4 lo = *reinterpret_cast<const u32x4 *>(lds + kmaj_off(r, 2 * g));
        u32x4 hi = *reinterpret_cast<const u32x4 *>(lds + kmaj_off(r, 2 * g + 1));
        out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
        out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
    } else {
        const int s = lane & 15, g = lane >> 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = 32 * g + 8 * q + (s >> 1);
            const int byte = rb + 8 * (s & 1);
            const int off = mnmaj_off<1, R>(k, byte >> 4) + (byte & 15);
            i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(as_lds<i32x2>(lds + off));
            out[2 * q] = v[0];
            out[2 * q + 1] = v[1];
        }
    }
    return out;
}

template <int IN>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if (IN == IN_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ tile raster

// Workgroup -> (tile_m, tile_n).  Blocks are dealt round-robin to the 8 XCDs;
// renumber so each XCD receives a contiguous run of the grouped raster order,
// in which `group_m` tile rows are walked column by column.
__device__ __forceinline__ void tile_of(int bid, int nblk, int tiles_m, int tiles_n, int group_m,
                                        int &tm, int &tn) {
    int t = bid;
    if ((nblk & 7) == 0) t = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int per_group = group_m * tiles_n;
    const int grp = t / per_group;
    const int first_m = grp * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in = t - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// ------------------------------------------------------------------ epilogue

// Store a wave's accumulators: element (i, j, e) is C[mb + 16i + e][nb + 16j].
// OUTK < 0: FP32 split-K partial into ws[z]; otherwise the epilogue and
// conversion to the C dtype (FUSED: with the bias, read once per column, and
// the activation).  One instantiation per output kind keeps the fully unrolled
// body small enough for the accumulators to stay in registers.
template <int TM, int TN, int OUTK, bool FUSED>
__device__ __forceinline__ void write_tile(const f32x4 (&acc)[TM][TN], const MfmaArgs &p, int mb, int nb,
                                           int z) {
    const Epilogue &ep = p.epi;
    float bias[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
        bias[j] = FUSED && ep.bias && nb + 16 * j < p.N ? load_bias(ep, nb + 16 * j) : 0.0f;
    // One 16 x 64 block at a time: all of its C_in loads (beta != 0, from
    // addresses clamped into the matrix, so no per-element branch), then all of
    // its values, then its stores.  A load, or a use of a loaded value, placed
    // after a store would also wait for that store (one counter tracks both),
    // and each element would pay a memory round trip.
    static_assert(TM * TN <= 16, "tiles of at most 64 accumulators per lane");
    constexpr int JB = TN < 4 ? TN : 4;   // 16-column blocks per batch (registers: 2 x 16 values)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j0 = 0; j0 < TN; j0 += JB) {
            float out[JB][4];
            if (OUTK >= 0) {
                float cin[JB][4];
                if (ep.beta != 0.0f) {
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = min(mb + 16 * i + e, p.M - 1), n = min(nb + 16 * (j0 + j), p.N - 1);
                            cin[j][e] = load_out(ep.C + (int64_t)m * ep.c_rs + (int64_t)n * ep.c_cs, OUTK);
                        }
                }
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = ep.alpha * acc[i][j0 + j][e];
                        if (ep.beta != 0.0f) v = fmaf(ep.beta, cin[j][e], v);
                        if (FUSED) {
                            if (ep.bias) v += bias[j0 + j];
                            v = activate(ep.act, v);
                        }
                        out[j][e] = v;
                        asm volatile("" : "+v"(out[j][e]));   // computed here, not sunk past earlier stores
                    }
            }
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int n = nb + 16 * (j0 + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = mb + 16 * i + e;
                    if (m < p.M && n < p.N) {
                        if (OUTK < 0) p.ws[((int64_t)z * p.M + m) * p.N + n] = acc[i][j0 + j][e];
                        else store_out(ep.C + (int64_t)m * ep.c_rs + (int64_t)n * ep.c_cs, OUTK, out[j][e]);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ the kernel

template <int IN, int BM, int BN, int AMODE, int BMODE, int SLOW>
__global__ void __launch_bounds__(NT) mfma_gemm(MfmaArgs p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int EB = InT<IN>::EB;
    constexpr bool F8 = (IN == IN_F8);
    // stage = A tile, B tile, and (FP8) the BM row scales of the A tile's K block
    constexpr int A_BYTES = BM * KBYTES, B_BYTES = BN * KBYTES;
    constexpr int STAGE = A_BYTES + B_BYTES + (F8 ? BM * 4 : 0);
    constexpr int WTM = BM / 2, WTN = BN / 2, TM = WTM / 16, TN = WTN / 16;
    constexpr int KEL = KBYTES / EB;   // K elements per tile
    using AIO = TileIO<AMODE, BM, EB, SLOW>;
    using BIO = TileIO<BMODE, BN, EB, SLOW>;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int z = blockIdx.z;
    const int kt0 = z * p.kt_per_split;
    const int kt1 = min(kt0 + p.kt_per_split, p.ktiles);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[AIO::NCH], rb[BIO::NCH];
    // FP8 scales of the next K block: one row scale per thread (threads < BM) and
    // the wave's column-block scale (its BN/2 <= 128 columns lie in one block).
    float sa_reg = 0.f, sb_reg = 0.f;
    const int sa_row = m0 + tid;
    const int wave_n0 = n0 + wn * WTN;

    if (kt0 < kt1) {
        AIO::load(ra, p.a, m0, kt0 * KEL, p.M, p.K, tid);
        BIO::load(rb, p.b, n0, kt0 * KEL, p.N, p.K, tid);
        if (F8) {
            if (tid < BM && sa_row < p.M)
                sa_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sa) +
                                                          (int64_t)sa_row * p.sa_rs + (int64_t)kt0 * p.sa_cs);
            if (wave_n0 < p.N)
                sb_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sb) +
                                                          (int64_t)kt0 * p.sb_rs + (int64_t)(wave_n0 >> 7) * p.sb_cs);
        }
        AIO::store(smem, ra, tid);
        BIO::store(smem + A_BYTES, rb, tid);
        if (F8 && tid < BM) *reinterpret_cast<float *>(smem + A_BYTES + B_BYTES + 4 * tid) = sa_reg;
    }
    __syncthreads();

    for (int kt = kt0; kt < kt1; ++kt) {
        const int stage = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        const float sb_cur = sb_reg;
        if (more) {
            AIO::load(ra, p.a, m0, (kt + 1) * KEL, p.M, p.K, tid);
            BIO::load(rb, p.b, n0, (kt + 1) * KEL, p.N, p.K, tid);
            if (F8) {
                if (tid < BM && sa_row < p.M)
                    sa_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sa) +
                                                              (int64_t)sa_row * p.sa_rs + (int64_t)(kt + 1) * p.sa_cs);
                if (wave_n0 < p.N)
                    sb_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sb) +
                                                              (int64_t)(kt + 1) * p.sb_rs + (int64_t)(wave_n0 >> 7) * p.sb_cs);
            }
        }
        const char *la = smem + stage * STAGE;
        const char *lb = la + A_BYTES;
        if constexpr (F8) {
            const float *lsa = reinterpret_cast<const float *>(la + A_BYTES + B_BYTES);
            i32x8 fb[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = frag8<BMODE, BN>(lb, wn * WTN + 16 * j, lane);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const i32x8 fa = frag8<AMODE, BM>(la, wm * WTM + 16 * i, lane);
                // scale product sA[m, kb] * sB[kb, nb] for the lane's 4 rows
                const f32x4 sa4 = *reinterpret_cast<const f32x4 *>(lsa + wm * WTM + 16 * i + 4 * (lane >> 4));
                const f32x4 s4 = sa4 * sb_cur;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    // block sum over this 128-wide K block on the matrix cores, then
                    // promotion into the FP32 accumulator with the scales applied once
                    const f32x4 blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fa, fb[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(s4[e], blk[e], acc[i][j][e]);
                }
            }
        } else {
            (void)sb_cur;
#pragma unroll
            for (int ks = 0; ks < InT<IN>::KSTEPS; ++ks) {
                u32x4 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[i] = frag16<AMODE, BM>(la, wm * WTM + 16 * i, ks, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[j] = frag16<BMODE, BN>(lb, wn * WTN + 16 * j, ks, lane);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<IN>(fa[i], fb[j], acc[i][j]);
            }
        }
        if (more) {
            char *na = smem + (stage ^ 1) * STAGE;
            AIO::store(na, ra, tid);
            BIO::store(na + A_BYTES, rb, tid);
            if (F8 && tid < BM) *reinterpret_cast<float *>(na + A_BYTES + B_BYTES + 4 * tid) = sa_reg;
        }
        __syncthreads();
    }

    // Epilogue: lane holds D rows 4*(lane/16) + e, column lane%16 of each block.
    const int mb = m0 + wm * WTM + 4 * (lane >> 4), nb = n0 + wn * WTN + (lane & 15);
    if (p.splits > 1) write_tile<TM, TN, -1, false>(acc, p, mb, nb, z);
    else if (!p.epi.plain()) {
        if (p.epi.out_kind == OUT_F32) write_tile<TM, TN, OUT_F32, true>(acc, p, mb, nb, z);
        else if (p.epi.out_kind == OUT_BF16) write_tile<TM, TN, OUT_BF16, true>(acc, p, mb, nb, z);
        else write_tile<TM, TN, OUT_F16, true>(acc, p, mb, nb, z);
    } else if (p.epi.out_kind == OUT_F32) write_tile<TM, TN, OUT_F32, false>(acc, p, mb, nb, z);
    else if (p.epi.out_kind == OUT_BF16) write_tile<TM, TN, OUT_BF16, false>(acc, p, mb, nb, z);
    else write_tile<TM, TN, OUT_F16, false>(acc, p, mb, nb, z);
}

template <int IN, int BM, int BN, int AM, int BMd, int SLOW>
hipError_t launch_t(const MfmaArgs &a, hipStream_t s) {
    const int lds = 2 * ((BM + BN) * KBYTES + (IN == IN_F8 ? BM * 4 : 0));
    auto k = mfma_gemm<IN, BM, BN, AM, BMd, SLOW>;
    static bool attr_done = false;   // benign race: setting the attribute twice is harmless
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    dim3 grid(a.tiles_m * a.tiles_n, 1, a.splits);
    hipLaunchKernelGGL(k, grid, dim3(NT), lds, s, a);
    return hipGetLastError();
}

template <int IN, int BM, int BN, int SLOW>
hipError_t launch_modes(int am, int bm, const MfmaArgs &a, hipStream_t s) {
    if (am == KMAJ && bm == KMAJ) return launch_t<IN, BM, BN, KMAJ, KMAJ, SLOW>(a, s);
    if (am == KMAJ && bm == MNMAJ) return launch_t<IN, BM, BN, KMAJ, MNMAJ, SLOW>(a, s);
    if (am == MNMAJ && bm == KMAJ) return launch_t<IN, BM, BN, MNMAJ, KMAJ, SLOW>(a, s);
    return launch_t<IN, BM, BN, MNMAJ, MNMAJ, SLOW>(a, s);
}

template <int IN, int SLOW>
hipError_t launch_tiles(int tile, int am, int bm, const MfmaArgs &a, hipStream_t s) {
    switch (tile) {
    case T128x128: return launch_modes<IN, 128, 128, SLOW>(am, bm, a, s);
    case T64x64: return launch_modes<IN, 64, 64, SLOW>(am, bm, a, s);
    case T128x64: return launch_modes<IN, 128, 64, SLOW>(am, bm, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma(int in_kind, int tile, int a_mode, int b_mode, int slow,
                       const MfmaArgs &args, hipStream_t stream) {
    if (slow) {
        // The element-wise path serves unusual views only; it uses the small tile.
        switch (in_kind) {
        case IN_F16: return launch_modes<IN_F16, 64, 64, 1>(a_mode, b_mode, args, stream);
        case IN_BF16: return launch_modes<IN_BF16, 64, 64, 1>(a_mode, b_mode, args, stream);
        case IN_F8: return launch_modes<IN_F8, 64, 64, 1>(a_mode, b_mode, args, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (in_kind) {
    case IN_F16: return launch_tiles<IN_F16, 0>(tile, a_mode, b_mode, args, stream);
    case IN_BF16: return launch_tiles<IN_BF16, 0>(tile, a_mode, b_mode, args, stream);
    case IN_F8: return launch_tiles<IN_F8, 0>(tile, a_mode, b_mode, args, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
