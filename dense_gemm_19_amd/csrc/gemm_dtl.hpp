// gemm_dtl.hpp -- matrix-core GEMM for gfx950 with direct HBM -> LDS tile loads
// (templates; instantiated per input type by gemm_dtl_{f16,bf16,f8}.hip).
//
// Same computation as gemm_mfma.hip (C = alpha * A * B + beta * C, FP32
// accumulation, and the FP8 E4M3 variant whose per-token and per-128x128-block
// scales are applied once per 128-wide K block: kwkr.cn view-native GEMM
// article, section 2.3; sheratonhq.com deep dive, sections 1.1 and 2.4), for
// the common case where every 16-byte piece of a K tile is either wholly in
// the matrix or past its M/N edge, and K is a whole number of tiles.
//
// What differs from the general kernel: the global -> LDS copies of the next K
// tile are gfx950 "load to LDS" instructions (global_load_lds_dwordx4): the
// data goes from memory straight into the LDS ring without passing through
// registers, which leaves the register file to the accumulators and operand
// fragments of large macro tiles (the double-buffered staging of the
// sheratonhq.com deep dive, sections 2.3 and 3.3, without the register hop).
// Such a load writes lane i's 16 bytes at LDS address base + 16*i, so the
// XOR swizzle of the LDS layout is applied on the global side: lane i fetches
// the chunk that belongs at position i.  Rows past M (or columns past N) read
// a clamped in-range row: their products only reach outputs that are never
// stored.  K-tail padding would reach valid outputs, hence K % tile == 0.
//
// LDS layouts, fragment reads (16-byte reads for K-contiguous operands, the
// gfx950 LDS transpose reads for M/N-contiguous ones), the XCD-aware tile
// raster and the epilogue are those of gemm_mfma.hip.
#pragma once
#include "device_common.hpp"

namespace dg {
namespace dtl {

constexpr int KBYTES = 128;      // bytes of K per tile and row

typedef __attribute__((address_space(3))) void lds_void;

template <int IN> struct InT;
template <> struct InT<IN_F16>  { static constexpr int EB = 2; static constexpr int KSTEPS = 2; };
template <> struct InT<IN_BF16> { static constexpr int EB = 2; static constexpr int KSTEPS = 2; };
template <> struct InT<IN_F8>   { static constexpr int EB = 1; static constexpr int KSTEPS = 1; };

// ------------------------------------------------------------------ LDS layout (as gemm_mfma.hip)

__device__ __forceinline__ int kmaj_off(int r, int c) { return r * KBYTES + ((c ^ (r & 7)) << 4); }

template <int EB, int CPR>
__device__ __forceinline__ int mn_swz(int k) {
    int s;
    if (EB == 2) s = ((k & 3) << 1) | (((k >> 3) & 3) << 3);
    else s = (k & 7) | (((k >> 5) & 3) << 3);
    return s & (CPR - 1);
}
template <int EB, int R>
__device__ __forceinline__ int mnmaj_off(int k, int c) {
    constexpr int CPR = R * EB / 16;
    return k * (R * EB) + ((c ^ mn_swz<EB, CPR>(k)) << 4);
}

// ------------------------------------------------------------------ HBM -> LDS

// One operand's K tile: R rows (M for A, N for B) x 128 bytes of K, 8*R chunks
// of 16 bytes, i.e. R/8 load instructions of a wave (64 chunks each), shared
// by the NW waves.  Instruction j of wave w fills LDS bytes [1024*(w + NW*j), +1024).
template <int MODE, int R, int EB, int NW>
struct DtlIO {
    static constexpr int INSTS = R * 8 / 64 / NW;   // per wave
    static constexpr int EPC = 16 / EB;             // elements per chunk
    static constexpr int CPR = R * EB / 16;         // chunks per K row (MNMAJ)
    static_assert(R * 8 % (64 * NW) == 0, "tile must split evenly over the waves");

    // Issue the wave's loads of the tile whose first K element is k0 into lds.
    __device__ static void issue(char *lds, const Operand &op, int r0, int k0, int Rlim, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < INSTS; ++j) {
            const int blk = wave + NW * j;            // 1 KB block of the tile
            const int pos = blk * 64 + lane;          // chunk position this lane fills
            int r, k;                                 // logical (row, K element) of that chunk
            if (MODE == KMAJ) {
                const int row = pos >> 3, p = pos & 7;
                r = row;
                k = ((p ^ (row & 7)) * EPC);
            } else {
                const int kk = pos / CPR, p = pos % CPR;
                k = kk;
                r = (p ^ mn_swz<EB, CPR>(kk)) * EPC;
            }
            // rows past the edge read a real row (a whole in-range chunk for
            // MNMAJ, where a chunk spans EPC rows); their results are not stored
            const int gr = min(r0 + r, MODE == KMAJ ? Rlim - 1 : Rlim - EPC);
            const char *src = op.ptr + (int64_t)gr * op.r_stride + (int64_t)(k0 + k) * op.k_stride;
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(lds + blk * 1024), 16, 0, 0);
        }
    }
};

// ------------------------------------------------------------------ fragments (as gemm_mfma.hip)

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

// ------------------------------------------------------------------ tile raster (as gemm_mfma.hip)

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

// ------------------------------------------------------------------ epilogue (as gemm_mfma.hip)

template <int TM, int TN, int OUTK>
__device__ __forceinline__ void write_tile(const f32x4 (&acc)[TM][TN], const MfmaArgs &p, int mb, int nb,
                                           int z) {
    const Epilogue &ep = p.epi;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = nb + 16 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = mb + 16 * i + e;
                if (m < p.M && n < p.N) {
                    const float a = acc[i][j][e];
                    if (OUTK < 0) {
                        p.ws[((int64_t)z * p.M + m) * p.N + n] = a;
                    } else {
                        char *q = ep.C + (int64_t)m * ep.c_rs + (int64_t)n * ep.c_cs;
                        float v = ep.alpha * a;
                        if (ep.beta != 0.0f) v = fmaf(ep.beta, load_out(q, OUTK), v);
                        store_out(q, OUTK, v);
                    }
                }
            }
        }
}

// ------------------------------------------------------------------ the kernel

// The two LDS stages are separate __shared__ arrays and the K loop is unrolled
// by two, so the compiler can see that the loads filling one stage never alias
// the fragment reads of the other, and need not wait for them before reading.
template <int IN, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(64 * WGM * WGN) mfma_dtl(MfmaArgs p) {
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    constexpr int EB = InT<IN>::EB;
    constexpr bool F8 = (IN == IN_F8);
    constexpr int A_BYTES = BM * KBYTES, B_BYTES = BN * KBYTES;
    constexpr int STAGE = A_BYTES + B_BYTES + (F8 ? BM * 4 : 0);
    constexpr int WTM = BM / WGM, WTN = BN / WGN, TM = WTM / 16, TN = WTN / 16;
    constexpr int KEL = KBYTES / EB;
    static_assert(BM <= NT || !F8, "one thread per row scale");
    static_assert(WTN <= 128, "a wave's columns lie in one 128-column scale block");
    using AIO = DtlIO<AMODE, BM, EB, NW>;
    using BIO = DtlIO<BMODE, BN, EB, NW>;
    __shared__ __attribute__((aligned(16))) char stage0[STAGE];
    __shared__ __attribute__((aligned(16))) char stage1[STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
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

    // FP8 scales: one row scale per thread (threads < BM) per K block, staged in
    // LDS beside the tile, and the wave's column-block scale.
    float sa_reg = 0.f, sb_reg = 0.f;
    const int sa_row = m0 + tid;
    const int wave_n0 = n0 + wn * WTN;
    auto load_scales = [&](int kt) {
        if (F8) {
            if (tid < BM && sa_row < p.M)
                sa_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sa) +
                                                          (int64_t)sa_row * p.sa_rs + (int64_t)kt * p.sa_cs);
            if (wave_n0 < p.N)
                sb_reg = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.sb) +
                                                          (int64_t)kt * p.sb_rs + (int64_t)(wave_n0 >> 7) * p.sb_cs);
        }
    };
    auto fill = [&](char *st, int kt) {   // issue the loads of K tile kt into stage st
        AIO::issue(st, p.a, m0, kt * KEL, p.M, wave, lane);
        BIO::issue(st + A_BYTES, p.b, n0, kt * KEL, p.N, wave, lane);
        load_scales(kt);
    };
    auto compute = [&](const char *la, float sb_cur) {
        const char *lb = la + A_BYTES;
        if constexpr (F8) {
            const float *lsa = reinterpret_cast<const float *>(la + A_BYTES + B_BYTES);
            i32x8 fb[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = frag8<BMODE, BN>(lb, wn * WTN + 16 * j, lane);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const i32x8 fa = frag8<AMODE, BM>(la, wm * WTM + 16 * i, lane);
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
            // Interleave each matrix-core block sum with the four promotions of an
            // earlier one, so only a few block results are live at a time (left
            // alone, the scheduler issues every block sum first and runs out of
            // registers).
#pragma unroll
            for (int t = 0; t < TM * TN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
            }
        } else {
            (void)sb_cur;
#pragma unroll
            for (int ks = 0; ks < InT<IN>::KSTEPS; ++ks) {
                // the wave's B fragments of this K step stay in registers; A
                // fragments are read one 16-row block at a time
                u32x4 fb[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[j] = frag16<BMODE, BN>(lb, wn * WTN + 16 * j, ks, lane);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const u32x4 fa = frag16<AMODE, BM>(la, wm * WTM + 16 * i, ks, lane);
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<IN>(fa, fb[j], acc[i][j]);
                }
            }
        }
    };
    // one K tile: start filling `nxt` with tile kt+1 (if any), multiply `cur`,
    // stage the next row scales, wait for this thread's loads, then sync
    auto step = [&](const char *cur, char *nxt, int kt) {
        const bool more = kt + 1 < kt1;
        const float sb_cur = sb_reg;
        if (more) fill(nxt, kt + 1);
        compute(cur, sb_cur);
        if (F8 && more && tid < BM) *reinterpret_cast<float *>(nxt + A_BYTES + B_BYTES + 4 * tid) = sa_reg;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (kt0 < kt1) {
        fill(stage0, kt0);
        if (F8 && tid < BM) *reinterpret_cast<float *>(stage0 + A_BYTES + B_BYTES + 4 * tid) = sa_reg;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kt = kt0;
    for (; kt + 1 < kt1; kt += 2) {
        step(stage0, stage1, kt);
        step(stage1, stage0, kt + 1);
    }
    if (kt < kt1) step(stage0, stage1, kt);

    const int mb = m0 + wm * WTM + 4 * (lane >> 4), nb = n0 + wn * WTN + (lane & 15);
    if (p.splits > 1) write_tile<TM, TN, -1>(acc, p, mb, nb, z);
    else if (p.epi.out_kind == OUT_F32) write_tile<TM, TN, OUT_F32>(acc, p, mb, nb, z);
    else if (p.epi.out_kind == OUT_BF16) write_tile<TM, TN, OUT_BF16>(acc, p, mb, nb, z);
    else write_tile<TM, TN, OUT_F16>(acc, p, mb, nb, z);
}

template <int IN, int BM, int BN, int WGM, int WGN, int AM, int BMd>
hipError_t launch_t(const MfmaArgs &a, hipStream_t s) {
    auto k = mfma_dtl<IN, BM, BN, WGM, WGN, AM, BMd>;
    dim3 grid(a.tiles_m * a.tiles_n, 1, a.splits);
    hipLaunchKernelGGL(k, grid, dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

template <int IN, int BM, int BN, int WGM, int WGN>
hipError_t launch_modes(int am, int bm, const MfmaArgs &a, hipStream_t s) {
    if (am == KMAJ && bm == KMAJ) return launch_t<IN, BM, BN, WGM, WGN, KMAJ, KMAJ>(a, s);
    if (am == KMAJ && bm == MNMAJ) return launch_t<IN, BM, BN, WGM, WGN, KMAJ, MNMAJ>(a, s);
    if (am == MNMAJ && bm == KMAJ) return launch_t<IN, BM, BN, WGM, WGN, MNMAJ, KMAJ>(a, s);
    return launch_t<IN, BM, BN, WGM, WGN, MNMAJ, MNMAJ>(a, s);
}

template <int IN>
hipError_t launch_tiles(int tile, int am, int bm, const MfmaArgs &a, hipStream_t s) {
    switch (tile) {
    // 8 waves (2 per SIMD) of 128x64: the FP8 promotion runs on the vector ALUs,
    // which cannot address accumulation registers, so a wave's accumulators must
    // fit in its share of the vector registers alongside everything else
    case T256x256: return launch_modes<IN, 256, 256, 2, 4>(am, bm, a, s);
    case T128x128: return launch_modes<IN, 128, 128, 2, 2>(am, bm, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtl
}  // namespace dg
