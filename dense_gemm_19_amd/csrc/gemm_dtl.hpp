// gemm_dtl.hpp -- matrix-core GEMM for gfx950 with direct HBM -> LDS tile loads
// (templates; instantiated per input type by gemm_dtl_{f16,bf16,f8,f8s}.hip).
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
#include <type_traits>

#include "device_common.hpp"

namespace dg {
namespace dtl {

constexpr int KB = 128;      // bytes of K per tile and row

typedef __attribute__((address_space(3))) void lds_void;

template <int IN> struct InT;
template <> struct InT<IN_F16>  { static constexpr int EB = 2; };
template <> struct InT<IN_BF16> { static constexpr int EB = 2; };
template <> struct InT<IN_F8>   { static constexpr int EB = 1; };

// ------------------------------------------------------------------ LDS layout (as gemm_mfma.hip)

// K-contiguous operands: row r holds 8 chunks of 16 bytes, XOR-swizzled so that
// the 8 rows one fragment read touches per LDS cycle, all at the same logical
// chunk, fall on distinct banks.
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * KB + ((c ^ (r & 7)) << 4); }

// XOR swizzle of the 16-byte chunks of K row k (M/N-contiguous operands).  The
// transpose reads of one 16-lane group touch 4 (16-bit) or 8 (8-bit) consecutive
// K rows; the swizzle spreads those rows, and the K rows of the lane group read
// in the same LDS cycle (K bits 3-4 for 16-bit; for 8-bit, bit 4, which tells
// lane groups 0/1 and 2/3 of a read apart), over distinct banks.  8-bit rows of
// 256 bytes (16 chunks) all start on bank 0: chunk (k & 7) ^ 8 * (bit 4 of k)
// gives lane groups 0 and 1 (and 2 and 3), which read together, the two halves
// of the banks.
template <int EB, int CPR>
__device__ __forceinline__ int mn_swz(int k) {
    int s;
    // 16-bit rows of 128 bytes (8 chunks): rows k and k + 2 (and k + 8, read by
    // the next lane group) share a bank half; K bits 1 and 3 pick the chunk pair.
    if (EB == 2 && CPR == 8) s = (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1;
    else if (EB == 2) s = ((k & 3) << 1) | (((k >> 3) & 3) << 3);
    else if (CPR >= 32) s = (k & 7) | (((k >> 5) & 3) << 3);
    else if (CPR >= 16) s = (k & 7) ^ (((k >> 4) & 1) << 3);
    else s = (k & 7) ^ ((k >> 4) & 1);
    return s & (CPR - 1);
}
template <int EB, int R>
__device__ __forceinline__ int mnmaj_off(int k, int c) {
    constexpr int CPR = R * EB / 16;
    return k * (R * EB) + ((c ^ mn_swz<EB, CPR>(k)) << 4);
}

// FP8 row scales of a stage: lane row l (0..15) owns BM / 16 floats, i.e.
// BM / 64 chunks of 16 bytes; the 16 segments, read together, start at
// l * BM / 4 bytes, so lane rows 64 / BM * 16 apart would share banks.  Their
// chunks are XOR-swizzled by this value, which differs between such rows.
template <int BM>
__device__ __forceinline__ int sa_swz(int l) {
    constexpr int SC = BM / 64 > 0 ? BM / 64 : 1;   // chunks per segment
    return (l / (16 / SC)) & (SC - 1);
}

// ------------------------------------------------------------------ HBM -> LDS

// One load-to-LDS instruction: lane i's `size` bytes from g land at LDS address
// lds + size*i (lds must be wave-uniform).  Written as inline assembly so that
// the compiler's own wait insertion does not treat it as an LDS store that every
// later LDS read must wait for (it cannot tell the ring's stages apart across
// the loop back-edge); the kernel waits for these loads itself, with exact
// counts.  The memory clobber keeps other memory accesses in program order
// around it.  Every vector-memory instruction of the main loop is one of these,
// so the kernel's counts are exact; any wait the compiler adds for its own
// loads can only be stricter, since these are in-order counters.
__device__ __forceinline__ uint32_t lds_addr(const char *lds) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)lds;
}
// `a` is a wave-uniform LDS byte address and `base` a wave-uniform global
// address (both SGPRs); this lane's source is base + off.  The per-lane part is
// a 32-bit offset that stays fixed over the K loop, so advancing a tile costs
// one scalar add of the base and no vector instructions.
__device__ __forceinline__ void lds_load16(const char *base, uint32_t off, uint32_t a) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(a), "v"(off), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const char *base, uint32_t off, uint32_t a) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(a), "v"(off), "s"(base)
                 : "memory", "m0");
}

// One operand's K tile: R rows (M for A, N for B) x 128 bytes of K, 8*R chunks
// of 16 bytes, i.e. R/8 load instructions of a wave (64 chunks each), shared
// by the NW waves.  Instruction j of wave w fills LDS bytes [1024*(w + NW*j), +1024).
template <int MODE, int R, int EB, int NW>
struct DtlIO {
    static constexpr int INSTS = R * 8 / 64 / NW;   // per wave
    static constexpr int EPC = 16 / EB;             // elements per chunk
    static constexpr int CPR = R * EB / 16;         // chunks per K row (MNMAJ)
    static_assert(R * 8 % (64 * NW) == 0, "tile must split evenly over the waves");

    // This lane's source for each of the wave's loads, as a byte offset from
    // the tile origin (row r0 at K tile 0); K tile kt adds kt * (K elements per
    // tile) * k_stride to the origin, the same for every lane.  The host keeps
    // these offsets below 2^31 (rows clamp into [r0, Rlim): r0 < Rlim, and for
    // M/N-contiguous operands Rlim is a multiple of EPC).
    struct Src { uint32_t off[INSTS]; };
    __device__ static Src sources(const Operand &op, int r0, int Rlim, int wave, int lane) {
        Src s;
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
            s.off[j] = (uint32_t)((int64_t)(gr - r0) * op.r_stride + (int64_t)k * op.k_stride);
        }
        return s;
    }

    // Issue the wave's loads of the tile whose origin is `base` (uniform) into
    // the LDS region at `lds` (uniform; wave_u the uniform wave index).
    __device__ static void issue(uint32_t lds, const Src &s, const char *base, int wave_u) {
#pragma unroll
        for (int j = 0; j < INSTS; ++j) lds_load16(base, s.off[j], lds + (uint32_t)((wave_u + NW * j) * 1024));
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

// 8-bit fragment (32 K values) of the 16 rows starting at rb.  The MFMA sums
// over K, so any assignment of K values to (lane group, byte) serves as long as
// A and B agree: lane group g = lane/16 takes K bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of the 128-byte tile, i.e. chunks g and g+4.  For a
// K-contiguous operand the four groups then read chunks 0-3 (and 4-7) of their
// rows together, the same conflict-free pattern as the 16-bit fragments.
template <int MODE, int R>
__device__ __forceinline__ i32x8 frag8(const char *lds, int rb, int lane) {
    i32x8 out;
    const int s = lane & 15, g = lane >> 4;
    if (MODE == KMAJ) {
        const int r = rb + s;
        u32x4 lo = *reinterpret_cast<const u32x4 *>(lds + kmaj_off(r, g));
        u32x4 hi = *reinterpret_cast<const u32x4 *>(lds + kmaj_off(r, g + 4));
        out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
        out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
    } else {
        // transpose reads: 8 consecutive K rows x 16 columns each, bytes 8q..8q+7
        // of the fragment = K rows kb(q)..kb(q)+7
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kb = (q < 2) ? 16 * g + 8 * q : 64 + 16 * g + 8 * (q - 2);
            const int k = kb + (s >> 1);
            const int byte = rb + 8 * (s & 1);
            const int off = mnmaj_off<1, R>(k, byte >> 4) + (byte & 15);
            i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(as_lds<i32x2>(lds + off));
            out[2 * q] = v[0];
            out[2 * q + 1] = v[1];
        }
    }
    return out;
}

// The kernel passes its B fragment as the instruction's first operand and its A
// fragment as the second, so each 16 x 16 result block comes out transposed:
// lane l holds row l % 16 and the 4 adjacent columns 4 (l / 16) .. + 3.  A lane
// then needs one FP8 row scale per block, and stores 4 adjacent elements of C.
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

// Workgroups are dealt to the 8 XCDs in turn (workgroup b to XCD b % 8); when
// the count is a multiple of 8 this permutation hands each XCD a contiguous
// run of work units, so neighbouring tiles share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    return (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
}

// Tile t of the raster: groups of group_m tile rows, walked column by column.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
    const int per_group = group_m * tiles_n;
    const int grp = t / per_group;
    const int first_m = grp * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in = t - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// ------------------------------------------------------------------ the kernel

// An NS-stage LDS ring.  The loads filling a stage are load-to-LDS
// instructions the compiler does not track (see lds_load16), so nothing makes
// a fragment read wait for loads into other stages; before the barrier that
// opens tile kt, each wave waits (explicit vmcnt) for its own loads into that
// tile's stage: exactly the loads of the later tiles may still be in flight.
//
// FP8 scales ride along in every stage: BM row scales sA[m][kt] and up to 64
// column-block scales sB[kt][nb], each staged with 4-byte load-to-LDS
// instructions (every wave issues the same two, so all waves count the same
// number of loads per tile).
//
// Split K (SPLIT, S = p.splits > 1): the first p.dp_tiles tiles run whole; each
// later tile runs as S pieces of K.  A piece writes its FP32 partial tile with
// agent-scope stores; the last of a tile's S pieces (arrival counter) sums the
// partials in the order s = 0..S-1, applies the epilogue, and re-arms the
// counter (sheratonhq.com deep dive, section 5.2, with a fixed summation order
// so that the bits do not depend on which piece finishes last).  With
// p.dp_tiles = 0 that is plain split K; with whole waves of tiles in front it
// is a Stream-K-style hybrid: the pieces of the leftover tiles fill the last
// wave of workgroup slots instead of leaving part of it idle (sheratonhq.com
// deep dive, section 5.2, names Stream-K for balancing tails).
// The workgroup body.  t_direct >= 0: this workgroup computes tile t_direct of
// p whole (the grouped kernel, which maps its grid itself); otherwise the tile
// (and K piece) follows from blockIdx.x and gridDim.x as described above.
template <int IN, int BM, int BN, int WGM, int WGN, int NS, int AMODE, int BMODE, bool SPLIT, int NL, bool SA4>
__device__ __forceinline__ void mfma_dtl_body(const MfmaArgs &p, const int t_direct) {
    constexpr int NW = WGM * WGN;
    // Waves 0 .. NLD-1 issue the tile loads; NLD < NW leaves the others to
    // matrix work alone (a wave stalls while it issues, the queue being full).
    constexpr int NLD = NL > 0 ? NL : NW;
    static_assert(NW % NLD == 0, "loader waves");
    constexpr int EB = InT<IN>::EB;
    constexpr bool F8 = (IN == IN_F8);
    constexpr int KSTEPS = F8 ? 1 : 2;          // 16-bit: matrix instructions of 32 K values
    constexpr int A_BYTES = BM * KB, B_BYTES = BN * KB;
    constexpr int SA_OFF = A_BYTES + B_BYTES, SB_OFF = SA_OFF + (F8 ? BM * 4 : 0);
    constexpr int STAGE = SB_OFF + (F8 ? 256 : 0);
    constexpr int WTM = BM / WGM, WTN = BN / WGN, TM = WTM / 16, TN = WTN / 16;
    constexpr int KEL = KB / EB;
    using AIO = DtlIO<AMODE, BM, EB, NLD>;
    using BIO = DtlIO<BMODE, BN, EB, NLD>;
    constexpr int PER_FILL = AIO::INSTS + BIO::INSTS + (F8 ? 2 : 0);   // loads per wave per tile
    static_assert(NS >= 2 && NS <= 8, "2..8 stages");
    static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns lie in one 128-column scale block");
    static_assert(BM % 64 == 0 || !F8, "row scales are staged 64 per wave");
    static_assert(!F8 || NLD >= BM / 64, "row scales are staged by the loader waves");
    static_assert((NS - 2) * PER_FILL <= 63, "vmcnt range");
    // SA4: FP8 row scales 4 K blocks at a time (see sa4_group below), in
    // SA4_NB buffers of [BM rows][4 blocks] floats.
    static_assert(!SA4 || (F8 && TM % 4 == 0), "SA4");
    constexpr int SA4_BUF = BM * 16, SA4_NB = NS == 2 ? 2 : 4;
    static_assert(NS * STAGE + (SA4 ? SA4_NB * SA4_BUF : 0) <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) char ring[NS * STAGE];
    __shared__ __attribute__((aligned(16))) char sa4_ring[SA4 ? SA4_NB * SA4_BUF : 16];
    __shared__ int is_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    // Work unit: units 0 .. dp_tiles-1 are whole tiles; later units are the S
    // pieces z of the remaining tiles, a tile's pieces consecutive.
    int t, z = 0, S = 1;
    if (t_direct >= 0) {
        t = t_direct;
    } else if (!SPLIT || (int)blockIdx.x < p.dp_tiles) {
        t = xcd_remap(blockIdx.x, SPLIT ? p.dp_tiles : (int)gridDim.x);
    } else {
        const int pc = xcd_remap(blockIdx.x - p.dp_tiles, (int)gridDim.x - p.dp_tiles);
        S = p.splits;
        t = p.dp_tiles + pc / S;
        z = pc - (pc / S) * S;
    }
    int tm, tn;
    raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt0 = S == 1 ? 0 : z * p.kt_per_split;
    const int kt1 = S == 1 ? p.ktiles : min(kt0 + p.kt_per_split, p.ktiles);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // FP8 scale sources of this thread's lane for the staging loads.  The BM
    // row scales of a stage sit in LDS grouped by row mod 16: lane row l = r % 16
    // owns a segment of BM / 16 floats holding its rows' scales in block order
    // b = r / 16, so that a lane finds the scales of its rows (one per 16-row
    // block, see compute) side by side.  The segment's 16-byte chunks are
    // XOR-swizzled by sa_swz(l) so that the 16 segments read together fall on
    // distinct banks.  The loader lane filling float p fetches the row stored
    // there.
    const int NBLK = (p.N + 127) >> 7;
    const int sa_pos = 64 * (wave % (F8 ? BM / 64 : 1)) + lane;
    const int sa_l = sa_pos / (BM / 16), sa_in = sa_pos % (BM / 16);
    const int sa_b = (((sa_in >> 2) ^ sa_swz<BM>(sa_l)) << 2) | (sa_in & 3);
    const int sa_row = min(m0 + sa_b * 16 + sa_l, p.M - 1);
    const int sb_blk = min((n0 >> 7) + lane, NBLK - 1);

    // Source addresses are computed once; each tile only adds a uniform K offset.
    // The LDS destinations are uniform too (the wave index, made uniform once).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const typename AIO::Src a_src = AIO::sources(p.a, m0, p.M, wave % NLD, lane);
    const typename BIO::Src b_src = BIO::sources(p.b, n0, p.N, wave % NLD, lane);
    const uint32_t sa_off = F8 ? (uint32_t)((int64_t)sa_row * p.sa_rs) : 0u;
    const uint32_t sb_off = F8 ? (uint32_t)((int64_t)sb_blk * p.sb_cs) : 0u;
    const char *a_org = p.a.ptr + (int64_t)m0 * p.a.r_stride;
    const char *b_org = p.b.ptr + (int64_t)n0 * p.b.r_stride;
    const int64_t a_kstep = (int64_t)KEL * p.a.k_stride, b_kstep = (int64_t)KEL * p.b.k_stride;
    const uint32_t ring_lds = lds_addr(ring);

    // FP8 row scales, 4 K blocks per load (SA4).  The per-tile 4-byte
    // load-to-LDS of a row scale touches a cache line of its own for every row
    // of the tile (the A and B tiles of a K tile take about 2 lines per tile
    // row).  Where the scales of a row are contiguous over K blocks (16-byte
    // aligned rows, K a multiple of 4 blocks; the launch checks), lane i of
    // wave w < BM/64 instead loads row 64 w + i's scales of the 4 blocks of
    // K-block group g = kt / 4 with one 16-byte load-to-LDS, into buffer
    // g % SA4_NB of sa4_ring ([BM rows][4 blocks]): a quarter of those
    // requests.  The prologue loads the first two groups.
    //  - Two-stage ring (every wait there is for all of a wave's loads, so the
    //    loads per tile may vary): 2 buffers; group g + 1 is loaded whole while
    //    group g's first block is computed (its buffer last served group g - 1,
    //    done by then).
    //  - Deeper rings count each wave's loads per tile exactly: the fill of tile
    //    kt keeps its one row-scale load, now lanes 16 j .. 16 j + 15 (j = kt % 4)
    //    of a 16-byte load of group kt / 4 + 1: the 4 fills of a group load the
    //    next group, a quarter of its rows each.  The fill of tile kt is issued
    //    NS - 1 tiles ahead of its compute, so a group is written up to NS + 3
    //    tiles before its first block is computed: 4 buffers, the one written
    //    last served the group 4 before, done by then.
    const uint32_t sa4_off = SA4 ? (uint32_t)((int64_t)min(m0 + 64 * (wave % (F8 ? BM / 64 : 1)) + lane, p.M - 1) * p.sa_rs) : 0u;
    const uint32_t sa4_lds = lds_addr(sa4_ring);
    auto sa4_group = [&](int g) __attribute__((always_inline)) {   // K-block group g into its buffer
        if (SA4 && wave_u < BM / 64)
            lds_load16(reinterpret_cast<const char *>(p.sa) + (int64_t)g * 16, sa4_off,
                       sa4_lds + (uint32_t)((g & (SA4_NB - 1)) * SA4_BUF + 1024 * wave_u));
    };
    // rows 16 j .. 16 j + 15 of each wave's 64 of group g (past the last group:
    // the last group again, the same values into its own buffer)
    auto sa4_quarter = [&](int g, int j) __attribute__((always_inline)) {
        g = min(g, (p.ktiles >> 2) - 1);
        if ((lane >> 4) == j)
            lds_load16(reinterpret_cast<const char *>(p.sa) + (int64_t)g * 16, sa4_off,
                       sa4_lds + (uint32_t)((g & (SA4_NB - 1)) * SA4_BUF + 1024 * (wave_u % (BM / 64))));
    };

    auto fill = [&](int stage_idx, int kt) __attribute__((always_inline)) {   // K tile kt into a stage
        if (NLD < NW && wave_u >= NLD) return;
        const uint32_t st = ring_lds + (uint32_t)(stage_idx * STAGE);
        AIO::issue(st, a_src, a_org + kt * a_kstep, wave_u);
        BIO::issue(st + A_BYTES, b_src, b_org + kt * b_kstep, wave_u);
        if constexpr (F8) {
            if constexpr (!SA4)
                lds_load4(reinterpret_cast<const char *>(p.sa) + (int64_t)kt * p.sa_cs, sa_off,
                          st + SA_OFF + 256 * (wave_u % (BM / 64)));
            else if constexpr (NS > 2)
                sa4_quarter((kt >> 2) + 1, kt & 3);
            lds_load4(reinterpret_cast<const char *>(p.sb) + (int64_t)kt * p.sb_rs, sb_off, st + SB_OFF);
            // two stages: tile kt - 1, the first of its group g, is being computed:
            // group g + 1 (the prologue loaded it where g is the first group)
            if (SA4 && NS == 2 && (kt & 3) == 1 && ((kt - 1) >> 2) > (kt0 >> 2) && ((kt >> 2) + 1) * 4 < kt1)
                sa4_group((kt >> 2) + 1);
        }
    };

    auto compute = [&](const char *la, int kt) __attribute__((always_inline)) {
        const char *lb = la + A_BYTES;
        if constexpr (F8) {
            // This lane's rows are wm * WTM + 16 i + lane % 16 (the products are
            // formed transposed, see mma), so it needs one row scale per 16-row
            // block: TM floats side by side in the stage's scale layout.
            const float *lsa = reinterpret_cast<const float *>(la + SA_OFF) + (lane & 15) * (BM / 16);
            const float *lsb = reinterpret_cast<const float *>(la + SB_OFF) + ((wn * WTN) >> 7);
            float sc[TM], sb = 0.0f;
            f32x4 sraw[TM % 4 == 0 ? TM / 4 : 1];
            auto read_scales = [&]() __attribute__((always_inline)) {
                sb = *lsb;
                if constexpr (SA4) {
                    // rows wm * WTM + 16 q + lane % 16 of block kt, from its group's buffer
                    const float *g4 = reinterpret_cast<const float *>(sa4_ring + ((kt >> 2) & (SA4_NB - 1)) * SA4_BUF) +
                                      4 * (wm * WTM + (lane & 15)) + (kt & 3);
#pragma unroll
                    for (int q = 0; q < TM; ++q) sraw[q / 4][q % 4] = g4[64 * q];
                } else if constexpr (TM % 4 == 0) {
#pragma unroll
                    for (int q = 0; q < TM; q += 4) {
                        const int chunk = ((wm * TM + q) >> 2) ^ sa_swz<BM>(lane & 15);
                        sraw[q / 4] = *reinterpret_cast<const f32x4 *>(lsa + 4 * chunk);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < TM; ++q) {
                        const int b = wm * TM + q;
                        sc[q] = lsa[4 * ((b >> 2) ^ sa_swz<BM>(lane & 15)) + (b & 3)];
                    }
                }
            };
            auto scales = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int q = 0; q < TM; ++q)
                    sc[q] = (TM % 4 == 0 ? sraw[TM % 4 == 0 ? q / 4 : 0][q % 4] : sc[q]) * sb;
            };
            // Block sums over this 128-wide K block on the matrix cores, then
            // promotion into the FP32 accumulators with the scales applied once.
            // The promotion of block t runs after the matrix instructions of blocks
            // t + 1 .. t + PL are issued, so the vector ALUs work while the matrix
            // core does, and a block's sums are complete when they are read
            // (measured on FP8 4096 x 7168 x 4096: lag 1 147.5 us, 2 130.8 us,
            // 3 to 6 about 127 us).  With A column-major the transposed A reads
            // need more registers, and a lag of 4 would spill: 2 there.
            constexpr int PL = AMODE == MNMAJ ? 2 : 4;   // promotion lag, in blocks
            // Each step is fenced (sched_barrier) so that the compiler keeps the
            // order written here: the matrix instruction of block t, then the
            // reads for later steps, then the promotion of block t - PL, whose
            // sums are complete by then; left free, it pulls each block's
            // promotion up behind its own matrix instruction and pads the wait
            // with nops.  Reads are issued just ahead of their use, so that few
            // are outstanding when a matrix instruction waits for its own (LDS
            // reads complete in order): the first block's B and A fragments
            // before the loop, B fragment j + 2 after block j's instruction (the
            // B fragments then stay for the whole K block), the A fragment of the
            // next 16-row block TN blocks ahead, and the scales after block 1,
            // their products formed at step PL.
            // Where A is M-contiguous its transposed reads hold more registers and
            // this order spills: there every fragment and scale is read before the
            // loop (EARLY), the A fragment of the next block ahead of the matrix
            // instruction.
            constexpr bool EARLY = AMODE == MNMAJ;
            i32x8 fb[TN];
            if constexpr (EARLY) {
                read_scales();
                scales();
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[j] = frag8<BMODE, BN>(lb, wn * WTN + 16 * j, lane);
            } else {
                fb[0] = frag8<BMODE, BN>(lb, wn * WTN, lane);
            }
            i32x8 fa = frag8<AMODE, BM>(la, wm * WTM, lane), fa_next = fa;
            if constexpr (!EARLY && TN > 1) fb[1] = frag8<BMODE, BN>(lb, wn * WTN + 16, lane);
            f32x4 blk[PL + 1];
#pragma unroll
            for (int t = 0; t < TM * TN + PL; ++t) {
                if (t < TM * TN) {
                    const int i = t / TN, j = t % TN;
                    if (EARLY && j == 0 && i + 1 < TM) fa_next = frag8<AMODE, BM>(la, wm * WTM + 16 * (i + 1), lane);
                    blk[t % (PL + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fb[j], fa, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                    if constexpr (!EARLY) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (i == 0 && j + 2 < TN) fb[j + 2] = frag8<BMODE, BN>(lb, wn * WTN + 16 * (j + 2), lane);
                        if (t == 1 || (TM * TN == 1 && t == 0)) read_scales();
                        if (j == 0 && i + 1 < TM) fa_next = frag8<AMODE, BM>(la, wm * WTM + 16 * (i + 1), lane);
                    }
                    if (j == TN - 1) fa = fa_next;
                }
                if (!EARLY && t == PL) scales();
                if (t >= PL) {
                    const int u = t - PL, pi = u / TN, pj = u % TN;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[pi][pj][e] = fmaf(sc[pi], blk[u % (PL + 1)][e], acc[pi][pj][e]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // The wave's B fragments of a K step stay in registers; A fragments
            // are read one 16-row block at a time, PD blocks ahead of the matrix
            // instructions that use them (a K step's B fragments with the first
            // block of that step), so that each read's LDS latency hides behind
            // the matrix instructions of the blocks before it.
            constexpr int RA = AMODE == KMAJ ? 1 : 2, RB = BMODE == KMAJ ? 1 : 2;   // LDS reads per fragment
            constexpr int STEPS = KSTEPS * TM, PD = 2;
            u32x4 fb[KSTEPS][TN], fa[PD + 1];
            auto read_step = [&](int t) __attribute__((always_inline)) {   // fragments of step t
                const int ks = t / TM, i = t % TM;
                if (i == 0) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) fb[ks][j] = frag16<BMODE, BN>(lb, wn * WTN + 16 * j, ks, lane);
                    __builtin_amdgcn_sched_group_barrier(0x100, TN * RB, 0);
                }
                fa[t % (PD + 1)] = frag16<AMODE, BM>(la, wm * WTM + 16 * i, ks, lane);
                __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
            };
#pragma unroll
            for (int t = 0; t < PD && t < STEPS; ++t) read_step(t);
#pragma unroll
            for (int t = 0; t < STEPS; ++t) {
                if (t + PD < STEPS) read_step(t + PD);
                const int ks = t / TM, i = t % TM;
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<IN>(fb[ks][j], fa[t % (PD + 1)], acc[i][j]);
                __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            }
        }
    };

    // wait until at most `later` tiles' loads of this wave are still in flight
    auto wait_tiles = [&](int later) __attribute__((always_inline)) {
        constexpr int enc0 = (0x7 << 4) | (0xF << 8);   // expcnt, lgkmcnt: no wait
#define DG_VMCNT(n) (((n) & 0xF) | (((n) >> 4) << 14) | enc0)
        switch (later) {
        case 0: __builtin_amdgcn_s_waitcnt(DG_VMCNT(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 2 ? 1 * PER_FILL : 0)); break;
        case 2: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 3 ? 2 * PER_FILL : 0)); break;
        case 3: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 4 ? 3 * PER_FILL : 0)); break;
        case 4: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 5 ? 4 * PER_FILL : 0)); break;
        case 5: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 6 ? 5 * PER_FILL : 0)); break;
        default: __builtin_amdgcn_s_waitcnt(DG_VMCNT(NS > 7 ? 6 * PER_FILL : 0)); break;
        }
#undef DG_VMCNT
    };

    // prologue: the first NS - 1 tiles go out (and, SA4, the row scales of the
    // first two K-block groups)
    if (SA4 && kt0 < kt1) {
        sa4_group(kt0 >> 2);
        if (((kt0 >> 2) + 1) * 4 < kt1) sa4_group((kt0 >> 2) + 1);
    }
#pragma unroll
    for (int q = 0; q + 1 < NS; ++q)
        if (kt0 + q < kt1) fill(q, kt0 + q);
    // tile kt sits in stage `cur`; the stage freed by tile kt - 1 takes tile kt + NS - 1
    auto body = [&](int cur, int kt) __attribute__((always_inline)) {
        wait_tiles(min(NS - 2, kt1 - 1 - kt));
        // A plain barrier: __syncthreads() would add a wait for every outstanding
        // load-to-LDS (they count as LDS writes), draining the ring.  This wave's
        // loads into tile kt are complete (wait above); the memory clobber keeps
        // the compiler from moving LDS accesses or the refill across it, and the
        // LDS wait before it completes this wave's reads of the stage that the
        // refill below overwrites (the compiler may defer the matrix
        // instructions that consume them past this point).
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int nxt = cur == 0 ? NS - 1 : cur - 1;
        if (kt + NS - 1 < kt1) fill(nxt, kt + NS - 1);
        compute(ring + cur * STAGE, kt);
    };
    // With NS = 2 and 4 waves the loop runs two tiles per trip, so that each
    // stage's LDS addresses are fixed offsets (immediates) rather than a
    // per-trip vector add; the 256x256 tile's 8-wave kernel keeps a rolled loop
    // (unrolled, it needs more than its 256 registers and spills).
    if constexpr (NS == 2 && NW == 4) {
        int kt = kt0;
        for (; kt + 1 < kt1; kt += 2) {
            body(0, kt);
            body(1, kt + 1);
        }
        if (kt < kt1) body(0, kt);
    } else {
        int cur = 0;
        for (int kt = kt0; kt < kt1; ++kt) {
            body(cur, kt);
            cur = cur + 1 == NS ? 0 : cur + 1;
        }
    }

    // ---- epilogue: element (i, j, e) of a wave is C[mr + 16i][nc + 16j + e]
    // (the products are formed transposed: a lane holds 4 adjacent columns of
    // one row per 16 x 16 block)
    const int mr = m0 + wm * WTM + (lane & 15), nc = n0 + wn * WTN + 4 * (lane >> 4);
    const Epilogue &ep = p.epi;
    // FUSED: bias (read once per column) and activation after alpha/beta.
    // The value stored at (m, n): alpha * acc (+ beta * C_in) (+ bias), activated;
    // cin is C_in, loaded beforehand (used only when beta != 0).
    auto value = [&](auto FUSED, float a, float bias, float cin) __attribute__((always_inline)) {
        float v = ep.alpha * a;
        if (ep.beta != 0.0f) v = fmaf(ep.beta, cin, v);
        if constexpr (decltype(FUSED)::value) {
            if (ep.bias) v += bias;
            v = activate(ep.act, v);
        }
        return v;
    };
    // C_in of this lane's elements, loaded ahead by the split path (see below)
    // where the registers allow (at most 8 blocks: the 128 x 128 split kernel
    // would drop from two waves per SIMD to one); cin_pre[i][j][e] belongs to
    // element (i, j, e).  Unused otherwise.
    constexpr bool PRE_CIN = SPLIT && TM * TN <= 8;
    float cin_pre[PRE_CIN ? TM : 1][PRE_CIN ? TN : 1][4] = {};
    auto finish = [&](auto OUTK, auto FUSED, auto PRE) __attribute__((always_inline)) {
        constexpr int ok = decltype(OUTK)::value;
        constexpr bool fused = decltype(FUSED)::value;
        constexpr bool pre = decltype(PRE)::value;
        float bias[TN][4];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = nc + 16 * j + e;
                bias[j][e] = fused && ep.bias && n < p.N ? load_bias(ep, n) : 0.0f;
            }
        // One 16-row block at a time: all of the block's C_in loads (beta != 0),
        // then all of its values, then all of its stores.  A load or a use of a
        // loaded value placed after a store would wait for that store too (the
        // counter that tracks loads counts stores), and each element would pay
        // a memory round trip; so would a load inside a per-element branch.
        // Where C's rows are contiguous and 4-element aligned (ep.vec4), each
        // lane's 4 adjacent columns go in one vector load or store.
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = mr + 16 * i;
            // clamped into the matrix: every lane loads (no branch per element);
            // values past the edge are never stored
            const char *crow = ep.C + (int64_t)min(m, p.M - 1) * ep.c_rs;
            float cin[TN][4], out[TN][4];
            if constexpr (pre) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) cin[j][e] = cin_pre[PRE_CIN ? i : 0][PRE_CIN ? j : 0][e];
            } else if (ep.beta != 0.0f) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = nc + 16 * j;
                    if (ep.vec4 && n + 3 < p.N) {
                        const f32x4 v = load_out4(crow + (int64_t)n * ep.c_cs, ok);
#pragma unroll
                        for (int e = 0; e < 4; ++e) cin[j][e] = v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            cin[j][e] = load_out(crow + (int64_t)min(n + e, p.N - 1) * ep.c_cs, ok);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    out[j][e] = value(FUSED, acc[i][j][e], bias[j][e], cin[j][e]);
                    // pins the value here: the compiler would otherwise sink its
                    // computation into the store's branch, after earlier stores
                    asm volatile("" : "+v"(out[j][e]));
                }
            if (m < p.M) {
                char *row = ep.C + (int64_t)m * ep.c_rs;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = nc + 16 * j;
                    if (ep.vec4 && n + 3 < p.N) {
                        store_out4(row + (int64_t)n * ep.c_cs, ok, out[j]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) store_out(row + (int64_t)(n + e) * ep.c_cs, ok, out[j][e]);
                    }
                }
            }
        }
    };
    auto finish_kind = [&](auto FUSED, auto PRE) __attribute__((always_inline)) {
        if (ep.out_kind == OUT_F32) finish(std::integral_constant<int, OUT_F32>{}, FUSED, PRE);
        else if (ep.out_kind == OUT_BF16) finish(std::integral_constant<int, OUT_BF16>{}, FUSED, PRE);
        else finish(std::integral_constant<int, OUT_F16>{}, FUSED, PRE);
    };
    auto finish_any = [&](auto PRE) __attribute__((always_inline)) {
        if (ep.plain()) finish_kind(std::false_type{}, PRE);
        else finish_kind(std::true_type{}, PRE);
    };
    // Split K is a separate instantiation (SPLIT), so that the kernels without
    // it keep their registers; it exists for tiles of at most 64 accumulator
    // registers per lane (the reduction stages partials beside them).
    static_assert(!SPLIT || TM * TN <= 16, "split K only for small tiles");
    if (!SPLIT || S == 1) {
        finish_any(std::false_type{});
        return;
    }
    // split K: publish this piece's partial tile with agent-scope stores, wait
    // for the stores, take a ticket (take_last_ticket: the last piece then
    // sees every partial).
    // Partials of split tile w = t - dp_tiles live at
    //   ws[((w * S + q) * NW + wave) * (TM * TN * 4) + element) * 64 + lane]:
    // every thread writes and reads its own elements (the last piece runs the
    // same thread layout), each store or load instruction covers 256
    // contiguous bytes, and rows or columns past the matrix need no test.
    const int64_t piece = (int64_t)BM * BN;
    const float *wtile = p.ws + (int64_t)(t - p.dp_tiles) * S * piece + (int64_t)wave * (TM * TN * 4 * 64) + lane;
    auto slot = [&](int q, int i, int j, int e) __attribute__((always_inline)) {
        return const_cast<float *>(wtile) + q * piece + ((i * TN + j) * 4 + e) * 64;
    };
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __hip_atomic_store(slot(z, i, j, e), acc[i][j][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    // With beta != 0 every piece loads its elements' C_in now, after its
    // partials are acknowledged and before the ticket: the loads then overlap
    // the ticket's round trip and the partial loads of the last piece, which
    // alone uses them (one C_in round trip per 16-row block at the end
    // otherwise).  The other pieces' loads mostly hit the L2 of their XCD.
    auto preload = [&](auto OUTK) __attribute__((always_inline)) {
        constexpr int ok = decltype(OUTK)::value;
        if constexpr (PRE_CIN) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const char *crow = ep.C + (int64_t)min(mr + 16 * i, p.M - 1) * ep.c_rs;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = nc + 16 * j;
                if (ep.vec4 && n + 3 < p.N) {
                    const f32x4 v = load_out4(crow + (int64_t)n * ep.c_cs, ok);
#pragma unroll
                    for (int e = 0; e < 4; ++e) cin_pre[i][j][e] = v[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        cin_pre[i][j][e] = load_out(crow + (int64_t)min(n + e, p.N - 1) * ep.c_cs, ok);
                }
            }
        }
        }
    };
    if (PRE_CIN && ep.beta != 0.0f) {
        if (ep.out_kind == OUT_F32) preload(std::integral_constant<int, OUT_F32>{});
        else if (ep.out_kind == OUT_BF16) preload(std::integral_constant<int, OUT_BF16>{});
        else preload(std::integral_constant<int, OUT_F16>{});
    }
    __syncthreads();
    const int tile = tm * p.tiles_n + tn;
    if (tid == 0) is_last = take_last_ticket(p.counters + tile, S);
    __syncthreads();
    if (!is_last) return;
    // The sum runs over s = 0..S-1 in order, this workgroup's own partial
    // included (from registers where own[] exists: the same values).  Loads go out in batches of QB splits x IB 16-row blocks (at
    // most 64 values in flight beside the accumulators), every load of a batch
    // before any add, so a batch costs one memory round trip; a batch running
    // past the last split re-reads split S-1 (unconditional loads keep the
    // waits exact) and ignores it.
    auto part = [&](int q, int i, int j, int e) __attribute__((always_inline)) {
        return __hip_atomic_load(slot(q, i, j, e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    constexpr int IB = TM < (8 / TN > 0 ? 8 / TN : 1) ? TM : (8 / TN > 0 ? 8 / TN : 1);
    constexpr int QB = 16 / (IB * TN) > 0 ? 16 / (IB * TN) : 1;
    // This piece's own partial comes from a register copy, not from memory,
    // where the registers allow (as for cin_pre): a 1/S smaller load volume.
    f32x4 own[PRE_CIN ? TM : 1][PRE_CIN ? TN : 1];
    if constexpr (PRE_CIN) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) own[i][j] = acc[i][j];
    }
#pragma unroll
    for (int i0 = 0; i0 < TM; i0 += IB) {
        for (int q0 = 0; q0 < S; q0 += QB) {
            f32x4 v[QB][IB][TN];
#pragma unroll
            for (int qq = 0; qq < QB; ++qq) {
                const int q = min(q0 + qq, S - 1);
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        if (PRE_CIN && q == z) {
                            v[qq][i][j] = own[PRE_CIN ? i0 + i : 0][PRE_CIN ? j : 0];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[qq][i][j][e] = part(q, i0 + i, j, e);
                        }
                    }
            }
#pragma unroll
            for (int qq = 0; qq < QB; ++qq) {
                if (q0 + qq >= S) break;
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i0 + i][j] = q0 + qq == 0 ? v[qq][i][j] : acc[i0 + i][j] + v[qq][i][j];
            }
        }
    }
    finish_any(std::integral_constant<bool, PRE_CIN>{});
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int IN, int BM, int BN, int WGM, int WGN, int NS, int AMODE, int BMODE, bool SPLIT, int NL, bool SA4>
__global__ void __launch_bounds__(64 * WGM * WGN) mfma_dtl(MfmaArgs p) {
    mfma_dtl_body<IN, BM, BN, WGM, WGN, NS, AMODE, BMODE, SPLIT, NL, SA4>(p, -1);
}

// Several problems of one tile configuration in one grid (the experts of an
// MoE layer with more than a few tokens each, say): the grid is mapped onto
// the XCDs as one problem would be, then workgroup u belongs to the group g
// with unit_begin[g] <= u < unit_begin[g + 1] and computes that group's tile
// u - unit_begin[g] whole (no K split).
template <int IN, int BM, int BN, int WGM, int WGN, int NS, int AMODE, int BMODE, int NL>
__global__ void __launch_bounds__(64 * WGM * WGN) mfma_dtl_grouped(GroupedMfmaArgs ga) {
    const int u = xcd_remap(blockIdx.x, gridDim.x);
    int g = 0;
    while (g + 1 < ga.ngroups && u >= ga.unit_begin[g + 1]) ++g;
    // The group's arguments, word by word through readfirstlane: the body needs
    // them wave-uniform (its load-to-LDS instructions take scalar bases), which
    // the compiler cannot see through the run-time group index.
    MfmaArgs p;
    static_assert(sizeof(MfmaArgs) % 4 == 0, "word copy");
    const int *src = reinterpret_cast<const int *>(&ga.g[g]);
    int *dst = reinterpret_cast<int *>(&p);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(MfmaArgs) / 4); ++i) dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
    mfma_dtl_body<IN, BM, BN, WGM, WGN, NS, AMODE, BMODE, false, NL, false>(p, u - ga.unit_begin[g]);
}

template <int IN, int BM, int BN, int WGM, int WGN, int NS, int AM, int BMd, int NL, bool SA4>
hipError_t launch_t2(const MfmaArgs &a, hipStream_t s) {
    constexpr int TM = BM / WGM / 16, TN = BN / WGN / 16;
    const int tiles = a.tiles_m * a.tiles_n;
    dim3 grid(tiles);
    if (a.splits > 1) {
        grid = dim3(a.dp_tiles + (tiles - a.dp_tiles) * a.splits);
        if constexpr (TM * TN <= 16) {
            hipLaunchKernelGGL((mfma_dtl<IN, BM, BN, WGM, WGN, NS, AM, BMd, true, NL, SA4>), grid, dim3(64 * WGM * WGN), 0, s, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;   // no split K for this tile (the planner never asks)
        }
    }
    hipLaunchKernelGGL((mfma_dtl<IN, BM, BN, WGM, WGN, NS, AM, BMd, false, NL, SA4>), grid, dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

// FP8 kernels with a two-stage ring, and the 64x128 tile, load 4 K blocks of
// row scales at once where every row's scales are contiguous, 16-byte aligned
// and whole groups of 4 K blocks (SA4 in the kernel body).
template <int IN, int BM, int BN, int WGM, int WGN, int NS, int AM, int BMd, int NL>
hipError_t launch_t(const MfmaArgs &a, hipStream_t s) {
    constexpr bool SA4_OK = IN == IN_F8 && (NS == 2 || BM == 64) && (BM / WGM / 16) % 4 == 0;
    if constexpr (SA4_OK) {
        if (a.sa_cs == 4 && a.sa_rs % 16 == 0 && (reinterpret_cast<uintptr_t>(a.sa) & 15) == 0 && a.ktiles % 4 == 0)
            return launch_t2<IN, BM, BN, WGM, WGN, NS, AM, BMd, NL, true>(a, s);
    }
    return launch_t2<IN, BM, BN, WGM, WGN, NS, AM, BMd, NL, false>(a, s);
}

template <int IN, int BM, int BN, int WGM, int WGN, int NS, int NL = 0>
hipError_t launch_grouped_modes(int am, int bm, const GroupedMfmaArgs &a, int units, hipStream_t s) {
    const dim3 grid(units), block(64 * WGM * WGN);
    if (am == KMAJ && bm == KMAJ)
        hipLaunchKernelGGL((mfma_dtl_grouped<IN, BM, BN, WGM, WGN, NS, KMAJ, KMAJ, NL>), grid, block, 0, s, a);
    else if (am == KMAJ && bm == MNMAJ)
        hipLaunchKernelGGL((mfma_dtl_grouped<IN, BM, BN, WGM, WGN, NS, KMAJ, MNMAJ, NL>), grid, block, 0, s, a);
    else if (am == MNMAJ && bm == KMAJ)
        hipLaunchKernelGGL((mfma_dtl_grouped<IN, BM, BN, WGM, WGN, NS, MNMAJ, KMAJ, NL>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mfma_dtl_grouped<IN, BM, BN, WGM, WGN, NS, MNMAJ, MNMAJ, NL>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int IN, int BM, int BN, int WGM, int WGN, int NS, int NL = 0>
hipError_t launch_modes(int am, int bm, const MfmaArgs &a, hipStream_t s) {
    if (am == KMAJ && bm == KMAJ) return launch_t<IN, BM, BN, WGM, WGN, NS, KMAJ, KMAJ, NL>(a, s);
    if (am == KMAJ && bm == MNMAJ) return launch_t<IN, BM, BN, WGM, WGN, NS, KMAJ, MNMAJ, NL>(a, s);
    if (am == MNMAJ && bm == KMAJ) return launch_t<IN, BM, BN, WGM, WGN, NS, MNMAJ, KMAJ, NL>(a, s);
    return launch_t<IN, BM, BN, WGM, WGN, NS, MNMAJ, MNMAJ, NL>(a, s);
}

// Tile configurations (see kernels.hpp): 256x256 runs 8 waves of 128x64 with 2
// stages (one workgroup per CU), of which waves 0-3 (one per SIMD) issue all
// the tile loads and waves 4-7 only compute: a wave stalls while it issues
// (the memory queue is full), and this way every SIMD keeps a wave on the
// matrix cores meanwhile (BF16 4096^3: 115 -> 109 us); 128x128 4 waves of 64x64 with 2 stages (two
// workgroups share a CU, so that one's loads overlap the other's matrix
// work); the small tiles, used for HBM-bound shapes with few rows, 4 waves
// with deep rings (6 or 8 stages), so that enough bytes stream per CU to cover
// the memory latency (64x128 runs as 1 x 4 waves of 64x32, so each stage
// carries twice as much of B as of A).
template <int IN>
hipError_t launch_tiles(int tile, int am, int bm, const MfmaArgs &a, hipStream_t s) {
    switch (tile) {
    case T256x256: return launch_modes<IN, 256, 256, 2, 4, 2, 4>(am, bm, a, s);
    case T128x128: return launch_modes<IN, 128, 128, 2, 2, 2>(am, bm, a, s);
    case T128x64: return launch_modes<IN, 128, 64, 2, 2, 6>(am, bm, a, s);
    case T64x64: return launch_modes<IN, 64, 64, 2, 2, 8>(am, bm, a, s);
    case T64x128: return launch_modes<IN, 64, 128, 1, 4, 6>(am, bm, a, s);
    }
    return hipErrorInvalidValue;
}

// launch_tiles in two parts, the two-stage tiles (256x256, 128x128) and the
// others, so that one input type's kernels can be compiled as two translation
// units side by side.
template <int IN, bool TWO_STAGE>
hipError_t launch_tiles_part(int tile, int am, int bm, const MfmaArgs &a, hipStream_t s) {
    if constexpr (TWO_STAGE) {
        switch (tile) {
        case T256x256: return launch_modes<IN, 256, 256, 2, 4, 2, 4>(am, bm, a, s);
        case T128x128: return launch_modes<IN, 128, 128, 2, 2, 2>(am, bm, a, s);
        }
    } else {
        switch (tile) {
        case T128x64: return launch_modes<IN, 128, 64, 2, 2, 6>(am, bm, a, s);
        case T64x64: return launch_modes<IN, 64, 64, 2, 2, 8>(am, bm, a, s);
        case T64x128: return launch_modes<IN, 64, 128, 1, 4, 6>(am, bm, a, s);
        }
    }
    return hipErrorInvalidValue;
}

// The grouped kernel with the tile configurations of launch_tiles.
template <int IN>
hipError_t launch_grouped_tiles(int tile, int am, int bm, const GroupedMfmaArgs &a, int units, hipStream_t s) {
    switch (tile) {
    case T256x256: return launch_grouped_modes<IN, 256, 256, 2, 4, 2, 4>(am, bm, a, units, s);
    case T128x128: return launch_grouped_modes<IN, 128, 128, 2, 2, 2>(am, bm, a, units, s);
    case T128x64: return launch_grouped_modes<IN, 128, 64, 2, 2, 6>(am, bm, a, units, s);
    case T64x64: return launch_grouped_modes<IN, 64, 64, 2, 2, 8>(am, bm, a, units, s);
    case T64x128: return launch_grouped_modes<IN, 64, 128, 1, 4, 6>(am, bm, a, units, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtl
}  // namespace dg
