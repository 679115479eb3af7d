// kernels.hpp -- argument blocks and launchers shared by the host code and the
// gfx950 kernels.  All strides are in bytes.
#pragma once
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace dg {

// Operand storage modes inside a K tile.
//  KMAJ : the operand is stored K-contiguous (A row-major, or B given as B^T
//         row-major).  LDS holds [rows][128 bytes of K]; fragments are plain
//         16-byte LDS reads.
//  MNMAJ: the operand is stored M- or N-contiguous (B row-major [K][N], or A
//         column-major).  LDS holds [K][rows]; fragments come from the gfx950
//         LDS transpose reads (ds_read_b64_tr_b16 / ds_read_b64_tr_b8).
enum OpMode : int { KMAJ = 0, MNMAJ = 1 };

// Input element kinds of the matrix-core path.
enum InKind : int { IN_F16 = 0, IN_BF16 = 1, IN_F8 = 2 };

// Output element kinds (match dg_dtype numbering for F32/F16/BF16).
enum OutKind : int { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };

struct Operand {
    const char *ptr;
    int64_t r_stride;   // bytes per step of the operand's M (A) or N (B) index
    int64_t k_stride;   // bytes per step of K
    int vec;            // 1: 16-byte vector loads are legal for full chunks
};

// Element-wise activation applied after the bias (numbering matches dg_act).
enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };

// out[m][n] = act(alpha * acc + beta * C_in[m][n] + bias[n]), rounded to the C dtype.
struct Epilogue {
    char *C;
    int64_t c_rs, c_cs; // bytes
    int out_kind;       // OutKind
    float alpha, beta;  // beta == 0: C is not read
    const char *bias;   // N-vector added to every row, or null (no bias)
    int64_t bias_s;     // bytes between consecutive bias elements (0: one value for every column)
    int bias_kind;      // OutKind numbering: OUT_F32 / OUT_F16 / OUT_BF16
    int act;            // Act
    int vec4;           // C's rows are contiguous and 4-element aligned (c_cs == element size,
                        // C and c_rs multiples of 4 elements): 4 adjacent columns in one access
    constexpr bool plain() const { return bias == nullptr && act == ACT_NONE; }
};

struct MfmaArgs {
    Operand a, b;               // a: M x K, b: N x K (as "rows x K")
    const float *sa; int64_t sa_rs, sa_cs;   // FP8 only: [M][KB] scales (bytes)
    const float *sb; int64_t sb_rs, sb_cs;   // FP8 only: [KB][NB] scales (bytes)
    Epilogue epi;
    float *ws;                  // split-K partials [S][M][N] FP32, or null when S == 1
    int *counters;              // direct-to-LDS kernel, S > 1: one per tile, 0 on entry and exit
    int M, N, K;
    int tiles_m, tiles_n;
    int ktiles;                 // ceil(K / BK)
    int kt_per_split;           // K tiles handled by one split piece
    int splits;                 // S
    int group_m;                // tile raster: group of tile rows walked together
    // Direct-to-LDS kernel with S > 1: the first dp_tiles tiles (in raster
    // order) run whole, one workgroup each; every later tile runs as S pieces of
    // kt_per_split K tiles, whose partials the tile's last piece adds up.  The
    // grid is dp_tiles + (tiles - dp_tiles) * S workgroups (1-D).  dp_tiles = 0
    // is plain split K; dp_tiles > 0 fills the last, partial wave of workgroups
    // with pieces of the tiles left over by the whole waves (a Stream-K-style
    // hybrid).  The register-staged kernel ignores it (grid.z = S).
    int dp_tiles;
};


struct SkinnyArgs {
    const char *A; int64_t a_rs, a_cs;   // M x K
    const char *B; int64_t b_rs, b_cs;   // K x N
    Epilogue epi;
    float *ws;                            // [S][M][N] partials when S > 1
    int *counters;                        // SK_BN, S > 1: one per column slab, 0 on entry and exit
    int M, N, K;
    int in_kind;                          // IN_F16 / IN_BF16
    int a_vec;                            // A rows K-contiguous and 16-byte aligned (SK_BN: and K % 8 == 0)
    int splits;                           // S
    int k_per_split;                      // rows of K per split (multiple of 8)
    int kc;                               // SK_BN: rows of A staged in LDS at a time
    int cols;                             // SK_BN: columns per slab (multiple of 8, <= SKINNY_BN_WIDE_COLS)
};

// SK_BN geometry: 512 threads, a slab of at most 256 columns per workgroup
// (32 lanes per row piece), or of 264 to 512 columns (64 lanes per row piece,
// the wide layout, for M <= SKINNY_WIDE_MMAX); the slab width is chosen per
// problem so that the slabs times the K splits fill the CUs.  K splits and A
// chunks are multiples of 128 rows.
constexpr int SKINNY_BN_THREADS = 512;
constexpr int SKINNY_BN_COLS = 256;
constexpr int SKINNY_BN_WIDE_COLS = 512;
constexpr int SKINNY_WIDE_MMAX = 4;
constexpr int SKINNY_BN_SWEEP = 128;
// LDS bytes of SK_BN: the A chunk [mmax][kc] 16-bit plus a spare 16-byte slot,
// or the cross-wave reduction buffer [8 waves][mmax][256 or 512] FP32,
// whichever is larger.
inline int skinny_bn_lds(int mmax, int kc, int cols) {
    const int w = cols > SKINNY_BN_COLS ? SKINNY_BN_WIDE_COLS : SKINNY_BN_COLS;
    const int a = mmax * kc * 2 + 16, r = (SKINNY_BN_THREADS / 64) * mmax * w * 4;
    return a > r ? a : r;
}

// Grouped SK_BN launch (several independent thin GEMMs in one grid): workgroup
// u belongs to the group g with unit_begin[g] <= u < unit_begin[g + 1] and runs
// that group's column slab (u - unit_begin[g]) % slabs[g] and K split
// (u - unit_begin[g]) / slabs[g].  Passed by value (kernel arguments are at
// most 4 KB), so one launch holds at most SKINNY_GROUP_MAX groups.
constexpr int SKINNY_GROUP_MAX = 16;
struct GroupedSkinnyArgs {
    int ngroups;
    int unit_begin[SKINNY_GROUP_MAX + 1];
    int slabs[SKINNY_GROUP_MAX];
    SkinnyArgs g[SKINNY_GROUP_MAX];
};
static_assert(sizeof(GroupedSkinnyArgs) <= 4096, "kernel arguments are limited to 4 KB");

// Grouped direct-to-LDS launch (several matrix-core GEMMs of one tile
// configuration in one grid, e.g. MoE experts with more than a few tokens
// each): workgroup u (after the grid's XCD mapping) belongs to the group g with
// unit_begin[g] <= u < unit_begin[g + 1] and computes that group's tile
// u - unit_begin[g] whole.  Passed by value (at most 4 KB of kernel arguments).
constexpr int MFMA_GROUP_MAX = 16;
struct GroupedMfmaArgs {
    int ngroups;
    int unit_begin[MFMA_GROUP_MAX + 1];
    MfmaArgs g[MFMA_GROUP_MAX];
};
static_assert(sizeof(GroupedMfmaArgs) <= 4096, "kernel arguments are limited to 4 KB");

struct ReduceArgs {
    const float *ws;    // [S][M][N]
    Epilogue epi;
    int M, N, S;
};

struct ScaleArgs {      // C <- act(beta * C + bias) (beta == 0: C not read), for alpha == 0 or K == 0
    Epilogue epi;
    int M, N;
};

// Tile configurations of the matrix-core kernel (index = MfmaTile).
// T64x128 exists only in the direct-to-LDS kernel (gemm_dtl.hpp).
enum MfmaTile : int { T256x256 = 0, T128x128 = 1, T64x64 = 2, T128x64 = 3, T64x128 = 4, NUM_MFMA_TILES = 5 };
inline int mfma_tile_bm(int t) { const int v[] = {256, 128, 64, 128, 64}; return v[t]; }
inline int mfma_tile_bn(int t) { const int v[] = {256, 128, 64, 64, 128}; return v[t]; }
// Workgroups of the direct-to-LDS kernel that one CU holds at once, by tile
// (LDS ring: 2 stages of 128x128 fit twice in 160 KB; the other rings fill one
// CU; every variant runs at most 2 waves per SIMD).
inline int mfma_dtl_wgs_per_cu(int t) { return t == T128x128 ? 2 : 1; }
// LDS bytes: two stages of (BM + BN) rows x 128 bytes of K (+ BM FP32 row scales for FP8).
inline int mfma_tile_lds(int t, bool fp8) {
    return 2 * ((mfma_tile_bm(t) + mfma_tile_bn(t)) * 128 + (fp8 ? mfma_tile_bm(t) * 4 : 0));
}

// Skinny (M <= 8) variants.
enum SkinnyKind : int { SK_BN = 0 /* B N-contiguous */, SK_BK = 1 /* B K-contiguous */ };

// slow != 0 selects the element-wise loader (any strides, any K) on a 64x64 tile.
hipError_t launch_mfma(int in_kind, int tile, int a_mode, int b_mode, int slow,
                       const MfmaArgs &args, hipStream_t stream);
// waves: SK_BK waves (columns) per workgroup; ignored by SK_BN.
// Matrix-core kernel with direct HBM -> LDS tile loads (gemm_dtl.hip): needs
// 16-byte chunks (vec) on both operands and K a multiple of the K tile.
bool mfma_dtl_tile(int tile);
hipError_t launch_mfma_dtl(int in_kind, int tile, int a_mode, int b_mode, const MfmaArgs &args,
                           hipStream_t stream);
// units: the sum of the groups' tile counts (unit_begin[ngroups]); FP16/BF16 only.
hipError_t launch_mfma_dtl_grouped(int in_kind, int tile, int a_mode, int b_mode, const GroupedMfmaArgs &args,
                                   int units, hipStream_t stream);
hipError_t launch_skinny(int kind, int m_max, const SkinnyArgs &args, int grid_x, int waves,
                         hipStream_t stream);
// m_max: the largest M class of the groups (1, 2, 4 or 8); wide: the groups'
// slabs are wider than SKINNY_BN_COLS (all or none of them); lds_bytes: the
// largest skinny_bn_lds of the groups.
hipError_t launch_skinny_grouped(int in_kind, int m_max, bool wide, const GroupedSkinnyArgs &args, int units,
                                 int lds_bytes, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs &args, hipStream_t stream);
hipError_t launch_scale(const ScaleArgs &args, hipStream_t stream);
hipError_t launch_fill_zero(int *p, int64_t n, hipStream_t stream);

// Fixed split-K scratch of dg_gemm_noalloc (noalloc.hip): 16 MiB of FP32
// partials and 16384 arrival counters per device, held from module load until
// the process ends.  noalloc_scratch returns the current device's addresses
// (taken with hipGetSymbolAddress at its first call on that device, which also
// zeroes the counters on `stream`).
constexpr size_t NOALLOC_WS_BYTES = size_t(16) << 20;
constexpr int NOALLOC_COUNTERS = 16384;
hipError_t noalloc_scratch(hipStream_t stream, float **ws, int **counters);

}  // namespace dg
