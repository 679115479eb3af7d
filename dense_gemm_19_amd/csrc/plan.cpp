// plan.cpp -- see plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

namespace dg {
namespace {

struct Overrides {
    int force_path = 0;    // 0 none, 1 skinny, 2 mfma
    int force_splitk = 0;
    int force_tile = -1;
    int skinny_cols = 0;   // SK_BN slab width (multiple of 8, at most 256)
    bool no_vec = false;
    bool no_dtl = false;
    bool no_tail_split = false;
    bool log = false;
};

const Overrides &overrides() {
    static const Overrides o = [] {
        Overrides r;
        if (const char *s = std::getenv("DG_FORCE_PATH")) {
            if (!std::strcmp(s, "skinny")) r.force_path = 1;
            else if (!std::strcmp(s, "mfma")) r.force_path = 2;
        }
        if (const char *s = std::getenv("DG_FORCE_SPLITK")) r.force_splitk = std::atoi(s);
        if (const char *s = std::getenv("DG_FORCE_TILE")) {
            for (int t = 0; t < NUM_MFMA_TILES; ++t) {
                char name[32];
                std::snprintf(name, sizeof name, "%dx%d", mfma_tile_bm(t), mfma_tile_bn(t));
                if (!std::strcmp(s, name)) r.force_tile = t;
            }
        }
        if (const char *s = std::getenv("DG_SKINNY_COLS")) {
            const int v = std::atoi(s);
            if (v > 0 && v % 8 == 0 && v <= SKINNY_BN_WIDE_COLS) r.skinny_cols = v;
        }
        if (const char *s = std::getenv("DG_NO_VEC")) r.no_vec = s[0] == '1';
        if (const char *s = std::getenv("DG_NO_DTL")) r.no_dtl = s[0] == '1';
        if (const char *s = std::getenv("DG_NO_TAIL_SPLIT")) r.no_tail_split = s[0] == '1';
        if (const char *s = std::getenv("DG_LOG")) r.log = s[0] == '1';
        return r;
    }();
    return o;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A as an M x K operand ("rows" = M).
OperandPlan plan_a(const Mat &A, int64_t M, int64_t K, int epc) {
    OperandPlan o;
    if (A.cols_contig()) {
        o.mode = KMAJ; o.r_stride = A.rs; o.k_stride = A.cs;
        o.vec = A.align_ptr >= 16 && (M <= 1 || A.align_rs >= 16) && K % epc == 0 && A.cs == A.esize;
    } else if (A.rows_contig()) {
        o.mode = MNMAJ; o.r_stride = A.rs; o.k_stride = A.cs;
        o.vec = A.align_ptr >= 16 && (K <= 1 || A.align_cs >= 16) && M % epc == 0 && A.rs == A.esize;
    } else {
        o.mode = KMAJ; o.r_stride = A.rs; o.k_stride = A.cs; o.vec = false;
    }
    return o;
}

// B (K x N) as an N x K operand ("rows" = N).
OperandPlan plan_b(const Mat &B, int64_t N, int64_t K, int epc) {
    OperandPlan o;
    if (B.rows_contig() && !(B.cols_contig() && K <= 1)) {
        o.mode = KMAJ; o.r_stride = B.cs; o.k_stride = B.rs;
        o.vec = B.align_ptr >= 16 && (N <= 1 || B.align_cs >= 16) && K % epc == 0 && B.rs == B.esize;
    } else if (B.cols_contig()) {
        o.mode = MNMAJ; o.r_stride = B.cs; o.k_stride = B.rs;
        o.vec = B.align_ptr >= 16 && (K <= 1 || B.align_rs >= 16) && N % epc == 0 && B.cs == B.esize;
    } else {
        o.mode = KMAJ; o.r_stride = B.cs; o.k_stride = B.rs; o.vec = false;
    }
    return o;
}

bool skinny_ok(const Problem &p, Plan &pl, const Device &d, const PlanChoice &c) {
    if (p.fp8 || p.M > 8) return false;
    const Mat &A = p.A, &B = p.B;
    const int mmax = p.M <= 1 ? 1 : p.M <= 2 ? 2 : p.M <= 4 ? 4 : 8;
    const bool no_vec = overrides().no_vec;
    // B N-contiguous: stream row pieces of B, a slab of at most 256 columns per
    // workgroup (512 in the 64-lane layout, M <= SKINNY_WIDE_MMAX).
    if (!no_vec && B.cols_contig() && B.cs == B.esize && B.align_ptr >= 16 && (p.K <= 1 || B.align_rs >= 16)) {
        pl.sk_kind = SK_BN;
        // Slabs x K splits should fill the CUs once: a CU streams at a bounded
        // rate, so an idle CU is lost bandwidth, and a CU holding two workgroups
        // streams twice as much as the others and sets the pace.  For each
        // split count S (whole sweeps of as nearly equal length as S allows, at
        // least two each) the slab is the narrowest multiple of 8 columns (at
        // most 256, or 512 in the wide layout for M <= SKINNY_WIDE_MMAX, and at
        // least 64, i.e. 128-byte lines, where N allows) that keeps slabs x S
        // within the CUs.  The score is the CUs kept busy, discounted for
        // unequal splits and for the bytes of 128-byte lines a row's slabs
        // touch beyond the row itself (a slab edge inside a line makes two
        // workgroups fetch that line).  Among scores within 3% of the best: the
        // fewest splits whose slab is at least 128 columns (256-byte row pieces;
        // a split adds the partial sum's round trips at the end), else the
        // widest slab.  Measured on x.W1 (BF16, N = 14336, K = 4096, 256 CUs):
        // 448-byte pieces (slab edges inside lines) on 256 workgroups 23.8 us
        // against 21.1 us for 896-byte pieces on line boundaries, 256-byte pieces
        // (224 workgroups) 25.7 us, 128-byte pieces 34.6 us; on 8 grouped
        // [1,512] x [512,4096] experts, 128-column slabs without a split 9.2 us
        // against 10.1 us for 256-column slabs in 2 splits.
        const int64_t sweep = SKINNY_BN_SWEEP;
        const int64_t sweeps = cdiv(std::max<int64_t>(p.K, 1), sweep);
        const int64_t maxcols = mmax <= SKINNY_WIDE_MMAX ? SKINNY_BN_WIDE_COLS : SKINNY_BN_COLS;
        auto geometry = [&](int64_t S, int64_t &kps, int64_t &cols, int64_t &slabs) {
            kps = cdiv(sweeps, S) * sweep;
            S = cdiv(std::max<int64_t>(p.K, 1), kps);
            const int64_t target = std::max<int64_t>(1, d.cus / S);
            const int64_t lo = std::min<int64_t>(64, cdiv(std::max<int64_t>(p.N, 1), 8) * 8);
            cols = std::min<int64_t>(maxcols, std::max<int64_t>(lo, cdiv(cdiv(p.N, target), 8) * 8));
            if (overrides().skinny_cols > 0) cols = std::min<int64_t>(maxcols, overrides().skinny_cols);
            slabs = cdiv(p.N, cols);
            return S;
        };
        // bytes of a row of B over the bytes of the 128-byte lines its slabs
        // fetch (rows assumed to start on a line)
        auto line_eff = [&](int64_t cols, int64_t slabs) {
            const int64_t es = B.esize, row = p.N * es;
            int64_t lines = 0;
            for (int64_t sl = 0; sl < slabs; ++sl) {
                const int64_t b0 = sl * cols * es, b1 = std::min(row, (sl + 1) * cols * es);
                lines += (b1 - 1) / 128 - b0 / 128 + 1;
            }
            return (double)row / (double)(lines * 128);
        };
        int64_t S = 1;
        const int64_t forced = c.splits > 0 ? c.splits : overrides().force_splitk;
        if (forced > 0) {
            S = std::min<int64_t>(forced, sweeps);
        } else {
            const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(sweeps / 2, d.cus));
            struct Opt { int64_t S, cols; double score, eff; };
            std::vector<Opt> opts;
            double best = 0.0;
            for (int64_t s = 1; s <= smax; ++s) {
                int64_t kps, cols, slabs;
                if (geometry(s, kps, cols, slabs) != s) continue;   // the rounding gives another count
                const double units = (double)(slabs * s);
                const double busy = units / std::max<double>(1.0, std::ceil(units / d.cus));   // per wave of CUs
                const double eff = line_eff(cols, slabs);
                const double score = busy * ((double)sweeps / (double)(s * (kps / sweep))) * eff;
                opts.push_back({s, cols, score, eff});
                best = std::max(best, score);
            }
            // (slab edges on line boundaries first, at equal scores)
            int64_t wide_cols = 0, pick = 0, pick_aligned = 0;
            for (const Opt &o : opts) {                                  // in increasing S
                if (o.score < 0.97 * best) continue;
                if (pick_aligned == 0 && o.cols >= 128 && o.eff > 0.99) pick_aligned = o.S;
                if (pick == 0 && o.cols >= 128) pick = o.S;
                if (o.cols > wide_cols) { S = o.S; wide_cols = o.cols; }
            }
            if (pick_aligned > 0) S = pick_aligned;
            else if (pick > 0) S = pick;
        }
        int64_t kps, cols, slabs;
        geometry(S, kps, cols, slabs);
        pl.sk_grid_x = (int)slabs;
        pl.sk_cols = (int)cols;
        pl.sk_k_per_split = (int)kps;
        pl.splits = (int)cdiv(std::max<int64_t>(p.K, 1), kps);
        pl.sk_mmax = mmax;
        // A chunk in LDS: a multiple of the sweep, at most 32 KB
        const int64_t kc_max = std::max<int64_t>(sweep, (16384 / mmax) / sweep * sweep);
        pl.sk_kc = (int)std::min<int64_t>(cdiv(kps, sweep) * sweep, kc_max);
        pl.lds_bytes = skinny_bn_lds(mmax, pl.sk_kc, pl.sk_cols);
        pl.counters = pl.splits > 1 ? pl.sk_grid_x : 0;
        // A staged with 16-byte loads: K-contiguous 16-byte-aligned rows, and K a
        // multiple of 8 so that no piece crosses the end of a row
        pl.sk_a_vec = A.cols_contig() && A.cs == A.esize && A.align_ptr >= 16 && (p.M <= 1 || A.align_rs >= 16) &&
                      p.K % 8 == 0;
        return true;
    }
    // B K-contiguous (e.g. a transposed cache): one wave per column.
    if (!no_vec && B.rows_contig() && B.rs == B.esize && B.align_ptr >= 16 && (p.N <= 1 || B.align_cs >= 16)) {
        pl.sk_kind = SK_BK;
        pl.sk_waves = p.N < 1024 ? 1 : 4;   // few columns: one per workgroup, spread over CUs
        pl.sk_grid_x = (int)cdiv(p.N, pl.sk_waves);
        int64_t S = 1;
        if (overrides().force_splitk > 0) S = overrides().force_splitk;
        if (c.splits > 0) S = c.splits;
        int64_t kps = cdiv(cdiv(std::max<int64_t>(p.K, 1), S), 8) * 8;
        pl.sk_k_per_split = (int)kps;
        pl.splits = (int)cdiv(std::max<int64_t>(p.K, 1), kps);
        pl.sk_mmax = mmax;
        pl.sk_a_vec = A.cols_contig() && A.cs == A.esize && A.align_ptr >= 16 && (p.M <= 1 || A.align_rs >= 16);
        pl.lds_bytes = 0;
        return true;
    }
    return false;
}

// Fraction of a tile grid's area that is real (not padding past M or N).
double tile_eff(int64_t M, int64_t N, int t) {
    const int64_t tm = cdiv(M, mfma_tile_bm(t)), tn = cdiv(N, mfma_tile_bn(t));
    return (double)M * (double)N / ((double)tm * mfma_tile_bm(t) * (double)tn * mfma_tile_bn(t));
}

int64_t tile_count(int64_t M, int64_t N, int t) {
    return cdiv(M, mfma_tile_bm(t)) * cdiv(N, mfma_tile_bn(t));
}

void plan_mfma(const Problem &p, Plan &pl, const Device &d, const PlanChoice &c) {
    const int epc = p.fp8 ? 16 : 8;              // elements per 16-byte chunk
    const int kel = p.fp8 ? 128 : 64;            // K elements per tile
    pl.path = Path::Mfma;
    pl.a = plan_a(p.A, p.M, p.K, epc);
    pl.b = plan_b(p.B, p.N, p.K, epc);
    if (overrides().no_vec) pl.a.vec = pl.b.vec = false;
    pl.slow = !(pl.a.vec && pl.b.vec);
    pl.ktiles = (int)cdiv(p.K, kel);
    // The direct-to-LDS kernel serves whole 16-byte chunks and whole K tiles,
    // and addresses a lane's chunks with 32-bit offsets from the tile's first
    // row (and the FP8 scales with 32-bit offsets from their K column): every
    // such offset must stay below 2^31.
    const int64_t lim = int64_t(1) << 31;
    const bool a_fits = 255 * pl.a.r_stride + (kel - 1) * pl.a.k_stride + 16 < lim;
    const bool b_fits = 255 * pl.b.r_stride + (kel - 1) * pl.b.k_stride + 16 < lim;
    const bool s_fits = !p.fp8 || ((p.M - 1) * p.SA.rs + 4 < lim && (cdiv(p.N, 128) - 1) * p.SB.cs + 4 < lim);
    pl.dtl = !pl.slow && p.K % kel == 0 && a_fits && b_fits && s_fits && !overrides().no_dtl;
    // Tile: the heuristic below, or the caller's choice where the kernel has it.
    int tile = T64x64;
    if (pl.dtl) {
        if (p.M <= 128) {
            // Few rows: the shape is bound by streaming B, and the work is split
            // over K to keep enough workgroups streaming.  Measured on MI355X
            // (64x4096x4096 FP16, 128x7168x4096 FP8, 64x512x512): 64x64 tiles for
            // 16-bit inputs and 64x128 for FP8 (twice the B bytes per K tile of
            // A), each split holding at least 16 K tiles, up to about one
            // workgroup per CU; each split adds a fixed cost (partials written,
            // a ticket, partials read back by the last workgroup).
            tile = p.fp8 ? T64x128 : T64x64;
            if (p.M > 64 && !p.fp8 && tile_eff(p.M, p.N, T128x64) > tile_eff(p.M, p.N, tile) + 1e-9) tile = T128x64;
        } else if (p.fp8 && p.N <= 128 && tile_count(p.M, p.N, T64x128) < d.cus) {
            // A tall FP8 strip (the columns a column split leaves): 64x128 tiles
            // span its columns, so A is read once, and its K split (below) fills
            // the CUs.  Measured on 4096 x 128 x 4096: 64x128 in 4 splits 14.9 us,
            // 128x64 in 4 15.4, 64x64 in 2 16.1, 128x128 in 4 19.3.
            tile = T64x128;
        } else {
            // Enough rows for a compute-bound shape: the largest tile that still
            // gives every CU a tile, else the one giving the most tiles.  FP8 takes
            // 256x256 (one workgroup per CU, no K split) only where its tiles fill
            // at least 3/4 of the CU waves they occupy; a short last wave is
            // better served by 128x128 and its split tail.  Measured on
            // 4096x7168x4096: 256x256 148.9 us, 128x128 171 us.
            const int order[] = {T256x256, T128x128, T128x64, T64x64};
            int64_t best_tiles = -1;
            for (int t : order) {
                if (p.fp8 && t == T256x256) {
                    const int64_t nt = tile_count(p.M, p.N, t);
                    if (nt < d.cus || (double)nt / (double)(cdiv(nt, d.cus) * d.cus) < 0.75) continue;
                }
                if (tile_eff(p.M, p.N, t) < 0.75 && t != T64x64) continue;
                const int64_t nt = tile_count(p.M, p.N, t);
                if (nt >= d.cus) { tile = t; break; }
                if (nt > best_tiles) { best_tiles = nt; tile = t; }
            }
        }
        if (overrides().force_tile >= 0) tile = overrides().force_tile;
        if (c.tile >= 0) tile = c.tile;
    } else if (!pl.slow) {
        // general kernel (register-staged loads, K tails): tiles it implements
        // (no 256x256: its accumulators and staging registers would spill)
        const int order[] = {T128x128, T128x64, T64x64};
        int best = T64x64;
        int64_t best_tiles = -1;
        bool found = false;
        for (int t : order) {
            if (tile_eff(p.M, p.N, t) < 0.75 && t != T64x64) continue;
            const int64_t nt = tile_count(p.M, p.N, t);
            if (nt >= d.cus) { tile = t; found = true; break; }
            if (nt > best_tiles) { best_tiles = nt; best = t; }
        }
        if (!found) tile = best;
        const auto general_has = [](int t) { return t != T64x128 && t != T256x256; };
        if (overrides().force_tile >= 0 && general_has(overrides().force_tile)) tile = overrides().force_tile;
        if (c.tile >= 0 && general_has(c.tile)) tile = c.tile;
    }
    // K split for that tile.
    int64_t S = 1;
    const int64_t nt = tile_count(p.M, p.N, tile);
    if (pl.dtl) {
        if (p.M <= 128) {
            S = std::max<int64_t>(1, std::min<int64_t>(cdiv(d.cus, nt), pl.ktiles / 16));
            // Very few tiles (a quarter of the CUs or less): up to 4 splits of as
            // few as 2 K tiles; the split-K sum loads its partials in one round
            // trip, so short splits pay (FP16 64x512x512: 6.9 -> 6.4 us with 4).
            if (nt * 4 <= d.cus)
                S = std::max<int64_t>(S, std::min<int64_t>({cdiv(d.cus, nt), std::max<int64_t>(1, pl.ktiles / 2), 4}));
        } else if (nt < d.cus && tile != T256x256 && tile != T128x128)
            S = std::max<int64_t>(1, std::min<int64_t>(cdiv(d.cus, nt), pl.ktiles / 8));
    } else if (!pl.slow) {
        if (nt < d.cus) S = std::min<int64_t>(cdiv(d.cus, nt), std::max<int64_t>(1, pl.ktiles / 2));
        S = std::min<int64_t>(S, 16);
    }
    pl.tile = tile;
    pl.tiles_m = (int)cdiv(p.M, mfma_tile_bm(tile));
    pl.tiles_n = (int)cdiv(p.N, mfma_tile_bn(tile));
    if (overrides().force_splitk > 0) S = std::min<int64_t>(overrides().force_splitk, std::max(pl.ktiles, 1));
    if (c.splits > 0) S = std::min<int64_t>(c.splits, std::max(pl.ktiles, 1));
    // the direct kernel splits K only on tiles of at most 64 accumulators per lane
    if (pl.dtl && (tile == T256x256)) S = 1;
    S = std::max<int64_t>(S, 1);
    // Tail of the last wave (direct kernel, whole tiles): when the tiles fill
    // whole waves of workgroup slots and the tiles left over would keep at most
    // half of the CUs busy, those tiles are split along K into pieces that
    // spread over the idle CUs (the earlier tiles stay whole, so the split
    // costs only on the tail).  A last wave with a tile on every CU needs no
    // help: a CU running one workgroup instead of two runs it about twice as
    // fast (measured on FP8 4096 x 7168, 1792 tiles = 3.5 waves of 512 slots:
    // splitting its last 256 tiles made it slower, 189 us against 185 us).
    pl.dp_tiles = 0;
    if (pl.dtl && S == 1 && tile != T256x256 && overrides().force_splitk <= 0 && !overrides().no_tail_split &&
        c.splits <= 0 && c.tail != 0) {
        const int64_t slots = (int64_t)d.cus * mfma_dtl_wgs_per_cu(tile);
        const int64_t full = nt / slots, left = nt - full * slots;
        if (full >= 1 && left > 0 && 2 * left <= d.cus) {
            const int64_t St = std::min<int64_t>(d.cus / left, pl.ktiles / 8);
            if (St >= 2) {
                S = St;
                pl.dp_tiles = (int)(full * slots);
            }
        }
    }
    pl.kt_per_split = (int)cdiv(std::max(pl.ktiles, 1), S);
    pl.splits = (int)cdiv(std::max(pl.ktiles, 1), pl.kt_per_split);
    // tile raster: a group of tile rows walked together (measured on the
    // 4096-sized workloads: 4 rows of 256x256 tiles, 8 of 128x128)
    pl.group_m = std::min(pl.tiles_m, tile == T128x128 ? 8 : 4);
    pl.lds_bytes = mfma_tile_lds(pl.slow ? T64x64 : tile, p.fp8);
    pl.counters = pl.dtl && pl.splits > 1 ? pl.tiles_m * pl.tiles_n : 0;
    // the direct kernel's partials: one BM x BN tile per piece of each split tile
    if (pl.dtl && pl.splits > 1)
        pl.ws_bytes = (size_t)(pl.tiles_m * pl.tiles_n - pl.dp_tiles) * (size_t)pl.splits *
                      (size_t)mfma_tile_bm(tile) * (size_t)mfma_tile_bn(tile) * sizeof(float);
}

}  // namespace

Plan select_plan(const Problem &p, const Device &d) { return select_plan(p, d, PlanChoice()); }

namespace {

int ptr_align(const char *p) {
    const uintptr_t v = reinterpret_cast<uintptr_t>(p);
    int a = 1;
    while (a < 16 && (v % (2 * a)) == 0) a *= 2;
    return a;
}

void cut_columns(Mat &m, int64_t c0, int64_t n) {
    m.ptr += c0 * m.cs;
    m.cols = n;
    m.align_ptr = ptr_align(m.ptr);
}

}  // namespace

void split_columns(const Problem &p, int64_t n1, Problem *lo, Problem *hi) {
    *lo = p;
    *hi = p;
    lo->N = n1;
    hi->N = p.N - n1;
    cut_columns(lo->B, 0, n1);
    cut_columns(hi->B, n1, p.N - n1);
    cut_columns(lo->C, 0, n1);
    cut_columns(hi->C, n1, p.N - n1);
    if (p.fp8) {
        const int64_t nb = cdiv(p.N, 128), nb1 = n1 / 128;
        cut_columns(lo->SB, 0, nb1);
        cut_columns(hi->SB, nb1, nb - nb1);
    }
    if (p.has_bias) {
        cut_columns(lo->bias, 0, n1);
        cut_columns(hi->bias, n1, p.N - n1);
    }
}

namespace {

Plan select_plan_one(const Problem &p, const Device &d, const PlanChoice &c) {
    Plan pl;
    if (p.M == 0 || p.N == 0) { pl.path = Path::Noop; return pl; }
    if (p.alpha == 0.0f || p.K == 0) { pl.path = Path::Scale; return pl; }
    const int fp = c.path ? c.path : overrides().force_path;
    if (fp != 2 && skinny_ok(p, pl, d, c)) {
        pl.path = Path::Skinny;
    } else {
        pl = Plan();
        plan_mfma(p, pl, d, c);
    }
    if (!(pl.path == Path::Mfma && pl.dtl))
        pl.ws_bytes = pl.splits > 1 ? (size_t)pl.splits * (size_t)p.M * (size_t)p.N * sizeof(float) : 0;
    return pl;
}

}  // namespace

Plan select_plan(const Problem &p, const Device &d, const PlanChoice &c) {
    Plan pl = select_plan_one(p, d, c);
    // Column split of the built-in plan: where the grid of 256 x 256 tiles
    // would end in a short wave (the direct kernel then took smaller tiles for
    // FP8, or 256 x 256 with that wave for 16-bit inputs), but the columns up to
    // the last multiple of 256 fill whole waves of 256 x 256 tiles (and fewer
    // than 256 columns remain), those columns run on that tile and the
    // remaining strip as a problem of its own (its K split spreads it over the
    // CUs) right after.  FP8 4096 x 4224 x 4096: 256 whole 256 x 256 tiles, then
    // a 4096 x 128 strip, instead of 128 x 128 tiles with a split tail; BF16
    // 4096 x 4160: 256 tiles and a 4096 x 64 strip instead of 272 tiles, whose
    // second wave of 16 would take as long as the first.
    if (!(c == PlanChoice()) || overrides().force_tile >= 0 || overrides().force_splitk > 0 ||
        pl.path != Path::Mfma || !pl.dtl || p.M < 256)
        return pl;
    if (pl.tile == T256x256) {   // (16-bit inputs take it whatever the last wave holds)
        const int64_t nt = tile_count(p.M, p.N, T256x256);
        if ((double)nt / (double)(cdiv(nt, d.cus) * d.cus) >= 0.9) return pl;
    }
    const int64_t n1 = p.N / 256 * 256;
    if (n1 == 0 || n1 == p.N) return pl;
    const int64_t nt1 = cdiv(p.M, 256) * (n1 / 256);
    if (nt1 < d.cus || (double)nt1 / (double)(cdiv(nt1, d.cus) * d.cus) < 0.9 || tile_eff(p.M, n1, T256x256) < 0.9)
        return pl;
    Problem lo, hi;
    split_columns(p, n1, &lo, &hi);
    const Plan a = select_plan_one(lo, d, c), b = select_plan_one(hi, d, c);
    if (!(a.path == Path::Mfma && a.dtl && a.tile == T256x256)) return pl;
    Plan out = a;
    out.split_n = n1;
    out.ws_bytes = std::max(a.ws_bytes, b.ws_bytes);
    out.counters = std::max(a.counters, b.counters);
    out.splits = std::max(a.splits, b.splits);
    out.part1 = std::make_shared<const Plan>(a);
    out.part2 = std::make_shared<const Plan>(b);
    return out;
}

namespace {

struct Key {
    char arch[16];            // device architecture name up to its first ':' or ' '
    int64_t M, N, K;
    int64_t ars, acs, brs, bcs, sars, sbcs;
    int fp8, in_kind, out_kind, scale_only;
    int aal, bal, aalr, aalc, balr, balc;
    int cus;
    bool operator==(const Key &o) const { return std::memcmp(this, &o, sizeof(Key)) == 0; }
};

struct KeyHash {
    size_t operator()(const Key &k) const {
        const unsigned char *b = reinterpret_cast<const unsigned char *>(&k);
        size_t h = 1469598103934665603ull;
        for (size_t i = 0; i < sizeof(Key); ++i) h = (h ^ b[i]) * 1099511628211ull;
        return h;
    }
};

Key make_key(const Problem &p, const Device &d) {
    Key k;
    std::memset(&k, 0, sizeof k);
    for (int i = 0; i < 15 && d.arch[i] && d.arch[i] != ':' && d.arch[i] != ' '; ++i) k.arch[i] = d.arch[i];
    k.M = p.M; k.N = p.N; k.K = p.K;
    k.ars = p.A.rs; k.acs = p.A.cs; k.brs = p.B.rs; k.bcs = p.B.cs;
    k.sars = p.fp8 ? p.SA.rs : 0; k.sbcs = p.fp8 ? p.SB.cs : 0;
    k.fp8 = p.fp8; k.in_kind = p.in_kind; k.out_kind = p.out_kind;
    k.scale_only = (p.alpha == 0.0f);
    k.aal = p.A.align_ptr; k.bal = p.B.align_ptr;
    k.aalr = p.A.align_rs; k.aalc = p.A.align_cs; k.balr = p.B.align_rs; k.balc = p.B.align_cs;
    k.cus = d.cus;
    return k;
}

// The plan cache and the tuned choices, under one mutex (a tuned choice
// replaces the cached plan of its key).
struct Tables {
    std::mutex mu;
    std::unordered_map<Key, Plan, KeyHash> plans;
    std::unordered_map<Key, PlanChoice, KeyHash> tuned;
};

Tables &tables() {
    static Tables t;
    return t;
}

}  // namespace

Plan cached_plan(const Problem &p, const Device &d) {
    const Key k = make_key(p, d);
    Tables &t = tables();
    PlanChoice c;
    {
        std::lock_guard<std::mutex> g(t.mu);
        auto it = t.plans.find(k);
        if (it != t.plans.end()) return it->second;
        auto tc = t.tuned.find(k);
        if (tc != t.tuned.end()) c = tc->second;
    }
    Plan pl = select_plan(p, d, c);
    std::lock_guard<std::mutex> g(t.mu);
    auto ins = t.plans.emplace(k, pl);
    if (ins.second && overrides().log) std::fprintf(stderr, "[dg] %s\n", describe(p, pl, d).c_str());
    return ins.first->second;
}

Plan tuned_or_selected(const Problem &p, const Device &d) {
    const Key k = make_key(p, d);
    Tables &t = tables();
    PlanChoice c;
    {
        std::lock_guard<std::mutex> g(t.mu);
        auto tc = t.tuned.find(k);
        if (tc != t.tuned.end()) c = tc->second;
    }
    return select_plan(p, d, c);
}

void tune_store(const Problem &p, const Device &d, const PlanChoice &c) {
    const Key k = make_key(p, d);
    Tables &t = tables();
    std::lock_guard<std::mutex> g(t.mu);
    t.tuned[k] = c;
    t.plans.erase(k);
}

void tune_clear() {
    Tables &t = tables();
    std::lock_guard<std::mutex> g(t.mu);
    t.tuned.clear();
    t.plans.clear();
}

int tune_count() {
    Tables &t = tables();
    std::lock_guard<std::mutex> g(t.mu);
    return (int)t.tuned.size();
}

// One line per entry:
//   dgtune1 <arch> <cus> <M> <N> <K> <ars> <acs> <brs> <bcs> <sars> <sbcs> <fp8> <in> <out>
//           <scale_only> <aal> <bal> <aalr> <aalc> <balr> <balc> <path> <tile> <splits> <tail>
bool tune_save(const char *path) {
    Tables &t = tables();
    std::lock_guard<std::mutex> g(t.mu);
    FILE *f = std::fopen(path, "w");
    if (!f) return false;
    bool ok = std::fprintf(f, "# dense GEMM tuned plans: key fields, then path tile splits tail\n") > 0;
    for (const auto &e : t.tuned) {
        const Key &k = e.first;
        const PlanChoice &c = e.second;
        ok = ok && std::fprintf(f,
                                "dgtune1 %s %d %lld %lld %lld %lld %lld %lld %lld %lld %lld %d %d %d %d %d %d %d %d %d %d "
                                "%d %d %d %d\n",
                                k.arch[0] ? k.arch : "-", k.cus, (long long)k.M, (long long)k.N, (long long)k.K,
                                (long long)k.ars, (long long)k.acs, (long long)k.brs, (long long)k.bcs,
                                (long long)k.sars, (long long)k.sbcs, k.fp8, k.in_kind, k.out_kind, k.scale_only,
                                k.aal, k.bal, k.aalr, k.aalc, k.balr, k.balc, c.path, c.tile, c.splits, c.tail) > 0;
    }
    return std::fclose(f) == 0 && ok;
}

bool tune_load(const char *path) {
    FILE *f = std::fopen(path, "r");
    if (!f) return false;
    std::vector<std::pair<Key, PlanChoice>> got;
    char line[1024];
    bool ok = true;
    while (std::fgets(line, sizeof line, f)) {
        if (line[0] == '#' || line[0] == '\n') continue;
        Key k;
        std::memset(&k, 0, sizeof k);
        PlanChoice c;
        char arch[64];
        long long v[11];
        int n = std::sscanf(line,
                            "dgtune1 %63s %d %lld %lld %lld %lld %lld %lld %lld %lld %lld %d %d %d %d %d %d %d %d %d %d "
                            "%d %d %d %d",
                            arch, &k.cus, &v[0], &v[1], &v[2], &v[3], &v[4], &v[5], &v[6], &v[7], &v[8], &k.fp8,
                            &k.in_kind, &k.out_kind, &k.scale_only, &k.aal, &k.bal, &k.aalr, &k.aalc, &k.balr,
                            &k.balc, &c.path, &c.tile, &c.splits, &c.tail);
        if (n != 25 || c.path < 0 || c.path > 2 || c.tile < -1 || c.tile >= NUM_MFMA_TILES || c.splits < 0 ||
            c.splits > 64) {
            ok = false;
            break;
        }
        if (std::strcmp(arch, "-") != 0) std::snprintf(k.arch, sizeof k.arch, "%.15s", arch);
        k.M = v[0]; k.N = v[1]; k.K = v[2]; k.ars = v[3]; k.acs = v[4]; k.brs = v[5]; k.bcs = v[6];
        k.sars = v[7]; k.sbcs = v[8];
        got.emplace_back(k, c);
    }
    std::fclose(f);
    if (!ok) return false;   // nothing from a malformed file is used
    Tables &t = tables();
    std::lock_guard<std::mutex> g(t.mu);
    for (const auto &e : got) {
        t.tuned[e.first] = e.second;
        t.plans.erase(e.first);
    }
    return true;
}

std::vector<PlanChoice> candidate_choices(const Problem &p, const Device &d) {
    std::vector<PlanChoice> out;
    std::vector<std::string> seen;
    auto add = [&](const PlanChoice &c) {
        const std::string s = describe(p, select_plan(p, d, c), d);
        for (const std::string &x : seen)
            if (x == s) return;
        seen.push_back(s);
        out.push_back(c);
    };
    add(PlanChoice());   // the built-in selection
    const Plan def = select_plan(p, d);
    if (def.path == Path::Skinny) {
        for (int S : {1, 2, 3, 4, 6, 8, 12, 16}) {
            PlanChoice c;
            c.path = 1;
            c.splits = S;
            add(c);
        }
    } else if (def.path == Path::Mfma) {
        std::vector<int> tiles;
        if (def.dtl) tiles = {T256x256, T128x128, T128x64, T64x64, T64x128};
        else if (!def.slow) tiles = {T128x128, T128x64, T64x64};
        else tiles = {-1};
        for (int t : tiles) {
            // no tile larger than the matrix in either dimension
            if (t >= 0 && (mfma_tile_bm(t) > std::max<int64_t>(64, p.M) || mfma_tile_bn(t) > std::max<int64_t>(64, p.N)))
                continue;
            PlanChoice c;
            c.path = 2;
            c.tile = t;
            add(c);
            // K splits only where the tile's grid holds fewer than two waves of
            // workgroup slots (a fuller grid has parallelism to spare)
            const int64_t nt = tile_count(p.M, p.N, t >= 0 ? t : T64x64);
            if (nt >= 2 * (int64_t)d.cus * mfma_dtl_wgs_per_cu(t >= 0 ? t : T64x64)) continue;
            for (int S : {1, 2, 4, 8}) {
                c.splits = S;
                c.tail = 0;
                add(c);
            }
        }
    }
    return out;
}

std::string describe_choice(const PlanChoice &c) {
    char b[128];
    std::snprintf(b, sizeof b, "path=%d tile=%s splits=%d tail=%d", c.path,
                  c.tile < 0 ? "auto" : (std::to_string(mfma_tile_bm(c.tile)) + "x" + std::to_string(mfma_tile_bn(c.tile))).c_str(),
                  c.splits, c.tail);
    return b;
}

std::string describe_core(const Plan &pl);

std::string describe(const Problem &p, const Plan &pl, const Device &d) {
    static const char *kinds[] = {"f16", "bf16", "f8e4m3"};
    static const char *outs[] = {"f32", "f16", "bf16"};
    char buf[1024];
    int n = 0;
    auto add = [&](const char *fmt, auto... args) {
        if (n < (int)sizeof buf) n += std::snprintf(buf + n, sizeof buf - n, fmt, args...);
    };
    add("M=%lld N=%lld K=%lld in=%s out=%s alpha=%g beta=%g", (long long)p.M, (long long)p.N,
        (long long)p.K, kinds[p.in_kind], outs[p.out_kind], (double)p.alpha, (double)p.beta);
    if (pl.split_n > 0) {
        add(" path=split_n n1=%lld ws=%zu | part1 {%s} | part2 {%s}", (long long)pl.split_n, pl.ws_bytes,
            describe_core(*pl.part1).c_str(), describe_core(*pl.part2).c_str());
    } else {
        add("%s", describe_core(pl).c_str());
        add(" ws=%zu", pl.ws_bytes);
    }
    add(" | A %lldx%lld rs=%lld cs=%lld | B %lldx%lld rs=%lld cs=%lld | C %lldx%lld rs=%lld cs=%lld",
        (long long)p.A.rows, (long long)p.A.cols, (long long)p.A.rs, (long long)p.A.cs,
        (long long)p.B.rows, (long long)p.B.cols, (long long)p.B.rs, (long long)p.B.cs,
        (long long)p.C.rows, (long long)p.C.cols, (long long)p.C.rs, (long long)p.C.cs);
    add(" | device %s cus=%d", d.arch, d.cus);
    return std::string(buf, std::min<size_t>(n, sizeof buf - 1));
}

// The kernel-path part of a plan's description.
std::string describe_core(const Plan &pl) {
    static const char *modes[] = {"KMAJ", "MNMAJ"};
    char buf[512];
    int n = 0;
    auto add = [&](const char *fmt, auto... args) {
        if (n < (int)sizeof buf) n += std::snprintf(buf + n, sizeof buf - n, fmt, args...);
    };
    switch (pl.path) {
    case Path::Noop: add(" path=noop"); break;
    case Path::Scale: add(" path=scale"); break;
    case Path::Skinny:
        add(" path=skinny kind=%s mmax=%d grid=%dx%d k_per_split=%d splits=%d kc=%d waves=%d a_vec=%d lds=%d",
            pl.sk_kind == SK_BN ? "BN" : "BK", pl.sk_mmax, pl.sk_grid_x, pl.splits, pl.sk_k_per_split,
            pl.splits, pl.sk_kc, pl.sk_kind == SK_BN ? SKINNY_BN_THREADS / 64 : pl.sk_waves, pl.sk_a_vec, pl.lds_bytes);
        if (pl.sk_kind == SK_BN) add(" cols=%d", pl.sk_cols);
        break;
    case Path::Mfma:
        add(" path=mfma tile=%dx%d a=%s b=%s vec=%d/%d slow=%d dtl=%d tiles=%dx%d ktiles=%d splits=%d "
            "kt_per_split=%d dp_tiles=%d group_m=%d grid=%dx1x%d lds=%d",
            mfma_tile_bm(pl.slow ? T64x64 : pl.tile), mfma_tile_bn(pl.slow ? T64x64 : pl.tile),
            modes[pl.a.mode], modes[pl.b.mode], (int)pl.a.vec, (int)pl.b.vec, pl.slow, pl.dtl, pl.tiles_m,
            pl.tiles_n, pl.ktiles, pl.splits, pl.kt_per_split, pl.dp_tiles, pl.group_m,
            pl.dtl && pl.splits > 1 ? pl.dp_tiles + (pl.tiles_m * pl.tiles_n - pl.dp_tiles) * pl.splits
                                    : pl.tiles_m * pl.tiles_n,
            pl.dtl ? 1 : pl.splits, pl.lds_bytes);
        break;
    }
    return std::string(buf, std::min<size_t>(n, sizeof buf - 1));
}

}  // namespace dg
