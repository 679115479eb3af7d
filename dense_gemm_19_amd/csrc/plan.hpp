// plan.hpp -- per-shape path and tile selection (host only, no HIP calls).
//
// The selection is shape-, precision- and layout-aware rather than a fixed
// dispatch tree ("DeepGEMM is not a new model" article, cf-1.com, section 2;
// sheratonhq.com deep dive, sections 3.1 and 5.3): thin problems (M <= 8) take
// the streaming kernel; otherwise the matrix-core kernel with the largest
// macro tile that still gives every CU a workgroup, and split-K when even the
// smallest tile leaves CUs idle (sheratonhq.com deep dive, section 5.2).
// Plans are cached per problem key under a mutex (the kwkr.cn article's
// troubleshooting table, section 5.1, asks for thread-safe kernel caching).
#pragma once
#include <cstddef>
#include <cstdint>
#include <memory>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "view.hpp"

namespace dg {

struct Device {
    bool present = false;     // false: planning for the default description below
    bool gfx950 = true;
    int cus = 256;            // compute units
    int lds_bytes = 160 * 1024;
    char arch[64] = "gfx950 (assumed, no device)";
};

struct Problem {
    bool fp8 = false;
    int in_kind = IN_BF16;
    int out_kind = OUT_F32;
    Mat A, B, C, SA, SB;
    int64_t M = 0, N = 0, K = 0;
    float alpha = 1.f, beta = 0.f;
    // fused epilogue (no influence on the plan): bias N-vector and activation
    bool has_bias = false;
    Mat bias;
    int act = ACT_NONE;
};

enum class Path : int { Noop = 0, Scale = 1, Skinny = 2, Mfma = 3 };

struct OperandPlan {
    int mode = KMAJ;          // OpMode
    int64_t r_stride = 0;     // bytes per row step (M for A, N for B)
    int64_t k_stride = 0;     // bytes per K step
    bool vec = false;         // whole 16-byte chunks are legal
};

struct Plan {
    Path path = Path::Noop;
    // matrix-core path
    int tile = T256x256;
    OperandPlan a, b;
    int slow = 0;
    int dtl = 0;              // direct HBM -> LDS kernel (gemm_dtl.hip)
    int tiles_m = 0, tiles_n = 0, ktiles = 0, kt_per_split = 0, group_m = 1;
    int dp_tiles = 0;         // direct kernel with splits: tiles run whole before the split ones
    // streaming path
    int sk_kind = SK_BN, sk_mmax = 1, sk_grid_x = 0, sk_k_per_split = 0, sk_a_vec = 0;
    int sk_kc = 0;            // SK_BN: A rows staged in LDS per chunk
    int sk_cols = 0;          // SK_BN: columns per slab (multiple of 8, at most SKINNY_BN_WIDE_COLS)
    int sk_waves = 1;         // SK_BK: waves (columns) per workgroup
    // both
    int splits = 1;
    size_t ws_bytes = 0;
    int counters = 0;         // split-K arrival counters the kernel needs (0 on entry)
    int lds_bytes = 0;
    // Column split (split_n > 0): columns [0, split_n) run as part1 (256 x 256
    // tiles filling whole waves of CUs), then columns [split_n, N) as part2, in
    // stream order on the same workspace; the fields above are part1's, except
    // ws_bytes, counters and splits, the larger of the two parts'.
    int64_t split_n = 0;
    std::shared_ptr<const Plan> part1, part2;
};

// A caller's (or the tuner's) choice among the plans the kernels implement;
// every field left at its default keeps the built-in selection.
struct PlanChoice {
    int path = 0;      // 0 built-in, 1 streaming kernel if the shape allows, 2 matrix-core kernel
    int tile = -1;     // MfmaTile, where the selected matrix-core kernel has it
    int splits = 0;    // K splits (0: built-in); the matrix-core 256x256 direct tile never splits
    int tail = -1;     // 0: never split the tail of the last wave
    bool operator==(const PlanChoice &o) const {
        return path == o.path && tile == o.tile && splits == o.splits && tail == o.tail;
    }
};

// Choose the plan for a validated problem.  Honors DG_FORCE_PATH=skinny|mfma,
// DG_FORCE_SPLITK=<n>, DG_FORCE_TILE=<256x256|128x128|64x64|128x64> and
// DG_NO_VEC=1 (element-wise loads everywhere), DG_NO_DTL=1 (register-staged
// tile loads only) and DG_NO_TAIL_SPLIT=1 (no split of the last wave's tiles),
// read once per process.
// The two parts of a column split: columns [0, n1) and [n1, N) of B, C, the
// FP8 column scales (n1 a multiple of 128) and the bias.
void split_columns(const Problem &p, int64_t n1, Problem *lo, Problem *hi);

Plan select_plan(const Problem &p, const Device &d);
Plan select_plan(const Problem &p, const Device &d, const PlanChoice &c);

// The candidate set the tuner times for a problem, kept small (the tuning
// cost must stay a small fraction of the work it speeds up): the built-in plan
// first, then every tile the selected matrix-core kernel implements that is
// not larger than the matrix, with its built-in K split and, where its grid
// holds fewer than two waves of workgroup slots, 1, 2, 4 or 8 splits; for the
// streaming kernels 1 to 16 splits.  No two candidates give the same plan.
std::vector<PlanChoice> candidate_choices(const Problem &p, const Device &d);

// Tuned plans (a choice per problem key and device), consulted by
// cached_plan before the built-in selection.  Keys cover the device (arch
// name and CU count), M, N, K, byte strides, alignments and dtypes.
void tune_store(const Problem &p, const Device &d, const PlanChoice &c);
void tune_clear();
int tune_count();
// Text file of the tuned plans: one line per entry, the key fields then the
// choice.  Load keeps entries for other devices (they match no key here).
bool tune_save(const char *path);
bool tune_load(const char *path);
std::string describe_choice(const PlanChoice &c);

// Same as select_plan (with the tuned choice of the problem's key, if any),
// through a mutex-guarded cache keyed by everything the selection reads.
// DG_LOG=1 prints each newly cached plan to stderr.
Plan cached_plan(const Problem &p, const Device &d);
// The same plan without touching the cache (for descriptions).
Plan tuned_or_selected(const Problem &p, const Device &d);

std::string describe(const Problem &p, const Plan &pl, const Device &d);

}  // namespace dg
