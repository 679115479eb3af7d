// view.hpp -- byte-strided view parsing and validation (host only, no HIP calls).
//
// A view {ptr, shape[<=4], byte stride[<=4], dtype} (DeepGEMM view-native GEMM
// article, kwkr.cn, sections 2.1 and 3.2) is reduced to a 2-D matrix with one
// row stride and one column stride.  Following the view analysis of section 2.2
// of that article, size-1 dims are dropped and adjacent dims are merged where
// stride[i] == stride[i+1] * shape[i+1]; every extent and byte offset is
// computed in checked 64-bit arithmetic (section 2.3 and the troubleshooting
// table of section 5.1 trace a wrong result to an overflowing stride product).
#pragma once
#include <cstdint>

#include "dg.h"

namespace dg {

struct Mat {
    const char *ptr = nullptr;   // element (0, 0)
    int64_t rows = 0, cols = 0;  // logical matrix
    int64_t rs = 0, cs = 0;      // byte strides of a row step and a column step
    dg_dtype dtype = DG_F32;
    int esize = 0;
    uintptr_t lo = 0, hi = 0;    // byte span [lo, hi) touched by the view (empty: lo == hi)
    int align_ptr = 0;           // largest power of two <= 16 dividing ptr
    int align_rs = 0, align_cs = 0;  // same for rs and cs (16 when the stride is unused)

    bool empty() const { return rows == 0 || cols == 0; }
    // Elements along a row are adjacent (row-major / "K-major" for A).
    bool cols_contig() const { return cols <= 1 || cs == esize; }
    // Elements along a column are adjacent (column-major).
    bool rows_contig() const { return rows <= 1 || rs == esize; }
};

int esize_of(dg_dtype t);

// Parse and validate one view.  Returns DG_SUCCESS or the first error found.
dg_status canonicalize(const dg_view *v, Mat *out);

// True if the (rows, cols, rs, cs) map is not injective (C would be written twice).
bool self_overlaps(const Mat &m);

// True if the byte spans of a and b intersect (conservative alias test).
bool spans_overlap(const Mat &a, const Mat &b);

}  // namespace dg
