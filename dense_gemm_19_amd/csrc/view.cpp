// view.cpp -- see view.hpp.
#include "view.hpp"

namespace dg {

int esize_of(dg_dtype t) {
    switch (t) {
    case DG_F32: return 4;
    case DG_F16: case DG_BF16: return 2;
    case DG_F8E4M3: return 1;
    }
    return 0;
}

static int pow2_align(uint64_t x) {
    if (x == 0) return 16;
    int a = 1;
    while (a < 16 && (x % (uint64_t)(a * 2)) == 0) a *= 2;
    return a;
}

static bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }
static bool add_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_add_overflow(a, b, r); }

dg_status canonicalize(const dg_view *v, Mat *out) {
    if (!v) return DG_ERR_NULL;
    if (v->ndim < 1 || v->ndim > 4) return DG_ERR_NDIM;
    const int es = esize_of(v->dtype);
    if (es == 0) return DG_ERR_DTYPE;
    const int nd = v->ndim;
    for (int d = 0; d < nd; ++d) {
        if (v->shape[d] < 0 || v->stride[d] < 0) return DG_ERR_STRIDE;
        if (v->stride[d] % es != 0) return DG_ERR_STRIDE;
    }
    Mat m;
    m.dtype = v->dtype;
    m.esize = es;
    int64_t rows = 1;
    for (int d = 0; d + 1 < nd; ++d)
        if (!mul_ok(rows, v->shape[d], &rows)) return DG_ERR_OVERFLOW;
    m.rows = rows;
    m.cols = v->shape[nd - 1];
    int64_t total;
    if (!mul_ok(m.rows, m.cols, &total)) return DG_ERR_OVERFLOW;
    if (!m.empty() && v->ptr == nullptr) return DG_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(v->ptr) % (uintptr_t)es != 0) return DG_ERR_MISALIGNED;

    // Largest byte offset reached, in checked arithmetic.
    int64_t maxoff = 0;
    if (!m.empty()) {
        for (int d = 0; d < nd; ++d) {
            int64_t t;
            if (!mul_ok(v->shape[d] - 1, v->stride[d], &t) || !add_ok(maxoff, t, &maxoff))
                return DG_ERR_OVERFLOW;
        }
        int64_t end;
        if (!add_ok(maxoff, es, &end)) return DG_ERR_OVERFLOW;
        uintptr_t p = reinterpret_cast<uintptr_t>(v->ptr), hi;
        if (__builtin_add_overflow(p, (uintptr_t)end, &hi)) return DG_ERR_OVERFLOW;
        m.lo = p;
        m.hi = hi;
    } else {
        m.lo = m.hi = reinterpret_cast<uintptr_t>(v->ptr);
    }

    // Merge the leading (row) dims into one stride: drop size-1 dims (any
    // stride), then walk outward requiring stride[i] == stride_inner * extent.
    int64_t g_stride = 0, g_extent = 0;
    bool have = false;
    for (int d = nd - 2; d >= 0; --d) {
        if (v->shape[d] == 1) continue;
        if (v->shape[d] == 0) { have = false; g_stride = 0; break; }  // empty view
        if (!have) {
            g_stride = v->stride[d];
            g_extent = v->shape[d];
            have = true;
            continue;
        }
        int64_t want;
        if (!mul_ok(g_stride, g_extent, &want)) return DG_ERR_OVERFLOW;
        if (v->stride[d] != want) return DG_ERR_UNSUPPORTED_VIEW;
        if (!mul_ok(g_extent, v->shape[d], &g_extent)) return DG_ERR_OVERFLOW;
    }
    m.rs = have ? g_stride : 0;
    m.cs = v->stride[nd - 1];
    m.ptr = static_cast<const char *>(v->ptr);
    m.align_ptr = pow2_align(reinterpret_cast<uintptr_t>(v->ptr));
    m.align_rs = m.rows > 1 ? pow2_align((uint64_t)m.rs) : 16;
    m.align_cs = m.cols > 1 ? pow2_align((uint64_t)m.cs) : 16;
    *out = m;
    return DG_SUCCESS;
}

bool self_overlaps(const Mat &m) {
    if (m.empty() || (m.rows <= 1 && m.cols <= 1)) return false;
    const int64_t es = m.esize;
    // Row-major-like: columns step by >= esize, rows step past a whole row.
    if (m.cols == 1 || m.cs >= es) {
        if (m.rows == 1) return false;
        if (m.rs >= (m.cols - 1) * m.cs + es) return false;
    }
    // Column-major-like: rows step by >= esize, columns step past a whole column.
    if (m.rows == 1 || m.rs >= es) {
        if (m.cols == 1) return false;
        if (m.cs >= (m.rows - 1) * m.rs + es) return false;
    }
    return true;
}

bool spans_overlap(const Mat &a, const Mat &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace dg
