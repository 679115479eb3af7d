/*
 * oracle.c -- plain, slow, obviously correct FP64 reference for the dense GEMM
 *
 *     C = alpha * A * B + beta * C
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The GPU product path never
 * calls it, links it or includes anything from this directory, and this file
 * includes nothing from the product (its own view type, its own dtype codes,
 * its own decoders).
 *
 * What it follows (the pages are cited by title and section):
 *  - Definition C[M,N] = A[M,K] x B[K,N], op() folded into strides:
 *      "DeepGEMM deep dive: from GEMM fundamentals to Tensor Core performance"
 *      (sheratonhq.com), section 1.1;
 *      "DeepGEMM: GEMM micro-kernel modelling and generation methodology for
 *      heterogeneous chips" (xdnf.cn), section 3.1 (C = alpha*A*B + beta*C);
 *      DeepGEMM view-native GEMM article (kwkr.cn), sections 2.3 and 4.1.
 *  - Addressing: element address = base + sum_d i_d * stride_d, strides in
 *      BYTES (kwkr.cn article, sections 2.3 and 3.2).  This file walks every
 *      view itself, dimension by dimension, without merging dimensions.
 *  - Reference = naive triple loop, k ascending (sheratonhq.com, section 4.2).
 *  - FP8: the operand is the dequantized value (code * scale) with each scale
 *      applied exactly once (sheratonhq.com, sections 2.4 and 4.2); scale
 *      blocks are 128 wide along K for A (per token) and 128 x 128 for B.
 *  - alpha = 0 still applies beta * C (kwkr.cn, section 4.3); beta = 0 does not
 *      read C; K = 0 gives beta * C (BLAS convention; the pages are silent).
 *
 * Decoders are written from the format definitions: IEEE binary16, bfloat16
 * (upper half of binary32), binary32, and OCP FP8 E4M3FN (bias 7, 3 mantissa
 * bits, subnormals m * 2^-9, no infinities, S.1111.111 = NaN, max 448).
 *
 * Every product a*b is exact in FP64 for these inputs; sums are rounded in
 * FP64 in ascending k.  Built with -ffp-contract=off so no FMA contraction
 * changes the rounding of the naive loop.  The same pass accumulates
 * S = sum_k |a*b|, which the comparator uses to scale the tolerance.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle's own dtype codes. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_E4M3 = 3 };

/* Oracle's own view: base points at element (0,..,0) inside a host copy of the
 * operand's whole storage; strides are in bytes. */
typedef struct {
    const unsigned char *base;
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
    int32_t dtype;
} or_view;

static int elem_size(int dt) {
    switch (dt) {
    case OR_F32: return 4;
    case OR_F16: case OR_BF16: return 2;
    case OR_E4M3: return 1;
    default: return 0;
    }
}

/* ---- decoders (from the format definitions) ---- */

static double dec_f16(uint32_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)       v = ldexp((double)m, -24);             /* subnormal / zero */
    else if (e == 31) v = m ? NAN : INFINITY;
    else              v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) 2^(e-15) */
    return s ? -v : v;
}

static double dec_f32(uint32_t u) {
    int s = (u >> 31) & 1, e = (u >> 23) & 0xff;
    uint32_t m = u & 0x7fffff;
    double v;
    if (e == 0)        v = ldexp((double)m, -149);
    else if (e == 255) v = m ? NAN : INFINITY;
    else               v = ldexp((double)(0x800000u + m), e - 150);
    return s ? -v : v;
}

static double dec_bf16(uint32_t b) { return dec_f32(b << 16); }

static double dec_e4m3(uint32_t q) {
    int s = (q >> 7) & 1, e = (q >> 3) & 0xf, m = q & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;                 /* only NaN encoding; no Inf */
    else if (e == 0)       v = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
    else                   v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

double or_decode(int32_t dtype, uint32_t bits) {
    switch (dtype) {
    case OR_F32: return dec_f32(bits);
    case OR_F16: return dec_f16(bits & 0xffff);
    case OR_BF16: return dec_bf16(bits & 0xffff);
    case OR_E4M3: return dec_e4m3(bits & 0xff);
    default: return NAN;
    }
}

static double load_elem(const or_view *v, const unsigned char *p) {
    uint32_t bits = 0;
    switch (v->dtype) {
    case OR_F32: memcpy(&bits, p, 4); return dec_f32(bits);
    case OR_F16: { uint16_t h; memcpy(&h, p, 2); return dec_f16(h); }
    case OR_BF16: { uint16_t h; memcpy(&h, p, 2); return dec_bf16(h); }
    case OR_E4M3: return dec_e4m3(p[0]);
    }
    return NAN;
}

/* ---- the view walk ---- */

/* Logical matrix of a view: rows = product of dims 0..ndim-2 (row-major
 * flattening), cols = dim ndim-1.  A 1-D view is one row. */
static int64_t v_rows(const or_view *v) {
    int64_t r = 1;
    for (int d = 0; d + 1 < v->ndim; ++d) r *= v->shape[d];
    return r;
}
static int64_t v_cols(const or_view *v) { return v->shape[v->ndim - 1]; }

/* Byte offset of logical row r: decompose r over dims 0..ndim-2 (last of them
 * fastest) and add index * stride for each. */
static int64_t v_row_off(const or_view *v, int64_t r) {
    int64_t off = 0;
    for (int d = v->ndim - 2; d >= 0; --d) {
        int64_t n = v->shape[d];
        off += (r % n) * v->stride[d];
        r /= n;
    }
    return off;
}

static double v_at(const or_view *v, int64_t r, int64_t c) {
    return load_elem(v, v->base + v_row_off(v, r) + c * v->stride[v->ndim - 1]);
}

static int v_ok(const or_view *v) {
    if (!v || v->ndim < 1 || v->ndim > 4 || elem_size(v->dtype) == 0) return 0;
    for (int d = 0; d < v->ndim; ++d)
        if (v->shape[d] < 0) return 0;
    return 1;
}

/*
 * or_gemm -- reference GEMM over the rows listed in `rows` (or all rows).
 *
 *   A: M x K view, B: K x N view, Cin: M x N view (read only if beta != 0).
 *   As, Bs: NULL for FP16/BF16 inputs; for FP8, FP32 scale views of shape
 *           [M, ceil(K/128)] and [ceil(K/128), ceil(N/128)].
 *   alpha, beta: the exact FP32 values the GPU receives, widened to double.
 *   rows: indices into 0..M-1 (NULL = 0..M-1), nrows entries.
 *   out  [nrows x N]: C_ref;   sabs [nrows x N]: sum_k |a*b| (may be NULL);
 *   cin  [nrows x N]: decoded C_in when beta != 0, else zeros (may be NULL).
 *   nthreads <= 0: OpenMP default.
 * Returns 0, or a negative code for an inconsistent call.
 */
int or_gemm(const or_view *A, const or_view *As, const or_view *B, const or_view *Bs,
            const or_view *Cin, double alpha, double beta, const int64_t *rows, int64_t nrows,
            double *out, double *sabs, double *cin, int32_t nthreads) {
    if (!v_ok(A) || !v_ok(B) || !out) return -1;
    const int64_t M = v_rows(A), K = v_cols(A), N = v_cols(B);
    if (v_rows(B) != K) return -2;
    const int fp8 = (As != NULL);
    if (fp8 != (Bs != NULL)) return -3;
    const int64_t KB = (K + 127) / 128, NB = (N + 127) / 128;
    if (fp8) {
        if (!v_ok(As) || !v_ok(Bs)) return -4;
        if (v_rows(As) != M || v_cols(As) != KB || v_rows(Bs) != KB || v_cols(Bs) != NB) return -5;
    }
    if (beta != 0.0) {
        if (!v_ok(Cin) || v_rows(Cin) != M || v_cols(Cin) != N) return -6;
    }
    if (!rows) nrows = M;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return -7;

    /* Dequantized B, decoded once: b(k,n) = dec(qB[k,n]) * dec(sB[k/128, n/128]). */
    double *Bd = NULL;
    if (alpha != 0.0 && K > 0 && N > 0) {
        Bd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
        if (!Bd) return -8;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = 0; n < N; ++n) {
                double b = v_at(B, k, n);
                if (fp8) b *= v_at(Bs, k / 128, n / 128);
                Bd[k * N + n] = b;
            }
    }

    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double *P = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *S = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t m = rows ? rows[i] : i;
            for (int64_t n = 0; n < N; ++n) { P[n] = 0.0; S[n] = 0.0; }
            if (Bd) {
                /* a(m,k) = dec(qA[m,k]) * dec(sA[m, k/128]) */
                for (int64_t k = 0; k < K; ++k) {
                    double a = v_at(A, m, k);
                    if (fp8) a *= v_at(As, m, k / 128);
                    arow[k] = a;
                }
                /* P(m,n) = sum over ascending k of a(m,k) * b(k,n) */
                for (int64_t k = 0; k < K; ++k) {
                    const double a = arow[k];
                    const double *brow = Bd + k * N;
                    for (int64_t n = 0; n < N; ++n) {
                        const double t = a * brow[n];
                        P[n] += t;
                        S[n] += fabs(t);
                    }
                }
            }
            double *o = out + i * N;
            for (int64_t n = 0; n < N; ++n) {
                const double T = (alpha == 0.0) ? 0.0 : alpha * P[n];
                double c = 0.0;
                if (beta != 0.0) c = v_at(Cin, m, n);
                o[n] = (beta == 0.0) ? T : T + beta * c;
                if (sabs) sabs[i * N + n] = S[n];
                if (cin) cin[i * N + n] = c;
            }
        }
        free(arow); free(P); free(S);
    }
    free(Bd);
    return 0;
}

/* Plain gather of a view into a row-major FP64 matrix (rows x cols), used by the
 * tests to check the view walk against torch's own strided indexing. */
int or_gather(const or_view *V, double *out) {
    if (!v_ok(V) || !out) return -1;
    const int64_t R = v_rows(V), Cc = v_cols(V);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < Cc; ++c) out[r * Cc + c] = v_at(V, r, c);
    return 0;
}

int or_num_threads(void) { return omp_get_max_threads(); }
