/*
 * dg_calib.h -- measured denominators for roofline fractions (measurement
 * support beside the GEMM library; nothing on the GEMM path calls these).
 *
 * A kernel's fraction of a published peak mixes two losses: what the kernel
 * leaves on the table, and what the part cannot sustain at its running clock.
 * These entry points measure the second on the current device, so that a
 * report can give both fractions: the achieved rate over the published peak,
 * and over the rate the hardware sustains under ideal code (a register-only
 * matrix-instruction loop, a device-wide streaming read, the floor of
 * back-to-back kernel launches).  This follows the modelling advice of
 * "DeepGEMM: GEMM micro-kernel modelling and generation methodology for
 * heterogeneous chips" (xdnf.cn), section 4.1: a hardware model takes its
 * bandwidth from measurement with a plain streaming kernel, since the sustained
 * rate falls well short of the data-sheet figure.
 *
 * All three enqueue work on `stream`, time it with two HIP events recorded on
 * that stream (created and destroyed per call), and synchronize the stream
 * before returning.  Outputs are host pointers.  The only device memory they
 * use is a 4 KB result sink per device, allocated on first use and kept.
 * Safe to call from several host threads; concurrent calls on one device
 * disturb each other's timings.
 */
#ifndef DG_CALIB_H
#define DG_CALIB_H

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense matrix-instruction rate in TFLOP/s: every CU runs 8 workgroups of 4
 * waves, each wave a chain of independent register-only matrix instructions
 * (16x16x32 BF16 for DG_BF16, 16x16x128 FP8 E4M3 with unit block scales for
 * DG_F8E4M3) for about 2 ms.
 * Errors: DG_ERR_NULL (tflops == NULL), DG_ERR_DTYPE (another dtype),
 * DG_ERR_ARCH (device is not gfx950), DG_ERR_HIP. */
dg_status dg_calib_mfma(dg_dtype dtype, double *tflops, hipStream_t stream);

/* Streaming read rate in GB/s (1e9 bytes/s) over the caller's device buffer
 * `buf` of `bytes` bytes (16-byte aligned; bytes a positive multiple of 16;
 * the contents are read, never written): 16-byte nontemporal loads by every
 * CU, averaged over 10 launches after one warm-up.  For a DRAM figure the
 * buffer should be well above the 256 MB last-level cache (2 GiB is typical).
 * Errors: DG_ERR_NULL (buf or gbs NULL), DG_ERR_MISALIGNED (buf or bytes not
 * 16-byte multiples, or bytes == 0), DG_ERR_ARCH, DG_ERR_HIP. */
dg_status dg_calib_read(const void *buf, size_t bytes, double *gbs, hipStream_t stream);

/* Average duration in microseconds of 2000 back-to-back launches of an empty
 * one-wave kernel on `stream` (the launch floor below which no single-launch
 * kernel can go).
 * Errors: DG_ERR_NULL (us == NULL), DG_ERR_ARCH, DG_ERR_HIP. */
dg_status dg_calib_launch(double *us, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_CALIB_H */
