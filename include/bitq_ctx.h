/*
 * bitq_ctx.h -- measurement context kernels exported by libbitq.
 *
 * These calls are not part of the method.  They exist so that a bit-plane
 * GEMV's time can be set against what any single kernel can do on the same
 * GPU over the same bytes.  [HGF] §1.1 ("1.58位LLM混合门控流优化技术解析",
 * the memory-wall argument) bounds decode time below by weight bytes divided
 * by memory bandwidth; on one GPU a launch adds a fixed cost on top of that
 * bound, and for layers of a few MB the fixed cost is the larger term.
 *
 * Conventions are those of bitq.h: the caller owns every buffer, the library
 * allocates nothing, arguments are checked before anything is enqueued (a
 * negative bitq_status and bitq_last_error() on error), launches are
 * asynchronous on the given stream (a hipStream_t as void*, NULL = the null
 * stream) and never synchronize.  A non-gfx950 device gives
 * BITQ_E_UNSUPPORTED, a launch failure BITQ_E_DEVICE.
 */
#ifndef BITQ_CTX_H
#define BITQ_CTX_H

#include <stddef.h>
#include <stdint.h>

#include "bitq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A kernel of `grid` workgroups of 256 lanes that does nothing: the cost of
 * one launch of that grid (dispatch, wave start, completion).
 * 1 <= grid <= 2^20.
 */
bitq_status bitq_ctx_empty(int32_t grid, void* stream);

/*
 * A kernel of `grid` workgroups of 256 lanes that reads `bytes` bytes of
 * src_dev once and writes nout floats to out_dev, and does no other work.
 * Workgroup w reads the w-th of `grid` equal contiguous slices of the source
 * with 16-byte loads (lane l takes elements l, l + 256, ... of the slice,
 * up to eight loads issued before any is used) and writes rows
 * [w R, (w + 1) R) of the output, R = ceil(nout / grid).  The values written
 * are meaningless; out_dev exists so that the kernel ends with the same
 * stores as a GEMV with nout outputs.
 *   src_dev  device, 16-byte aligned; bytes a positive multiple of 16
 *   out_dev  device fp32 [nout], 4-byte aligned; 0 <= nout <= 2^24
 *            (out_dev may be NULL when nout = 0)
 *   1 <= grid <= 2^20
 */
bitq_status bitq_ctx_stream(const void* src_dev, size_t bytes, int32_t grid, float* out_dev, int32_t nout,
                            void* stream);

/*
 * One wave that waits `microseconds` of wall-clock time on the device's
 * constant clock, then exits.  Enqueued ahead of a timed region, it keeps
 * the GPU busy while the host submits the work that follows, so that host
 * submission is not part of the measured GPU time.  1 <= microseconds <=
 * 10000.
 */
bitq_status bitq_ctx_spin(int32_t microseconds, void* stream);

/*
 * Launch shape of the product kernel: the number of workgroups (*grid) and
 * lanes per workgroup (*block) of the kernel that bitq_gemv (M = 1) or
 * bitq_gemm_smallM (M >= 2) launches for these arguments (x_dtype and flags
 * as in that call; BITQ_DT_BINARY selects the XNOR kernel).  For context
 * kernels over the same grid.  Host only.
 */
bitq_status bitq_ctx_launch_shape(const bitq_wdesc* desc, int32_t M, int32_t x_dtype, uint32_t flags,
                                  int32_t* grid, int32_t* block);

#ifdef __cplusplus
}
#endif

#endif /* BITQ_CTX_H */
