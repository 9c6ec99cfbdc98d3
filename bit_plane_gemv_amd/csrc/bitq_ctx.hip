// Measurement context kernels of libbitq (not part of the method).
//
// [HGF] §1.1 bounds decode speed by memory bandwidth: a layer cannot take
// less time than its weight bytes divided by the memory bandwidth.  On one
// GPU that bound has a second term, the cost of a launch, which dominates
// for layers of a few MB.  These kernels measure both terms on the device
// the GEMV runs on, so that a GEMV's time can be compared with what any
// single kernel can do over the same bytes:
//   ctx_empty_kernel   a launch of the same grid that does nothing
//   ctx_stream_kernel  a launch of the same grid that reads the same bytes
//                      once, coalesced, and writes one fp32 per output row
//                      (what a GEMV writes)
//   ctx_spin_kernel    one wave that waits a fixed wall-clock time: queued
//                      ahead of a timed region, it keeps the GPU busy while
//                      the host submits the work to be timed, so host
//                      submission does not appear in the measurement
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bitq_internal.h"

namespace bitq {

__global__ __launch_bounds__(256) void ctx_empty_kernel() {}

// Workgroup w owns the uint4 range [w per_wg, (w + 1) per_wg) of the source
// (the last one is shorter).  Lane l loads elements l, l + 256, ... of its
// range, U loads issued before any is used, and XORs them; lanes below
// rows_per_wg then write out[w rows_per_wg + l], so the kernel writes nout
// floats in all, as a GEMV of nout rows does.
template <int U>
__global__ __launch_bounds__(256) void ctx_stream_kernel(const uint4* __restrict__ src, int64_t n16, int64_t per_wg,
                                                         float* __restrict__ out, int nout, int rows_per_wg) {
    const int64_t beg = static_cast<int64_t>(blockIdx.x) * per_wg;
    const int64_t end = beg + per_wg < n16 ? beg + per_wg : n16;
    uint32_t acc = 0;
    for (int64_t i0 = beg + threadIdx.x; i0 < end; i0 += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + 256 * u;
            v[u] = i < end ? src[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
    }
    const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_wg + threadIdx.x;
    if (static_cast<int>(threadIdx.x) < rows_per_wg && row < nout) out[row] = __uint_as_float(acc & 0x3FFFFFFFu);
}

// Waits until `ticks` periods of the constant wall clock have passed since
// the wave started.  The clock only counts up, so every wave exits.
__global__ __launch_bounds__(64) void ctx_spin_kernel(uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

int launch_ctx_empty(int grid, void* stream) {
    hipLaunchKernelGGL(ctx_empty_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream));
    return static_cast<int>(hipGetLastError());
}

int launch_ctx_stream(const void* src, size_t bytes, int grid, float* out, int nout, void* stream) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t per_wg = (n16 + grid - 1) / grid;
    const int rows_per_wg = (nout + grid - 1) / grid;
    const int64_t loads = (per_wg + 255) / 256;  // uint4 per lane
    hipStream_t st = static_cast<hipStream_t>(stream);
    const auto* s = static_cast<const uint4*>(src);
    if (loads <= 1)
        hipLaunchKernelGGL(ctx_stream_kernel<1>, dim3(grid), dim3(256), 0, st, s, n16, per_wg, out, nout, rows_per_wg);
    else if (loads <= 2)
        hipLaunchKernelGGL(ctx_stream_kernel<2>, dim3(grid), dim3(256), 0, st, s, n16, per_wg, out, nout, rows_per_wg);
    else if (loads <= 4)
        hipLaunchKernelGGL(ctx_stream_kernel<4>, dim3(grid), dim3(256), 0, st, s, n16, per_wg, out, nout, rows_per_wg);
    else
        hipLaunchKernelGGL(ctx_stream_kernel<8>, dim3(grid), dim3(256), 0, st, s, n16, per_wg, out, nout, rows_per_wg);
    return static_cast<int>(hipGetLastError());
}

int launch_ctx_spin(int microseconds, void* stream) {
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (khz <= 0) khz = 100000;  // the 100 MHz constant clock of gfx9 parts
    const uint64_t ticks = static_cast<uint64_t>(microseconds) * static_cast<uint64_t>(khz) / 1000u;
    hipLaunchKernelGGL(ctx_spin_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks);
    return static_cast<int>(hipGetLastError());
}

}  // namespace bitq
