// Internal declarations shared by the host side (bitq_host.cpp) and the HIP
// kernels (bitq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/bitq.h"

namespace bitq {

constexpr int kRowTile = 64;      // rows per tile = lanes per wave
constexpr int kKBlock = 128;      // inputs per k block = 4 words per row
constexpr int kHeaderBytes = 256;
constexpr uint32_t kMagic = 0x51544942u;
constexpr int kHdrHBound = 72;    // header: f32 [3] max_k |h_p[k]| (SIGN1: 1)
constexpr int kMaxFloatK = 63 * 8 * kKBlock;  // float formats: <= 63 splits of <= 8 k blocks
// HGF header fields: u64 off_c2, u32 rank, f32 alpha, f32 gate, f32 amax_a
constexpr int kHdrOffC2 = 88, kHdrRank = 96, kHdrAlpha = 100, kHdrGate = 104, kHdrAmaxA = 108;
constexpr int kMaxHgfK = 63 * 256;  // HGF: <= 63 runs of 256 inputs meet in one fixed-point word

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Byte layout of a packed blob (see include/bitq.h, "Packed blob layout").
struct BlobLayout {
    int64_t Np, Kp, P, Tn, Tb;
    size_t off_planes, planes_bytes;
    size_t off_c0, c0_bytes;
    size_t off_c1, c1_bytes;
    size_t off_c2, c2_bytes;  // HGF: B transposed (otherwise off_c2 = total, 0 bytes)
    size_t total;
};
BlobLayout blob_layout(const bitq_wdesc& d);

// Byte layout of an activation buffer (see bitq_quantize_act); rank > 0
// adds the HGF section h f32 [M][rank].
struct ActLayout {
    int64_t M, K, Kp, Kw;
    size_t off_planes, off_S, off_q, off_d, off_h, total;
};
ActLayout act_layout(int M, int K, int rank = 0);

// Byte layout of a binary activation buffer (see bitq_binarize_act).
struct BinActLayout {
    int64_t M, K, Kp, Kw;
    size_t off_beta, total;
};
BinActLayout binact_layout(int M, int K);

// How a GEMV/GEMM call is split over workgroups, and its workspace.
struct Plan {
    int waves_per_wg;      // 64-row waves per workgroup
    int rows_per_wg;       // 64 * waves_per_wg
    int row_groups;        // ceil(Np / rows_per_wg)
    int blocks_per_split;  // k blocks (128 inputs) per workgroup
    int splits;            // ceil((Kp/128) / blocks_per_split)
    int M;
    size_t off_partials;   // float formats: u64 [Np] split-k words (count + fixed-point sum)
    size_t ws_bytes;
    bool mfma;             // integer formats, M >= kMfmaMinM: the int8 matrix-core kernel
};
Plan make_plan(const bitq_wdesc& d, int M, bool fused = false);  // fused: BITQ_F_FUSE_QUANT
constexpr int kMfmaMinM = 4;  // tokens from which TERNARY/W2A8/WNAM use the matrix cores
constexpr int kMaxFusedK = 16384;    // BITQ_F_FUSE_QUANT: whole k range in one round of the kernel
constexpr int kLaunchNotBuilt = -1;  // launcher: no kernel built for this combination

// Kernel launchers (bitq_kernels.hip).  Arguments are already validated.
// Each returns hipSuccess or the HIP error code of the launch.
int launch_quantize_act(const void* x, int x_dtype, int M, int K, int abits, void* act, void* stream);
int launch_gemv_float(const bitq_wdesc& d, const Plan& plan, const void* w, const void* x,
                      int x_dtype, float* y, void* ws, void* stream);
int launch_gemv_int(const bitq_wdesc& d, const Plan& plan, const void* w, const void* act,
                    int M, float* y, void* ws, uint32_t flags, void* stream);
// Fused activation quantizer + GEMV, one token, raw x (bf16 or fp32); returns
// kLaunchNotBuilt when the plan has no such kernel.
int launch_gemv_fused(const bitq_wdesc& d, const Plan& plan, const void* w, const void* x, int x_dtype, float* y,
                      void* stream);
int launch_quantize_act_hgf(const void* x, int x_dtype, int M, int K, int rank, const void* w, const BlobLayout& L,
                            void* act, void* ws, void* stream);
int launch_binarize_act(const void* x, int x_dtype, int M, int K, void* act, void* stream);
int launch_gemv_xnor(const bitq_wdesc& d, const void* w, const void* act, int M, float* y, uint32_t flags,
                     void* stream);

// Device checks (bitq_kernels.hip): is the current device a gfx950?
int current_device_is_gfx950(int* is_gfx950);

}  // namespace bitq
