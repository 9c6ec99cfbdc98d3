// Internal declarations shared by the host side (bitq_host.cpp) and the HIP
// kernels (bitq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/bitq.h"
#include "../../include/bitq_ctx.h"

namespace bitq {

constexpr int kRowTile = 64;      // rows per tile = lanes per wave
constexpr int kKBlock = 128;      // inputs per k block = 4 words per row
constexpr int kHeaderBytes = 256;
constexpr uint32_t kMagic = 0x51544942u;
constexpr int kHdrHBound = 72;    // header: f32 [3] max_k |h_p[k]| (SIGN1: 1)
constexpr int kMaxFloatK = 63 * 8 * kKBlock;  // float formats: <= 63 splits of <= 8 k blocks
constexpr int kWholeRowGrid = 256;  // whole-row kernels: workgroups (one per CU of the MI355X)
// LDS a whole-row kernel's workgroup claims at least: more than half of a
// CU's 160 KB, so the 256 workgroups land on 256 distinct CUs
constexpr int kOneWgPerCuLds = 84 * 1024;
// HGF header fields: u64 off_c2, u32 rank, f32 alpha, f32 gate, f32 amax_a
constexpr int kHdrOffC2 = 88, kHdrRank = 96, kHdrAlpha = 100, kHdrGate = 104, kHdrAmaxA = 108;
constexpr int kMaxHgfK = 63 * 256;  // HGF: <= 63 runs of 256 inputs meet in one fixed-point word

// BVSR4 planes: nibble e (0..7) of a plane word holds the bitvector bits of
// input (e >> 1) + 4 (e & 1) of the word's 8 inputs (the order in which two
// words of 4 activation bytes split into nibble words most cheaply)
constexpr int bvsr_nibble_input(int e) { return (e >> 1) + 4 * (e & 1); }

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
    size_t off_planes, off_S, off_q, off_qm, off_d, off_amax, off_h, total;
};
// Rows longer than this get their amax from a separate pass (act_amax_kernel)
// instead of every workgroup of the quantizer reading the whole row.
constexpr int kAmaxOnePassK = 16384;
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
    bool mfma;             // TERNARY/W2A8/WNAM, M >= mfma_min_tokens: the int8 matrix-core kernel
};
Plan make_plan(const bitq_wdesc& d, int M, bool fused = false);  // fused: BITQ_F_FUSE_QUANT
// The fused-quantizer GEMV with 16 rows per workgroup, and the BVSR4 GEMV
// of one token with 16 rows, take 8 waves (32 k-groups) instead of 4 when
// the k range has more than this many 128-input blocks: then 4 waves would
// leave 4 or more blocks per lane.  Measured: fused W2A8 4096x11008 6.96 ->
// 6.57 us, fused BVSR 28672x8192 27.95 -> 27.58 us, BVSR 28672x8192
// 26.33 -> 25.75 us; slower with 4096 inputs (fused W2A8 11008x4096 5.67 ->
// 5.95 us, fused ternary 4096x4096 3.65 -> 3.92 us) and for the other
// formats' two-launch GEMVs (W2A8 4096x11008 5.02 -> 5.43 us).
constexpr int kWideMinBlocks = 48;

// Launch shape of the matrix-core kernel for M tokens: TT token tiles of 16,
// RS = kMfmaSubs (or 1, when the sub-tiles do not outnumber the workgroups)
// sub-tiles of 16 rows per pass of a workgroup, KW waves over
// k, CH k blocks whose loads a wave issues together; grid = one workgroup
// per CU (at most one per sub-tile), of 64 KW lanes.
constexpr int kMfmaSubs = 3;
struct MfmaShape {
    int TT, RS, KW, CH;
    int grid, block;
};
MfmaShape mfma_shape(const bitq_wdesc& d, int M);

// Workgroups and lanes per workgroup of the kernel a bitq_gemv /
// bitq_gemm_smallM call launches (x_dtype and flags as in that call).
struct LaunchShape {
    int grid, block;
};
LaunchShape launch_shape(const bitq_wdesc& d, int M, int x_dtype, uint32_t flags);
// Workgroups of the AND+popcount / XNOR kernels: 64/RG row groups per 64-row
// tile, tiles dealt round-robin to the 8 XCDs (padded to whole rounds).
inline int xcd_row_groups(int64_t tiles, int RG) { return static_cast<int>(8 * (64 / RG) * ((tiles + 7) / 8)); }
// Tokens from which TERNARY, W2A8 and WNAM run on the int8 matrix cores
// (measured on W2A8 11008x4096: 6.2 us at 2 and 3 tokens against 7.0 and
// 9.0 us on the VALU; ternary 4096x4096: 4.8 us at 2 and 3 tokens against
// 4.1 and 5.0 us).  0 for the formats that stay on the VALU.
inline int mfma_min_tokens(int fmt) {
    if (fmt == BITQ_W2A8 || fmt == BITQ_WNAM) return 2;
    if (fmt == BITQ_TERNARY) return 3;
    return 0;
}
constexpr int kMaxFusedK = 16384;    // BITQ_F_FUSE_QUANT: whole k range in one round of the kernel
constexpr int kLaunchNotBuilt = -1;  // launcher: no kernel built for this combination

// Kernel launchers (bitq_act.hip, bitq_sign.hip, bitq_bits.hip, bitq_mfma.hip,
// bitq_xnor.hip).  Arguments are already validated.
// Each returns hipSuccess or the HIP error code of the launch.
int launch_quantize_act(const void* x, int x_dtype, int M, int K, int abits, void* act, void* stream);
int launch_gemv_float(const bitq_wdesc& d, const Plan& plan, const void* w, const void* x,
                      int x_dtype, float* y, void* ws, void* stream);
// Small-M GEMM on the int8 matrix cores (plans with mfma set).
int launch_gemm_mfma(const bitq_wdesc& d, const void* w, const void* act, int M, float* y, uint32_t flags,
                     void* stream);
int launch_gemv_int(const bitq_wdesc& d, const Plan& plan, const void* w, const void* act,
                    int M, float* y, void* ws, uint32_t flags, void* stream);
// Fused activation quantizer + GEMV, one token, raw x (bf16 or fp32); returns
// kLaunchNotBuilt when the plan has no such kernel.
int launch_gemv_fused(const bitq_wdesc& d, const Plan& plan, const void* w, const void* x, int x_dtype, float* y,
                      void* stream);
int launch_quantize_act_hgf(const void* x, int x_dtype, int M, int K, int rank, const void* w, const BlobLayout& L,
                            void* act, void* ws, void* stream);
// The HGF activation step with its workspace in the library's static device
// scratch (bitq_quantize_act_hgf_noalloc): at most kNoAllocScratchWords
// 64-bit words (M * rank), allocates nothing.
constexpr int kNoAllocScratchWords = 64 * 64;
int launch_quantize_act_hgf_noalloc(const void* x, int x_dtype, int M, int K, int rank, const void* w,
                                    const BlobLayout& L, void* act, void* stream);
int launch_binarize_act(const void* x, int x_dtype, int M, int K, void* act, void* stream);
int launch_gemv_xnor(const bitq_wdesc& d, const void* w, const void* act, int M, float* y, uint32_t flags,
                     void* stream);

// Measurement context kernels (bitq_ctx.hip); arguments already validated.
int launch_ctx_empty(int grid, void* stream);
int launch_ctx_stream(const void* src, size_t bytes, int grid, float* out, int nout, void* stream);
int launch_ctx_spin(int microseconds, void* stream);

// Device check (bitq_act.hip): is the current device a gfx950?
int current_device_is_gfx950(int* is_gfx950);

}  // namespace bitq
