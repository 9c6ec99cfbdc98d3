// Small-M GEMM of libbitq on the int8 matrix cores (TERNARY, W2A8, WNAM).
#include <hip/hip_runtime.h>

#include "bitq_device.h"

namespace bitq {

// ============================== small-M GEMM on the int8 matrix cores
// With M tokens the AND+popcount work grows M-fold and the VALU path becomes
// compute-bound from M = 2 on (measured: W2A8 11008x4096 takes 2.1 us more
// per token; from 4 tokens on this kernel is faster).  The same integer contraction then goes to
// v_mfma_i32_16x16x64_i8: D[16 rows][16 tokens] += A[16][64] B[64][16], with
// A = the weight codes unpacked from their bit planes to int8 and B = the
// int8 activations q ([ABQ] computes with the binary decomposition because
// its target has 1-bit tensor cores; gfx950 has int8 ones, so the planes are
// recombined into codes in registers instead).
//
// Operand layout of the instruction (checked on the device): lane l holds 16
// int8 of A for row l % 16 and 16 int8 of B for column l % 16; byte e of
// lanes with l / 16 = g meets byte e of B lanes with the same g (one k
// position); D element i of lane l is row 4 (l / 16) + i, column l % 16.
// The k position of (g, e) is chosen so that each lane reads one plane word
// per 128-input block: in k step s (0, 1) of block b, lane group g covers
// inputs 128 b + 32 g + 16 s + e, i.e. bits 16 s .. 16 s + 15 of plane word g
// of its row, and the matching 16 bytes of q are one 16-byte load.
//
// A workgroup of KW waves owns RS row sub-tiles of 16 rows and all
// M <= 16 TT tokens; wave w takes the k blocks [NB w / KW, NB (w + 1) / KW)
// for its RS x TT output tiles, so every lane loads distinct weight words and
// each q operand serves RS sub-tiles.  The wave's loads are issued CH blocks
// at a time, so one memory latency is paid per CH blocks: a wave's time is
// about (its blocks / CH) latencies, which is why the launcher prefers many
// short waves (RS 1, KW 8 or 16) and keeps q reuse (RS 4) for many tokens on
// tall layers.  Per 128-group (W2A8, WNAM) the fp32 output takes delta
// (A - z S128).  Except in the 64-row, 16-wave shape, the zero point is
// folded into the A operand (code - z as a signed byte, row by row), so the
// matrix cores return A - z S128 itself, exactly, and neither the group sums
// S nor the subtraction are needed (the same value, and the same fp32 bits,
// as delta (A - z S) computed from the exact A and S); the int32 output of
// BITQ_F_ACC_INT32 keeps the unshifted A.
// TERNARY keeps int32 sums over all of k.  The waves' partials are added in
// wave order through LDS.
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// Bits 4j .. 4j + 3 of v moved to bit 0 of bytes 0..3 (nibble times
// 1 + 2^7 + 2^14 + 2^21: the four copies do not overlap, so there are no
// carries, and bit e of copy e lands on bit 8e).
__device__ __forceinline__ uint32_t spread_nibble(uint32_t v, int j) {
    return (__builtin_amdgcn_ubfe(v, 4 * j, 4) * 0x204081u) & 0x01010101u;
}

// Four int8 codes (bytes) for inputs 4j .. 4j + 3 of a 16-bit slice
// starting at bit `lo` of the P plane words w[]: unsigned codes sum_p 2^p
// bit_p (W2A8, WNAM) or ternary T = plus - minus (bytes 0x01 / 0xFF).
template <int FMT, int P>
__device__ __forceinline__ uint32_t codes4(const uint32_t (&w)[P], int lo, int j) {
    if constexpr (FMT == BITQ_TERNARY) {
        const uint32_t pl = spread_nibble(w[0] >> lo, j), mi = spread_nibble(w[1] >> lo, j);
        return pl | ((mi << 8) - mi);
    } else {
        uint32_t c = spread_nibble(w[0] >> lo, j);
#pragma unroll
        for (int p = 1; p < P; ++p) c |= spread_nibble(w[p] >> lo, j) << p;
        return c;
    }
}

// Everything one wave reads for one 128-input block.
template <int P, int RS, int TT, bool GRP, bool FOLD>
struct MfmaBlock {
    uint32_t wp[RS][P];  // plane word g of rows 16 R + li
    v4i32_t qv[2][TT];   // q operands of the two k steps
    uint4 cz[GRP ? RS : 1];
    uint32_t zr[FOLD ? RS : 1];          // coefficient word of row 16 R + li (its zero point)
    int4 s4[GRP && !FOLD ? TT : 1];      // group sums (zero point not folded)
};

template <int FMT, int P, bool ACC, int TT, int RS, int KW, int CH>
__global__ __launch_bounds__(64 * KW) void gemm_mfma_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                            const uint8_t* __restrict__ act, size_t act_off_S,
                                                            size_t act_off_q, size_t act_off_d, int M, int N,
                                                            int Tb, float* __restrict__ y) {
    constexpr bool GRP = FMT != BITQ_TERNARY;  // per-128-group epilogue (W2A8, WNAM)
    constexpr bool LOADC = GRP && !ACC;        // coefficients needed
    // zero point folded into the codes; not in the 64-row, 16-wave shape
    // (8-16 tokens on tall layers), where the extra per-row coefficient
    // loads cost more than the saved epilogue (W2A8 11008x4096, M = 8:
    // 11.4 -> 11.9 us folded)
    constexpr bool FOLD = LOADC && !(RS == 4 && KW == 16);
    // waves 1..KW-1 hand their partials to wave 0: RS row sub-tiles x TT
    // token tiles x 4 values per lane
    constexpr int NV = RS * TT * 4;
    __shared__ float s_part[KW - 1][NV][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int t = blockIdx.x / (4 / RS);           // 64-row tile
    const int r0 = 16 * RS * (blockIdx.x % (4 / RS));  // first row of the group inside the tile
    const int NB = Tb, Kp = Tb * 128, Kw = Tb * 4;
    const int bbeg = (NB * wave) / KW, bend = (NB * (wave + 1)) / KW;
    const uint8_t* tile_planes = blob + kHeaderBytes + static_cast<size_t>(t) * Tb * P * 1024;
    const uint32_t* tile_coef = reinterpret_cast<const uint32_t*>(blob + off_c0) + static_cast<size_t>(t) * Tb * 64;
    const int8_t* q = reinterpret_cast<const int8_t*>(act + act_off_q);
    const int32_t* S = reinterpret_cast<const int32_t*>(act + act_off_S);
    const float* ad = reinterpret_cast<const float*>(act + act_off_d);
    int mrow[TT];  // this lane's token of each token tile (clamped for loads)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) mrow[tt] = min(16 * tt + li, M - 1);

    v4i32_t acc[RS][TT];
    float yacc[RS][TT][4];
#pragma unroll
    for (int R = 0; R < RS; ++R)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            acc[R][tt] = v4i32_t{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) yacc[R][tt][i] = 0.0f;
        }

    auto load = [&](MfmaBlock<P, RS, TT, GRP, FOLD>& L, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int R = 0; R < RS; ++R)
#pragma unroll
            for (int p = 0; p < P; ++p)
                L.wp[R][p] = *reinterpret_cast<const uint32_t*>(tile_planes + (b * P + p) * 1024 +
                                                                (r0 + 16 * R + li) * 16 + 4 * g);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                L.qv[s][tt] = *reinterpret_cast<const v4i32_t*>(q + static_cast<size_t>(mrow[tt]) * Kp + 128 * b +
                                                                32 * g + 16 * s);
        if constexpr (LOADC) {
#pragma unroll
            for (int R = 0; R < RS; ++R) {
                L.cz[R] = *reinterpret_cast<const uint4*>(tile_coef + b * 64 + r0 + 16 * R + 4 * g);
                if (FOLD) L.zr[R] = tile_coef[b * 64 + r0 + 16 * R + li];
            }
            if (!FOLD) {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    L.s4[tt] = *reinterpret_cast<const int4*>(S + static_cast<size_t>(mrow[tt]) * Kw + 4 * b);
            }
        }
    };

    auto compute = [&](const MfmaBlock<P, RS, TT, GRP, FOLD>& L, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int R = 0; R < RS; ++R) {
                v4i32_t a;
                if constexpr (FOLD) {
                    // codes minus the row's zero point, as signed bytes: (c | 0x80) - z
                    // cannot borrow (c, z < 16), and ^ 0x80 turns c - z + 128 into c - z
                    const uint32_t zb = static_cast<uint32_t>(f16_bits_to_f32(L.zr[R] >> 16)) * 0x01010101u;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        a[j] = static_cast<int>(((codes4<FMT, P>(L.wp[R], 16 * s, j) | 0x80808080u) - zb) ^ 0x80808080u);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[j] = static_cast<int>(codes4<FMT, P>(L.wp[R], 16 * s, j));
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[R][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, L.qv[s][tt], acc[R][tt], 0, 0, 0);
            }
        }
        if constexpr (GRP) {
            if constexpr (ACC) {  // exact group sums A[m][n][b]
#pragma unroll
                for (int R = 0; R < RS; ++R)
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int n = 64 * t + r0 + 16 * R + 4 * g + i, m = 16 * tt + li;
                            if (n < N && m < M)
                                reinterpret_cast<int32_t*>(y)[(static_cast<size_t>(m) * N + n) * NB + b] = acc[R][tt][i];
                        }
            } else {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const float S128 =
                        FOLD ? 0.0f : static_cast<float>((L.s4[tt].x + L.s4[tt].y) + (L.s4[tt].z + L.s4[tt].w));
#pragma unroll
                    for (int R = 0; R < RS; ++R) {
                        const uint32_t c[4] = {L.cz[R].x, L.cz[R].y, L.cz[R].z, L.cz[R].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float delta = f16_bits_to_f32(c[i]);
                            if (FOLD) {
                                yacc[R][tt][i] += delta * static_cast<float>(acc[R][tt][i]);  // acc = A - z S
                            } else {
                                const float z = f16_bits_to_f32(c[i] >> 16);
                                yacc[R][tt][i] += delta * (static_cast<float>(acc[R][tt][i]) - z * S128);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int R = 0; R < RS; ++R)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) acc[R][tt] = v4i32_t{0, 0, 0, 0};
        }
    };

    for (int c0 = bbeg; c0 < bend; c0 += CH) {
        // the chunk's loads are issued together (surplus slots re-read the
        // last block and are skipped below)
        MfmaBlock<P, RS, TT, GRP, FOLD> L[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) load(L[i], min(c0 + i, bend - 1));
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (c0 + i < bend) compute(L[i], c0 + i);
    }
    if constexpr (GRP && ACC) return;

    // ---- the waves' partials, added in wave order
    if (wave > 0) {
#pragma unroll
        for (int R = 0; R < RS; ++R)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = (R * TT + tt) * 4 + i;
                    s_part[wave - 1][v][lane] = GRP ? yacc[R][tt][i] : __int_as_float(acc[R][tt][i]);
                }
    }
    __syncthreads();
    if (wave != 0) return;
    const float gamma = (FMT == BITQ_TERNARY && !ACC) ? *reinterpret_cast<const float*>(blob + off_c0) : 1.0f;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int m = 16 * tt + li;
        const float scale = ACC ? 1.0f : (FMT == BITQ_TERNARY ? gamma * ad[mrow[tt]] : ad[mrow[tt]]);
#pragma unroll
        for (int R = 0; R < RS; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = (R * TT + tt) * 4 + i;
                const int n = 64 * t + r0 + 16 * R + 4 * g + i;
                if (GRP) {
                    float tot = yacc[R][tt][i];
#pragma unroll
                    for (int w = 0; w < KW - 1; ++w) tot += s_part[w][v][lane];
                    if (n < N && m < M) y[static_cast<size_t>(m) * N + n] = scale * tot;
                } else {
                    int tot = acc[R][tt][i];
#pragma unroll
                    for (int w = 0; w < KW - 1; ++w) tot += __float_as_int(s_part[w][v][lane]);
                    if (n < N && m < M) {
                        if (ACC)
                            reinterpret_cast<int32_t*>(y)[static_cast<size_t>(m) * N + n] = tot;
                        else
                            y[static_cast<size_t>(m) * N + n] = scale * static_cast<float>(tot);
                    }
                }
            }
    }
}

template <int FMT, int P, bool ACC>
static void launch_mfma(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M, float* y,
                        hipStream_t st) {
    ActLayout A = act_layout(M, d.K, d.rank);
    const auto* wb = static_cast<const uint8_t*>(w);
    const auto* ab = static_cast<const uint8_t*>(act);
    const int Tb = static_cast<int>(L.Tb);
    const MfmaShape sh = mfma_shape(d, M);
#define BITQ_MFMA(TT_, RS, KW, CH)                                                                             \
    hipLaunchKernelGGL((gemm_mfma_kernel<FMT, P, ACC, TT_, RS, KW, CH>), dim3(sh.grid), dim3(sh.block), 0, st, \
                       wb, L.off_c0, ab, A.off_S, A.off_q, A.off_d, M, d.N, Tb, y)
#define BITQ_MFMA_TT(TT_)                      \
    do {                                       \
        if (sh.RS == 4)                        \
            BITQ_MFMA(TT_, 4, 8, 2);           \
        else if (sh.KW == 16)                  \
            BITQ_MFMA(TT_, 1, 16, 2);          \
        else                                   \
            BITQ_MFMA(TT_, 1, 8, 2);           \
    } while (0)
    switch (sh.TT) {
        case 1:
            if (sh.RS == 4)
                BITQ_MFMA(1, 4, 16, 1);
            else
                BITQ_MFMA_TT(1);
            break;
        case 2: BITQ_MFMA_TT(2); break;
        case 3: BITQ_MFMA_TT(3); break;
        default: BITQ_MFMA_TT(4); break;
    }
#undef BITQ_MFMA_TT
#undef BITQ_MFMA
}

template <bool ACC>
static void launch_mfma_fmt(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M, float* y,
                            hipStream_t st) {
    switch (d.fmt) {
        case BITQ_TERNARY: launch_mfma<BITQ_TERNARY, 2, ACC>(d, L, w, act, M, y, st); break;
        case BITQ_W2A8: launch_mfma<BITQ_W2A8, 2, ACC>(d, L, w, act, M, y, st); break;
        default:
            switch (d.planes) {
                case 1: launch_mfma<BITQ_WNAM, 1, ACC>(d, L, w, act, M, y, st); break;
                case 2: launch_mfma<BITQ_WNAM, 2, ACC>(d, L, w, act, M, y, st); break;
                case 3: launch_mfma<BITQ_WNAM, 3, ACC>(d, L, w, act, M, y, st); break;
                default: launch_mfma<BITQ_WNAM, 4, ACC>(d, L, w, act, M, y, st); break;
            }
    }
}

int launch_gemm_mfma(const bitq_wdesc& d, const void* w, const void* act, int M, float* y, uint32_t flags,
                     void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (flags & BITQ_F_ACC_INT32)
        launch_mfma_fmt<true>(d, L, w, act, M, y, st);
    else
        launch_mfma_fmt<false>(d, L, w, act, M, y, st);
    return static_cast<int>(hipGetLastError());
}

}  // namespace bitq
