// HIP kernels of libbitq for gfx950 (MI355X): the per-token activation
// quantizer, the sign-apply GEMV for float activations (SIGN1/RABIT) and the
// AND+popcount GEMV for integer activations (TERNARY/W2A8/BVSR4).
//
// Sources are cited by the short names defined in include/bitq.h:
// [RaBiT], [HGF], [ABQ], [BVSR], [BitNet].
//
// Work decomposition shared by the GEMV kernels: lane l of a wave owns output
// row n = 64 t + l of row tile t and reads that row's packed words with one
// 16-byte load per plane and k block (the 64 lanes read 1 KB contiguously,
// see the blob layout in bitq.h).  A workgroup covers `waves` row tiles and a
// slice of `blocks_per_split` k blocks; the grid is (row groups, splits).
// When the k range is split, each workgroup stores its partial outputs in the
// workspace and the last workgroup of a row group to arrive (arrival counter,
// device-scope fences) adds the partials in split order and writes y, so the
// result does not depend on scheduling.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "bitq_internal.h"

namespace bitq {

// --------------------------------------------------------------- utilities
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float load_act(const void* x, int dt, size_t i) {
    if (dt == BITQ_DT_F32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h & 0xFFFFu)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Uniform value in a scalar register (all lanes hold the same value).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------- split-k reduction helper
// Called by every thread of the workgroup after it computed `part` (the
// partial output of row n, split s, token m).  Returns true in the workgroup
// that must finish the row group (the last to arrive); that workgroup then
// reads the partials back from the workspace.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int splits, int* s_flag) {
    __threadfence();  // make this workgroup's partial stores visible device-wide
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t prev = atomicAdd(counter, 1u);
        int last = (prev == static_cast<uint32_t>(splits - 1));
        if (last) *counter = 0u;  // reset for the next call on this workspace
        *s_flag = last;
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    if (last) __threadfence();  // acquire: see the other workgroups' partials
    return last;
}

// ======================================================= activation quantizer
// One workgroup (256 threads) per token.  [HGF] §1.2: int8 activations with a
// per-token absmax scale, dequantized with amax/127; [BVSR] intro: online
// conversion of activations to the bit format.  Arithmetic order fixed for
// bit-exactness: s = fl32(127/amax) correctly rounded, q = rint(fl32(x*s)).
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ x, int dt, int K, int Kw,
                                                        uint32_t* __restrict__ planes, int32_t* __restrict__ S,
                                                        int8_t* __restrict__ q, float* __restrict__ dq) {
    __shared__ float s_red[4];
    const int m = blockIdx.x;
    const size_t xrow = static_cast<size_t>(m) * K;
    float amax = 0.0f;
    for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(load_act(x, dt, xrow + k)));
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    float s = 0.0f, d = 0.0f;
    if (amax > 0.0f) {
        s = __fdiv_rn(127.0f, amax);
        d = __fdiv_rn(amax, 127.0f);
    }
    for (int w = threadIdx.x; w < Kw; w += 256) {
        uint32_t pl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t qb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int k = 32 * w + i;
            int qi = 0;
            if (k < K && amax > 0.0f) {
                float v = __fmul_rn(load_act(x, dt, xrow + k), s);
                v = fminf(fmaxf(rintf(v), -127.0f), 127.0f);
                qi = static_cast<int>(v);
            }
            sum += qi;
            const uint32_t byte = static_cast<uint32_t>(qi) & 0xFFu;
#pragma unroll
            for (int j = 0; j < 8; ++j) pl[j] |= ((byte >> j) & 1u) << i;
            qb[i >> 2] |= byte << (8 * (i & 3));
        }
        uint4* pdst = reinterpret_cast<uint4*>(planes + (static_cast<size_t>(m) * Kw + w) * 8);
        pdst[0] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        pdst[1] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
        S[static_cast<size_t>(m) * Kw + w] = sum;
        uint4* qdst = reinterpret_cast<uint4*>(q + (static_cast<size_t>(m) * Kw + w) * 32);
        qdst[0] = make_uint4(qb[0], qb[1], qb[2], qb[3]);
        qdst[1] = make_uint4(qb[4], qb[5], qb[6], qb[7]);
    }
    if (threadIdx.x == 0) dq[m] = d;
}

// ========================================================= sign-apply GEMV
// [RaBiT] §3.2 replaces the matrix multiply by applying the weight signs to
// the activations.  Here the signs of 4 consecutive inputs form a nibble that
// indexes a 16-entry table of all +-x~ sums of those inputs, built once per
// workgroup in LDS for its k slice and shared by its 256 rows:
//   T_c[j] = sum_{i<4} (bit i of j ? +x~_{4c+i} : -x~_{4c+i}),  x~ = h_p (.) x
// so acc_p[n] = sum_c T_c[nibble_c(B_p[n])] = sum_k B_p[n,k] x~_k exactly as
// the sign-apply sum, with one table read and one add per 4 weights.
// Every lane of a wave reads the same table (one k position), so the 16
// entries are broadcast without bank conflicts.
template <int P, int KB>
__global__ __launch_bounds__(256) void gemv_sign_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                        size_t off_c1, const void* __restrict__ x, int dt,
                                                        int fmt, int N, int K, int Np, int Tn, int Tb, int splits,
                                                        float* __restrict__ y, float* __restrict__ ws_part,
                                                        uint32_t* __restrict__ ws_cnt) {
    constexpr int CH = KB * 32;        // 4-input chunks in the k slice
    __shared__ float4 lut4[CH * P * 4];  // [chunk][plane][16 floats]
    __shared__ int s_flag;
    const int split = blockIdx.y;
    const int k0 = split * KB * kKBlock;

    // ---- build the tables for this k slice
    const uint16_t* hbits = reinterpret_cast<const uint16_t*>(blob + off_c1);
    for (int tbl = threadIdx.x; tbl < CH * P; tbl += 256) {
        const int c = tbl / P, p = tbl % P;
        float xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 4 * c + i;
            float v = 0.0f;
            if (k < K) {
                v = load_act(x, dt, k);
                if (fmt == BITQ_RABIT) v = v * f16_bits_to_f32(hbits[static_cast<size_t>(p) * (Tb * kKBlock) + k]);
            }
            xv[i] = v;
        }
        const float a = xv[0], b = xv[1], cc = xv[2], dd = xv[3];
        const float lo[4] = {-a - b, a - b, -a + b, a + b};
        const float hi[4] = {-cc - dd, cc - dd, -cc + dd, cc + dd};
        float4* dst = &lut4[tbl * 4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            dst[q4] = make_float4(lo[0] + hi[q4], lo[1] + hi[q4], lo[2] + hi[q4], lo[3] + hi[q4]);
    }
    __syncthreads();

    // ---- main loop: one row per lane
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    const int n = t * kRowTile + lane;
    float part = 0.0f;
    if (t < Tn) {
        const uint8_t* lut_bytes = reinterpret_cast<const uint8_t*>(lut4);
        uint4 wv[KB][P];
#pragma unroll
        for (int bb = 0; bb < KB; ++bb) {
            const int b = split * KB + bb;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                if (b < Tb) {
                    const size_t off = (static_cast<size_t>(t) * Tb + b) * P + p;
                    wv[bb][p] = *reinterpret_cast<const uint4*>(blob + kHeaderBytes + off * 1024 + lane * 16);
                } else {
                    wv[bb][p] = make_uint4(0, 0, 0, 0);
                }
            }
        }
        float acc[P];
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = 0.0f;
#pragma unroll
        for (int bb = 0; bb < KB; ++bb)
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const uint32_t words[4] = {wv[bb][p].x, wv[bb][p].y, wv[bb][p].z, wv[bb][p].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t w4 = words[w] << 2;   // nibble 2j at byte j, scaled by 4
                    const uint32_t w2 = words[w] >> 2;   // nibble 2j+1 at byte j, scaled by 4
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = bb * 32 + w * 8 + 2 * j;
                        const uint32_t a0 = (w4 >> (8 * j)) & 0x3Cu;
                        const uint32_t a1 = (w2 >> (8 * j)) & 0x3Cu;
                        acc[p] += *reinterpret_cast<const float*>(lut_bytes + a0 + ((c * P + p) * 64));
                        acc[p] += *reinterpret_cast<const float*>(lut_bytes + a1 + (((c + 1) * P + p) * 64));
                    }
                }
            }
        if (fmt == BITQ_RABIT) {
            const uint16_t* g = reinterpret_cast<const uint16_t*>(blob + off_c0);
#pragma unroll
            for (int p = 0; p < P; ++p) part += f16_bits_to_f32(g[static_cast<size_t>(p) * Np + n]) * acc[p];
        } else {
            part = reinterpret_cast<const float*>(blob + off_c0)[n] * acc[0];
        }
    }
    if (splits == 1) {
        if (t < Tn && n < N) y[n] = part;
        return;
    }
    if (t < Tn) ws_part[static_cast<size_t>(split) * Np + n] = part;
    if (arrive_last(&ws_cnt[blockIdx.x], splits, &s_flag) && t < Tn && n < N) {
        float s = 0.0f;
        for (int sp = 0; sp < splits; ++sp) s += ws_part[static_cast<size_t>(sp) * Np + n];
        y[n] = s;
    }
}

// ====================================================== AND+popcount GEMV
// Integer activations q (int8, two's-complement planes X_j with weights
// c_j = 2^j, c_7 = -128) against binary weight planes W_i:
//   sum_k qw_k q_k = sum_i sum_j u_i c_j popcount(W_i AND X_j)
// ([ABQ] abstract and §1: arbitrary-bit products rebuilt from binary
// operations instead of INT4/INT8 units; [BVSR] intro: AND and population
// count directly on the bitvectors, without dequantization).  The activation
// plane words are the same for all 64 rows of a wave, so they are read with
// scalar loads and enter the AND as scalar operands; each weight word costs
// one AND and one popcount-accumulate (v_bcnt_u32_b32) per activation plane.
//
// Per-token epilogues (y before the per-token factor d, applied at the end):
//   TERNARY ([HGF] §1.2): Y = sum_j c_j (popc(P & X_j) - popc(M & X_j)),
//           y = gamma d Y
//   W2A8 ([ABQ] Eq. 3): per 128-group A = sum_j c_j (a0_j + 2 a1_j),
//           y += delta (A - z S128)
//   BVSR4 ([BVSR]): per 32-group P_k = sum_j c_j popc(beta_k & X_j),
//           y += b S32 + sum_k c_k P_k with (c, b) = cache[idx]
template <int FMT>
struct IntCfg;
template <>
struct IntCfg<BITQ_TERNARY> { static constexpr int P = 2; };
template <>
struct IntCfg<BITQ_W2A8> { static constexpr int P = 2; };
template <>
struct IntCfg<BITQ_BVSR4> { static constexpr int P = 4; };

// Horner combination of per-plane popcounts: sum_j c_j a_j.
__device__ __forceinline__ int combine_planes(const int (&a)[8]) {
    int r = -a[7];
#pragma unroll
    for (int j = 6; j >= 0; --j) r = 2 * r + a[j];
    return r;
}

template <int FMT, bool ACC>
__global__ __launch_bounds__(64) void gemv_bits_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                       size_t off_c1, const uint8_t* __restrict__ act,
                                                       size_t act_off_S, size_t act_off_d, int M, int N,
                                                       int K, int Np, int Tn, int Tb, int KB, int splits,
                                                       float* __restrict__ y, float* __restrict__ ws_part,
                                                       uint32_t* __restrict__ ws_cnt) {
    constexpr int P = IntCfg<FMT>::P;
    __shared__ float4 s_cache[FMT == BITQ_BVSR4 ? 256 * 2 : 1];
    __shared__ int s_flag;
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const int n = t * kRowTile + lane;
    const int split = blockIdx.y;
    const int b0 = split * KB;
    const int b1 = min(Tb, b0 + KB);
    const int Kw = Tb * 4;
    const uint32_t* __restrict__ aplanes = reinterpret_cast<const uint32_t*>(act);
    const int32_t* __restrict__ aS = reinterpret_cast<const int32_t*>(act + act_off_S);
    const float* __restrict__ ad = reinterpret_cast<const float*>(act + act_off_d);

    if (FMT == BITQ_BVSR4) {
        const float* cache = reinterpret_cast<const float*>(blob + off_c1);
        for (int e = lane; e < 256; e += 64) {
            const float* c = cache + 5 * e;
            s_cache[2 * e] = make_float4(c[0], c[1], c[2], c[3]);
            s_cache[2 * e + 1] = make_float4(c[4], 0.0f, 0.0f, 0.0f);
        }
        __syncthreads();
    }

    for (int m = 0; m < M; ++m) {
        const uint32_t* __restrict__ xp = aplanes + static_cast<size_t>(m) * Kw * 8;
        const int32_t* __restrict__ xS = aS + static_cast<size_t>(m) * Kw;
        float yacc = 0.0f;
        int tacc[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) tacc[i][j] = 0;

        for (int b = b0; b < b1; ++b) {
            const int bu = uniform(b);
            uint4 wv[P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const size_t off = (static_cast<size_t>(t) * Tb + bu) * P + p;
                wv[p] = *reinterpret_cast<const uint4*>(blob + kHeaderBytes + off * 1024 + lane * 16);
            }
            uint32_t coef = 0;
            if (FMT == BITQ_W2A8 || FMT == BITQ_BVSR4)
                coef = reinterpret_cast<const uint32_t*>(blob + off_c0)[(static_cast<size_t>(t) * Tb + bu) * 64 + lane];

            if (FMT == BITQ_TERNARY) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t* xw = xp + static_cast<size_t>(bu * 4 + w) * 8;
                    const uint32_t wp = (&wv[0].x)[w], wm = (&wv[1].x)[w];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t xj = xw[j];
                        tacc[0][j] += __builtin_popcount(wp & xj);
                        tacc[1][j] += __builtin_popcount(wm & xj);
                    }
                }
            } else if (FMT == BITQ_W2A8) {
                int a[2][8];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) a[i][j] = 0;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t* xw = xp + static_cast<size_t>(bu * 4 + w) * 8;
                    const uint32_t w0 = (&wv[0].x)[w], w1 = (&wv[1].x)[w];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t xj = xw[j];
                        a[0][j] += __builtin_popcount(w0 & xj);
                        a[1][j] += __builtin_popcount(w1 & xj);
                    }
                }
                int t8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t8[j] = a[0][j] + 2 * a[1][j];
                const int A = combine_planes(t8);
                if (ACC) {
                    const size_t G = Tb;  // K is a multiple of 128 for W2A8
                    if (n < N) reinterpret_cast<int32_t*>(y)[(static_cast<size_t>(m) * N + n) * G + bu] = A;
                } else {
                    const int S128 = xS[bu * 4] + xS[bu * 4 + 1] + xS[bu * 4 + 2] + xS[bu * 4 + 3];
                    const float delta = f16_bits_to_f32(coef);
                    const float z = f16_bits_to_f32(coef >> 16);
                    yacc += delta * (static_cast<float>(A) - z * static_cast<float>(S128));
                }
            } else {  // BVSR4
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t* xw = xp + static_cast<size_t>(bu * 4 + w) * 8;
                    int a[4][8];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t bk = (&wv[k].x)[w];
#pragma unroll
                        for (int j = 0; j < 8; ++j) a[k][j] = __builtin_popcount(bk & xw[j]);
                    }
                    int Pk[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) Pk[k] = combine_planes(a[k]);
                    if (ACC) {
                        const int G = K / 32;  // groups of the real (unpadded) K
                        const int g = bu * 4 + w;
                        int4* dst = reinterpret_cast<int4*>(y) + (static_cast<size_t>(m) * N + n) * G + g;
                        if (n < N && g < G) *dst = make_int4(Pk[0], Pk[1], Pk[2], Pk[3]);
                    } else {
                        const int id = (coef >> (8 * w)) & 0xFF;
                        const float4 c = s_cache[2 * id];
                        const float bb = s_cache[2 * id + 1].x;
                        const float S32 = static_cast<float>(xS[bu * 4 + w]);
                        yacc += bb * S32 + c.x * static_cast<float>(Pk[0]) + c.y * static_cast<float>(Pk[1]) +
                                c.z * static_cast<float>(Pk[2]) + c.w * static_cast<float>(Pk[3]);
                    }
                }
            }
        }

        // ---- per-token result of this split
        float part = 0.0f;
        int ipart = 0;
        if (FMT == BITQ_TERNARY) {
            int Y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) Y[j] = tacc[0][j] - tacc[1][j];
            ipart = combine_planes(Y);
            const float gamma = *reinterpret_cast<const float*>(blob + off_c0);
            part = gamma * ad[m] * static_cast<float>(ipart);
        } else {
            part = ad[m] * yacc;
        }
        if (ACC && FMT != BITQ_TERNARY) continue;  // partials already written per group

        const bool int_out = ACC;  // TERNARY with ACC: reduce the exact integer Y
        if (splits == 1) {
            if (n < N) {
                if (int_out)
                    reinterpret_cast<int32_t*>(y)[static_cast<size_t>(m) * N + n] = ipart;
                else
                    y[static_cast<size_t>(m) * N + n] = part;
            }
            continue;
        }
        float* slot = ws_part + (static_cast<size_t>(split) * M + m) * Np + n;
        if (int_out)
            *reinterpret_cast<int32_t*>(slot) = ipart;
        else
            *slot = part;
        if (m == M - 1) {
            // all tokens of this split are stored: arrive once
            if (arrive_last(&ws_cnt[t], splits, &s_flag) && n < N) {
                for (int mm = 0; mm < M; ++mm) {
                    if (int_out) {
                        int s = 0;
                        for (int sp = 0; sp < splits; ++sp)
                            s += reinterpret_cast<const int32_t*>(ws_part)[(static_cast<size_t>(sp) * M + mm) * Np + n];
                        reinterpret_cast<int32_t*>(y)[static_cast<size_t>(mm) * N + n] = s;
                    } else {
                        float s = 0.0f;
                        for (int sp = 0; sp < splits; ++sp) s += ws_part[(static_cast<size_t>(sp) * M + mm) * Np + n];
                        y[static_cast<size_t>(mm) * N + n] = s;
                    }
                }
            }
        }
    }
}

// =============================================================== launchers
namespace {
std::atomic<int> g_arch_cache[64];
}

int current_device_is_gfx950(int* is_gfx950) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev >= 0 && dev < 64) {
        int c = g_arch_cache[dev].load();
        if (c) {
            *is_gfx950 = (c == 1);
            return 0;
        }
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const bool yes = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) g_arch_cache[dev].store(yes ? 1 : 2);
    *is_gfx950 = yes;
    return 0;
}

int launch_quantize_act(const void* x, int x_dtype, int M, int K, void* act, void* stream) {
    ActLayout A = act_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    hipLaunchKernelGGL(quant_act_kernel, dim3(M), dim3(256), 0, static_cast<hipStream_t>(stream), x, x_dtype, K,
                       static_cast<int>(A.Kw), reinterpret_cast<uint32_t*>(base + A.off_planes),
                       reinterpret_cast<int32_t*>(base + A.off_S), reinterpret_cast<int8_t*>(base + A.off_q),
                       reinterpret_cast<float*>(base + A.off_d));
    return static_cast<int>(hipGetLastError());
}

template <int P, int KB>
static void launch_sign(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                        int dt, float* y, void* ws, hipStream_t st) {
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    hipLaunchKernelGGL((gemv_sign_kernel<P, KB>), dim3(pl.row_groups, pl.splits), dim3(256), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, L.off_c1, x, dt, d.fmt, d.N, d.K,
                       static_cast<int>(L.Np), static_cast<int>(L.Tn), static_cast<int>(L.Tb), pl.splits, y,
                       reinterpret_cast<float*>(wsb + pl.off_partials),
                       reinterpret_cast<uint32_t*>(wsb + pl.off_counters));
}

template <int P>
static void launch_sign_kb(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w,
                           const void* x, int dt, float* y, void* ws, hipStream_t st) {
    switch (pl.blocks_per_split) {
        case 1: launch_sign<P, 1>(d, pl, L, w, x, dt, y, ws, st); break;
        case 2: launch_sign<P, 2>(d, pl, L, w, x, dt, y, ws, st); break;
        default: launch_sign<P, 4>(d, pl, L, w, x, dt, y, ws, st); break;
    }
}

int launch_gemv_float(const bitq_wdesc& d, const Plan& pl, const void* w, const void* x, int x_dtype, float* y,
                      void* ws, void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (d.planes) {
        case 1: launch_sign_kb<1>(d, pl, L, w, x, x_dtype, y, ws, st); break;
        case 2: launch_sign_kb<2>(d, pl, L, w, x, x_dtype, y, ws, st); break;
        default: launch_sign_kb<3>(d, pl, L, w, x, x_dtype, y, ws, st); break;
    }
    return static_cast<int>(hipGetLastError());
}

template <int FMT, bool ACC>
static void launch_bits(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* act,
                        int M, float* y, void* ws, hipStream_t st) {
    ActLayout A = act_layout(M, d.K);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    hipLaunchKernelGGL((gemv_bits_kernel<FMT, ACC>), dim3(pl.row_groups, pl.splits), dim3(64), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, L.off_c1, static_cast<const uint8_t*>(act),
                       A.off_S, A.off_d, M, d.N, d.K, static_cast<int>(L.Np), static_cast<int>(L.Tn),
                       static_cast<int>(L.Tb), pl.blocks_per_split, pl.splits, y,
                       reinterpret_cast<float*>(wsb + pl.off_partials),
                       reinterpret_cast<uint32_t*>(wsb + pl.off_counters));
}

int launch_gemv_int(const bitq_wdesc& d, const Plan& pl, const void* w, const void* act, int M, float* y,
                    void* ws, uint32_t flags, void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool acc = (flags & BITQ_F_ACC_INT32) != 0;
    switch (d.fmt) {
        case BITQ_TERNARY:
            acc ? launch_bits<BITQ_TERNARY, true>(d, pl, L, w, act, M, y, ws, st)
                : launch_bits<BITQ_TERNARY, false>(d, pl, L, w, act, M, y, ws, st);
            break;
        case BITQ_W2A8:
            acc ? launch_bits<BITQ_W2A8, true>(d, pl, L, w, act, M, y, ws, st)
                : launch_bits<BITQ_W2A8, false>(d, pl, L, w, act, M, y, ws, st);
            break;
        default:
            acc ? launch_bits<BITQ_BVSR4, true>(d, pl, L, w, act, M, y, ws, st)
                : launch_bits<BITQ_BVSR4, false>(d, pl, L, w, act, M, y, ws, st);
            break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace bitq
