// Sign-apply GEMV of libbitq for float activations (SIGN1, RABIT).
#include <hip/hip_runtime.h>

#include "bitq_device.h"

namespace bitq {

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

// Byte offset 4*nibble of the nibble held in bits 2..5 of byte B of w: one
// SDWA instruction (byte select + AND with the inline constant 60).
#define BITQ_NIB_ADDR(NAME, B)                                                                     \
    __device__ __forceinline__ uint32_t NAME(uint32_t w) {                                          \
        uint32_t r;                                                                                \
        asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "        \
            "src1_sel:BYTE_" #B                                                                    \
            : "=v"(r)                                                                              \
            : "v"(w));                                                                             \
        return r;                                                                                  \
    }
BITQ_NIB_ADDR(nib_addr0, 0)
BITQ_NIB_ADDR(nib_addr1, 1)
BITQ_NIB_ADDR(nib_addr2, 2)
BITQ_NIB_ADDR(nib_addr3, 3)
#undef BITQ_NIB_ADDR

__device__ __forceinline__ uint32_t nib_addr(uint32_t w, int byte) {
    switch (byte) {
        case 0: return nib_addr0(w);
        case 1: return nib_addr1(w);
        case 2: return nib_addr2(w);
        default: return nib_addr3(w);
    }
}

// Split-k hand-off of the float GEMV: one 64-bit device-scope atomic add per
// row and split.  Each split turns its partial p into the fixed-point integer
// v = rint(p 2^S) (S per row, below) and adds (1 << 58) + v to the row's
// word, so the top bits count arrivals and the rest hold the exact integer
// sum.  Integer addition is exact and associative, so the total does not
// depend on the order in which splits arrive (deterministic output).  The
// add returns the previous word: the split that sees splits - 1 arrivals in
// it is the last, already holds the whole sum, writes y and resets the word.
// S comes from a bound every split of the row computes identically:
//   |y_n| <= B_n = sum_p |g_p[n]| max_k |h_p[k]| sum_k |x_k|
// (max |h_p| is stored in the blob header), with 2^52 >= B_n 2^S, so
// |v| and every partial sum stay below 2^53 (the count field starts at bit
// 58; at most 63 splits) and the rounding error is at most splits/2 units of 2^-S, i.e. a
// relative 2^-52 of B_n per split.  A non-finite bound (inf/NaN in x, g or h)
// makes the row NaN.
__device__ __forceinline__ void split_k_add(unsigned long long* word, float part, float bound, int splits,
                                            float* y_n) {
    const bool finite = bound <= 3.402823466e38f;  // false for inf and NaN
    int e = 0;
    if (finite && bound > 0.0f) (void)frexpf(bound, &e);  // bound < 2^e
    const int S = 52 - e;
    const long long v = finite ? static_cast<long long>(rint(ldexp(static_cast<double>(part), S))) : 0;
    const unsigned long long add = (1ull << 58) + static_cast<unsigned long long>(v);
    const unsigned long long prev = __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // prev = c 2^58 + V (mod 2^64) with |V| < 2^57: c = (prev + 2^57) >> 58
    const unsigned long long arrived = (prev + (1ull << 57)) >> 58;
    if (arrived != static_cast<unsigned long long>(splits - 1)) return;
    const long long total = static_cast<long long>(prev + add - (static_cast<unsigned long long>(splits) << 58));
    *y_n = finite ? static_cast<float>(ldexp(static_cast<double>(total), -S)) : __builtin_nanf("");
    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT>
__device__ __forceinline__ float abs_sum8(uint4 v) {  // |.| summed over 8 bf16 or 4 f32 inputs
    if (DT == BITQ_DT_F32)
        return (fabsf(__uint_as_float(v.x)) + fabsf(__uint_as_float(v.y))) +
               (fabsf(__uint_as_float(v.z)) + fabsf(__uint_as_float(v.w)));
    float s = 0.0f;
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) s += fabsf(__uint_as_float(u[i] << 16)) + fabsf(__uint_as_float(u[i] & 0xFFFF0000u));
    return s;
}

template <int P, int KB, bool RABIT, int DT, int XPT>
__global__ __launch_bounds__(256) void gemv_sign_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                        size_t off_c1, const void* __restrict__ x, int N, int K,
                                                        int Np, int Tn, int Tb, int splits, float* __restrict__ y,
                                                        unsigned long long* __restrict__ ws_acc) {
    constexpr int CH = KB * 32;            // 4-input chunks in the k slice
    constexpr int NT = CH * P;             // tables in the k slice
    // SPLIT (2 or 4) threads share a table when 256 is a multiple of the
    // table count (each writes 4 / SPLIT of its 4 float4); otherwise TPT
    // tables per thread.  Surplus threads rebuild (parts of) the last table.
    constexpr int SPLIT = (NT < 256 && 256 % NT == 0) ? (256 / NT < 4 ? 256 / NT : 4) : 1;
    constexpr int TPT = (NT * SPLIT + 255) / 256;  // tables per thread
    // XPT: uint4 of x per thread for sum |x| (more: a loop), sized to K by
    // the launcher: clamped duplicate loads cost memory-pipeline slots and
    // registers (8 instead of 2 at K = 4096 measured 0.5 us slower)
    __shared__ float4 lut4[NT * 4];        // [chunk][plane][16 floats]
    __shared__ float s_xsum[4];
    const int split = blockIdx.y;
    const int k0 = split * KB * kKBlock;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    const int n = t * kRowTile + lane;
    const uint16_t* hbits = reinterpret_cast<const uint16_t*>(blob + off_c1);

    // ---- 1. activations and column scales of this thread's tables (small,
    //         shared by all workgroups: L2 hits), issued first so that the
    //         tables are built while the weight stream is still arriving.
    //         K is a multiple of 32: a chunk of 4 inputs is entirely in or out.
    uint2 xraw[TPT][2], hraw[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int tbl = min(static_cast<int>(threadIdx.x) / SPLIT + 256 * i, NT - 1);
        const int c = tbl / P, p = tbl % P;
        const int k = min(k0 + 4 * c, K - 4);  // clamped; chunks past K get zero tables below
        if (DT == BITQ_DT_F32) {
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const float*>(x) + k);
            xraw[i][0] = make_uint2(v.x, v.y);
            xraw[i][1] = make_uint2(v.z, v.w);
        } else {
            xraw[i][0] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + k);
        }
        if (RABIT) hraw[i] = *reinterpret_cast<const uint2*>(hbits + static_cast<size_t>(p) * (Tb * kKBlock) + k);
    }

    __builtin_amdgcn_sched_barrier(0);  // issue order: table inputs, weights, all of x

    // ---- 2. all of x, for the bound of the split-k hand-off (the same
    //         fixed-order sum in every workgroup), ahead of the weights
    const int n16 = (DT == BITQ_DT_F32 ? K / 4 : K / 8);  // uint4 of x
    // (through an address without the kernel argument's restrict/invariant
    // provenance: these loads are not moved across the memory clobber below)
    uintptr_t xaddr = reinterpret_cast<uintptr_t>(x);
    asm volatile("" : "+s"(xaddr));
    uint4 xall[XPT];  // unconditional: a conditional block of loads would make
                      // the compiler count the outstanding loads from its
                      // shorter path and wait too early for the others
#pragma unroll
    for (int i = 0; i < XPT; ++i) xall[i] = global_load16(xaddr, min(static_cast<int>(threadIdx.x) + 256 * i, n16 - 1));
    asm volatile("" ::: "memory");  // keeps these loads here, ahead of the weights

    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. weight words and row scales (raw bits, converted at the end).
    //         Loads are unconditional (no branch, so nothing waits on them
    //         early): a wave beyond the last row tile re-reads the last tile
    //         and stores nothing; a block beyond K re-reads the last block,
    //         whose chunks here have all-zero tables, so it adds nothing.
    const int tl = min(t, Tn - 1);
    const int nl = tl * kRowTile + lane;
    uint4 wv[KB][P];
    uint32_t graw[P];
#pragma unroll
    for (int bb = 0; bb < KB; ++bb) {
        const int b = min(split * KB + bb, Tb - 1);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const size_t off = (static_cast<size_t>(tl) * Tb + b) * P + p;
            wv[bb][p] = *reinterpret_cast<const uint4*>(blob + kHeaderBytes + off * 1024 + lane * 16);
        }
    }
    if (RABIT) {
        const uint16_t* g = reinterpret_cast<const uint16_t*>(blob + off_c0);
#pragma unroll
        for (int p = 0; p < P; ++p) graw[p] = g[static_cast<size_t>(p) * Np + nl];
    } else {
        graw[0] = reinterpret_cast<const uint32_t*>(blob + off_c0)[nl];  // alpha, fp32 bits
    }

    __builtin_amdgcn_sched_barrier(0);

    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. tables: x~ = h x, then the 16 signed sums of each chunk
    // No branch on the table index: a guarded build would let the compiler
    // move the input loads into it, behind the weight stream.  Lanes past the
    // last table rebuild that table and store the same values again.
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int tbl = min(static_cast<int>(threadIdx.x) / SPLIT + 256 * i, NT - 1);
        {
            const int c = tbl / P;
            float xv[4], hv[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if (DT == BITQ_DT_F32) {
                xv[0] = __uint_as_float(xraw[i][0].x); xv[1] = __uint_as_float(xraw[i][0].y);
                xv[2] = __uint_as_float(xraw[i][1].x); xv[3] = __uint_as_float(xraw[i][1].y);
            } else {
                xv[0] = __uint_as_float(xraw[i][0].x << 16); xv[1] = __uint_as_float(xraw[i][0].x & 0xFFFF0000u);
                xv[2] = __uint_as_float(xraw[i][0].y << 16); xv[3] = __uint_as_float(xraw[i][0].y & 0xFFFF0000u);
            }
            if (RABIT) {
                hv[0] = f16_bits_to_f32(hraw[i].x); hv[1] = f16_bits_to_f32(hraw[i].x >> 16);
                hv[2] = f16_bits_to_f32(hraw[i].y); hv[3] = f16_bits_to_f32(hraw[i].y >> 16);
            }
            const bool in = k0 + 4 * c < K;
            const float a = in ? xv[0] * hv[0] : 0.0f, bq = in ? xv[1] * hv[1] : 0.0f;
            const float cc = in ? xv[2] * hv[2] : 0.0f, dd = in ? xv[3] * hv[3] : 0.0f;
            const float lo[4] = {-a - bq, a - bq, -a + bq, a + bq};
            const float hi[4] = {-cc - dd, cc - dd, -cc + dd, cc + dd};
            float4* dst = &lut4[tbl * 4];
            const int q0 = (static_cast<int>(threadIdx.x) % SPLIT) * (4 / SPLIT);
#pragma unroll
            for (int qq = 0; qq < 4 / SPLIT; ++qq) {
                const int q4 = q0 + qq;
                dst[q4] = make_float4(lo[0] + hi[q4], lo[1] + hi[q4], lo[2] + hi[q4], lo[3] + hi[q4]);
            }
        }
    }
    {  // sum |x|: this thread's inputs (clamped duplicates masked to zero
       // bits, no branch), the wave's, then the workgroup's after the barrier
        float xs = 0.0f;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const uint32_t keep = static_cast<int>(threadIdx.x) + 256 * i < n16 ? 0xFFFFFFFFu : 0u;
            xs += abs_sum8<DT>(make_uint4(xall[i].x & keep, xall[i].y & keep, xall[i].z & keep, xall[i].w & keep));
        }
        for (int i = threadIdx.x + 256 * XPT; i < n16; i += 256) xs += abs_sum8<DT>(global_load16(xaddr, i));  // K > 16384 (bf16)
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) xs += __shfl_xor(xs, o, 64);
        if (lane == 0) s_xsum[wave] = xs;
    }
    __syncthreads();

    // ---- 5. table lookups: one row per lane
    float part = 0.0f;
    {
        const uint8_t* lut_bytes = reinterpret_cast<const uint8_t*>(lut4);
        float acc[P], acc2[P];  // even and odd nibbles: two add chains per path
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = acc2[p] = 0.0f;
#pragma unroll
        for (int bb = 0; bb < KB; ++bb)
#pragma unroll
            for (int p = 0; p < P; ++p) {
                // the empty asm keeps every use of this block's words (and the
                // wait for them) after the barrier, in block order
                uint32_t words[4] = {wv[bb][p].x, wv[bb][p].y, wv[bb][p].z, wv[bb][p].w};
                asm volatile("" : "+v"(words[0]), "+v"(words[1]), "+v"(words[2]), "+v"(words[3]));
                // the block's 32 table reads first, then the adds (same order
                // as reading and adding in turn): the compiler then keeps
                // more reads in flight per wait than it does when each read
                // feeds its add at once (6.24 -> 6.10 us at 11008x4096)
                float tv[32];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t w4 = words[w] << 2;   // nibble 2j in bits 2..5 of byte j
                    const uint32_t w2 = words[w] >> 2;   // nibble 2j+1 in bits 2..5 of byte j
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = bb * 32 + w * 8 + 2 * j;
                        const uint32_t a0 = nib_addr(w4, j);
                        const uint32_t a1 = nib_addr(w2, j);
                        tv[w * 8 + 2 * j] = *reinterpret_cast<const float*>(lut_bytes + a0 + ((c * P + p) * 64));
                        tv[w * 8 + 2 * j + 1] =
                            *reinterpret_cast<const float*>(lut_bytes + a1 + (((c + 1) * P + p) * 64));
                    }
                }
#pragma unroll
                for (int i = 0; i < 32; i += 2) {
                    acc[p] += tv[i];
                    acc2[p] += tv[i + 1];
                }
            }
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] += acc2[p];
        if (RABIT) {
#pragma unroll
            for (int p = 0; p < P; ++p) part += f16_bits_to_f32(graw[p]) * acc[p];
        } else {
            part = __uint_as_float(graw[0]) * acc[0];
        }
    }
    if (splits == 1) {
        if (t < Tn && n < N) y[n] = part;
        return;
    }
    if (t < Tn && n < N) {
        const float xsum = (s_xsum[0] + s_xsum[1]) + (s_xsum[2] + s_xsum[3]);
        const float* hbound = reinterpret_cast<const float*>(blob + kHdrHBound);
        float gh = 0.0f;
        if (RABIT) {
#pragma unroll
            for (int p = 0; p < P; ++p) gh += fabsf(f16_bits_to_f32(graw[p])) * hbound[p];
        } else {
            gh = fabsf(__uint_as_float(graw[0]));
        }
        split_k_add(&ws_acc[n], part, gh * xsum, splits, &y[n]);
    }
}

template <int P, int KB, bool RABIT, int DT, int XPT>
static void launch_sign_x(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                          float* y, void* ws, hipStream_t st) {
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    hipLaunchKernelGGL((gemv_sign_kernel<P, KB, RABIT, DT, XPT>), dim3(pl.row_groups, pl.splits), dim3(256), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, L.off_c1, x, d.N, d.K, static_cast<int>(L.Np),
                       static_cast<int>(L.Tn), static_cast<int>(L.Tb), pl.splits, y,
                       reinterpret_cast<unsigned long long*>(wsb + pl.off_partials));
}

template <int P, int KB, bool RABIT, int DT>
static void launch_sign(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                        float* y, void* ws, hipStream_t st) {
    // uint4 loads of x per thread for the split-k bound: all of x in one go
    // up to 8 per thread (16384 bf16 / 8192 fp32 inputs), the rest in a loop
    const int n16 = DT == BITQ_DT_F32 ? d.K / 4 : d.K / 8;
    if (n16 <= 256)
        launch_sign_x<P, KB, RABIT, DT, 1>(d, pl, L, w, x, y, ws, st);
    else if (n16 <= 512)
        launch_sign_x<P, KB, RABIT, DT, 2>(d, pl, L, w, x, y, ws, st);
    else if (n16 <= 1024)
        launch_sign_x<P, KB, RABIT, DT, 4>(d, pl, L, w, x, y, ws, st);
    else if (n16 <= 1536)
        launch_sign_x<P, KB, RABIT, DT, 6>(d, pl, L, w, x, y, ws, st);
    else
        launch_sign_x<P, KB, RABIT, DT, 8>(d, pl, L, w, x, y, ws, st);
}

template <int P, bool RABIT, int DT>
static void launch_sign_kb(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w,
                           const void* x, float* y, void* ws, hipStream_t st) {
    switch (pl.blocks_per_split) {
        case 1: launch_sign<P, 1, RABIT, DT>(d, pl, L, w, x, y, ws, st); break;
        case 2: launch_sign<P, 2, RABIT, DT>(d, pl, L, w, x, y, ws, st); break;
        case 4: launch_sign<P, 4, RABIT, DT>(d, pl, L, w, x, y, ws, st); break;
        default: launch_sign<P, 8, RABIT, DT>(d, pl, L, w, x, y, ws, st); break;
    }
}

template <int DT>
static void launch_sign_fmt(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w,
                            const void* x, float* y, void* ws, hipStream_t st) {
    if (d.fmt == BITQ_SIGN1) {
        launch_sign_kb<1, false, DT>(d, pl, L, w, x, y, ws, st);
        return;
    }
    switch (d.planes) {
        case 1: launch_sign_kb<1, true, DT>(d, pl, L, w, x, y, ws, st); break;
        case 2: launch_sign_kb<2, true, DT>(d, pl, L, w, x, y, ws, st); break;
        default: launch_sign_kb<3, true, DT>(d, pl, L, w, x, y, ws, st); break;
    }
}

int launch_gemv_float(const bitq_wdesc& d, const Plan& pl, const void* w, const void* x, int x_dtype, float* y,
                      void* ws, void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == BITQ_DT_F32)
        launch_sign_fmt<BITQ_DT_F32>(d, pl, L, w, x, y, ws, st);
    else
        launch_sign_fmt<BITQ_DT_BF16>(d, pl, L, w, x, y, ws, st);
    return static_cast<int>(hipGetLastError());
}

}  // namespace bitq
