// HIP kernels of libbitq for gfx950 (MI355X):
//   quant_act_kernel      per-token int8 / m-bit activation quantizer (and,
//                         for HGF layers, the correction's down projection)
//   gemv_sign_kernel      sign-apply GEMV for float activations (SIGN1, RABIT)
//   gemv_bits_nr_kernel   AND+popcount GEMV for integer activations (TERNARY,
//                         W2A8, BVSR4, WNAM, HGF), M = 1 and the VALU small-M path
//   gemm_mfma_kernel      small-M GEMM on the int8 matrix cores (TERNARY,
//                         W2A8, WNAM; M >= 4)
//   binarize_act_kernel, gemv_xnor_kernel   the fully binary XNOR path
//
// Sources are cited by the short names defined in include/bitq.h:
// [RaBiT], [HGF], [ABQ], [BVSR], [BitNet].
//
// Weights come in the packed blob layout of bitq.h: 64-row tiles in which
// each row owns 16 contiguous bytes per plane and 128-input block, so 64
// lanes reading one row each load 1 KB contiguously.  Each kernel's own
// comment gives its work decomposition.  Results never depend on workgroup
// scheduling: integer partial sums are exact, float partials are added in a
// fixed order or, across workgroups, as 64-bit fixed-point integers.

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

// 16-byte load of element i of a global array given by its address as an
// integer (so the load carries no restrict/invariant provenance and stays in
// program order around memory clobbers), as a global (not flat) access.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 global_load16(uintptr_t base, int i) {
    const u32x4_t v = ((const __attribute__((address_space(1))) u32x4_t*)base)[i];
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ======================================================= activation quantizer
// [HGF] §1.2: int8 activations with a per-token absmax scale, dequantized
// with amax/127; [BVSR] intro: online conversion of activations to the bit
// format.  Arithmetic order fixed for bit-exactness: s = fl32(127/amax)
// correctly rounded, q = clamp(rint(fl32(x*s)), -127, 127), d = fl32(amax/127).
// m-bit activations ([ABQ] §1) use Qm = 2^(m-1) - 1 in place of 127.
//
// Grid (words / 8, M): each workgroup (4 waves) owns 8 consecutive 32-input
// words of one token.  It first reduces amax over the token's whole row (the
// row is small and L2-resident, so every workgroup recomputing it is cheaper
// than a second launch; the same single pass parks the workgroup's own 256
// inputs in LDS), then each lane quantizes one input and each of the
// 8 planes of the wave's 64 inputs comes out of one ballot: bit i of the
// ballot of (q >> j) & 1 is plane j of input i.
//
// RANK > 0 (HGF layers) adds the correction path's down projection
// ([HGF] §2.1) h = silu(x A) over the same unquantized inputs: thread
// (c, j) = (tid / RANK, tid % RANK) sums x_k A[k][j] in fp32 over the run
// k = lo + RANK c + i, i < RANK (row j of A^T, RANK/8 16-byte loads issued
// together), the 256/RANK runs of a column are added in order through LDS,
// and the workgroups of a token meet in one 64-bit fixed-point word per
// column (lora_arrive below); the workgroup that completes a column applies
// silu and writes h.
template <int DT>
__device__ __forceinline__ float act_at(const void* x, size_t i) {
    if (DT == BITQ_DT_F32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// Exact cross-workgroup sum of the down projection: each of the `arrivals`
// workgroups of a token adds (1 << 58) + rint(part 2^S) to the column's word
// (the count in the top 6 bits, the fixed-point sum below, as in the float
// GEMV's split-k hand-off).  S = 52 - e with the bound K amax_x amax_a < 2^e,
// which bounds every partial sum of the column's terms, so the sum never
// reaches the count field.  The last arrival turns the total back into z,
// writes silu(z) = z / (1 + exp(-z)) and resets the word.
__device__ __forceinline__ void lora_arrive(unsigned long long* word, float part, double bound, int arrivals,
                                            float* h) {
    int e = 0;
    if (bound > 0.0) (void)frexp(bound, &e);  // bound < 2^e
    const int S = 52 - e;
    const long long v = static_cast<long long>(rint(ldexp(static_cast<double>(part), S)));
    const unsigned long long add = (1ull << 58) + static_cast<unsigned long long>(v);
    const unsigned long long prev = __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long arrived = (prev + (1ull << 57)) >> 58;
    if (arrived != static_cast<unsigned long long>(arrivals - 1)) return;
    const long long total = static_cast<long long>(prev + add - (static_cast<unsigned long long>(arrivals) << 58));
    const float z = static_cast<float>(ldexp(static_cast<double>(total), -S));
    *h = z / (1.0f + expf(-z));
    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int RANK>
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ x, int K, int Kw, float qmax,
                                                        uint32_t* __restrict__ planes, int32_t* __restrict__ S,
                                                        int8_t* __restrict__ q, float* __restrict__ dq,
                                                        const uint8_t* __restrict__ blob, size_t off_at, int Kp,
                                                        unsigned long long* __restrict__ ws,
                                                        float* __restrict__ hout) {
    constexpr int VEC = (DT == BITQ_DT_F32) ? 4 : 8;  // inputs per 16-byte load
    constexpr int HOLD = 4;                            // 16-byte loads kept per thread
    __shared__ float s_red[4];
    __shared__ float s_slice[256];                     // this workgroup's 256 inputs
    const int m = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t xrow = static_cast<size_t>(m) * K;
    const uint4* xv = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                     xrow * (DT == BITQ_DT_F32 ? 4 : 2));
    const int nvec = K / VEC;           // K is a multiple of 32
    const int lo = 256 * blockIdx.x;    // first input of this workgroup

    // ---- one pass over the row: amax, and this workgroup's inputs to LDS
    float amax = 0.0f;
    auto take = [&](int i, const uint4& u) {
        const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v0, v1;
            if (DT == BITQ_DT_F32) {
                v0 = __uint_as_float(a[e]);
                amax = fmaxf(amax, fabsf(v0));
                const int k = i * VEC + e;
                if (k >= lo && k < lo + 256) s_slice[k - lo] = v0;
            } else {
                v0 = __uint_as_float(a[e] << 16);
                v1 = __uint_as_float(a[e] & 0xFFFF0000u);
                amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
                const int k = i * VEC + 2 * e;
                if (k >= lo && k < lo + 256) {
                    s_slice[k - lo] = v0;
                    s_slice[k + 1 - lo] = v1;
                }
            }
        }
    };
    {
        uint4 hold[HOLD];
#pragma unroll
        for (int h = 0; h < HOLD; ++h) {  // all loads of the first pass in flight together
            const int i = tid + 256 * h;
            hold[h] = (i < nvec) ? xv[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int h = 0; h < HOLD; ++h)
            if (tid + 256 * h < nvec) take(tid + 256 * h, hold[h]);
    }
    for (int i = tid + 256 * HOLD; i < nvec; i += 256) take(i, xv[i]);
    amax = wave_max(amax);
    if (lane == 0) s_red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    if constexpr (RANK > 0) {
        __shared__ float s_part[256];
        const int c = tid / RANK, j = tid % RANK;
        const int k0 = lo + RANK * c;       // this thread's run; inputs past K count as 0
        const int kc = min(k0, Kp - RANK);  // in-bounds row position (runs past Kp have x = 0)
        const uint4* arow = reinterpret_cast<const uint4*>(blob + off_at) + (static_cast<size_t>(j) * Kp + kc) / 8;
        uint4 av[RANK / 8];
#pragma unroll
        for (int i = 0; i < RANK / 8; ++i) av[i] = arow[i];
        const float amax_a = *reinterpret_cast<const float*>(blob + kHdrAmaxA);
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < RANK / 8; ++i) {
            const uint32_t a[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = k0 + 8 * i + e;
                const float xk = (k < K) ? s_slice[k - lo] : 0.0f;
                part = fmaf(xk, f16_bits_to_f32(a[e >> 1] >> (16 * (e & 1))), part);
            }
        }
        s_part[tid] = part;
        __syncthreads();
        if (tid < RANK) {
            float col = 0.0f;
            for (int cc = 0; cc < 256 / RANK; ++cc) col += s_part[RANK * cc + tid];
            const double bound = static_cast<double>(K) * static_cast<double>(amax) * static_cast<double>(amax_a);
            lora_arrive(&ws[static_cast<size_t>(m) * RANK + tid], col, bound, static_cast<int>(gridDim.x),
                        &hout[static_cast<size_t>(m) * RANK + tid]);
        }
    }
    float s = 0.0f;
    if (amax > 0.0f) s = __fdiv_rn(qmax, amax);
    if (blockIdx.x == 0 && tid == 0) dq[m] = (amax > 0.0f) ? __fdiv_rn(amax, qmax) : 0.0f;

    // ---- this wave's 64 inputs = words w0 and w0 + 1
    const int w0 = 8 * blockIdx.x + 2 * wave;
    if (w0 >= Kw) return;
    const int k = 32 * w0 + lane;
    int qi = 0;
    if (k < K && amax > 0.0f) {
        const float r = rintf(__fmul_rn(s_slice[k - lo], s));
        qi = static_cast<int>(fminf(fmaxf(r, -qmax), qmax));
    }
    q[static_cast<size_t>(m) * (Kw * 32) + k] = static_cast<int8_t>(qi);
    // planes: lane j (< 8) keeps plane j of word w0, lane 8 + j of word w0 + 1
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t b = __ballot((qi >> j) & 1);
        if (lane == j) mine = static_cast<uint32_t>(b);
        if (lane == 8 + j) mine = static_cast<uint32_t>(b >> 32);
    }
    if (lane < 16) planes[(static_cast<size_t>(m) * Kw + w0) * 8 + lane] = mine;
    // group sums of the two words: reductions inside each half of the wave
    int sum = qi;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) S[static_cast<size_t>(m) * Kw + w0] = sum;
    if (lane == 32) S[static_cast<size_t>(m) * Kw + w0 + 1] = sum;
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

// ====================================================== AND+popcount GEMV
// Integer activations q (int8, two's-complement planes X_j with weights
// c_j = 2^j, c_7 = -128) against binary weight planes W_i:
//   sum_k qw_k q_k = sum_i sum_j u_i c_j popcount(W_i AND X_j)
// ([ABQ] abstract and §1: arbitrary-bit products rebuilt from binary
// operations instead of INT4/INT8 units; [BVSR] intro: AND and population
// count directly on the bitvectors, without dequantization).  Each weight
// word costs one AND and one popcount-accumulate (v_bcnt_u32_b32) per
// activation plane; the activation plane words come from LDS.
//
// Per-token epilogues (y before the per-token factor d, applied at the end):
//   TERNARY ([HGF] §1.2): Y = sum_j c_j (popc(P & X_j) - popc(M & X_j)),
//           y = gamma d Y
//   W2A8 ([ABQ] Eq. 3): per 128-group A = sum_j c_j (a0_j + 2 a1_j),
//           y += delta (A - z S128)
//   BVSR4 ([BVSR]): per 32-group P_k = sum_j c_j popc(beta_k & X_j),
//           y += b S32 + sum_k c_k P_k with (c, b) = cache[idx]

// popcount(v) + acc as one v_bcnt_u32_b32 (keeps the accumulation a chain
// of accumulating popcounts instead of separate popcounts plus adds).
__device__ __forceinline__ int bcnt_acc(uint32_t v, int acc) {
    int r;
    asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));
    return r;
}

// Workgroup barrier that first waits until at most N vector-memory loads of
// this wave are still outstanding (loads retire in issue order, so every load
// issued before the last N has landed, including copies into LDS) and all LDS
// accesses are done.  Loads issued after the copies can stay in flight.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// v of another lane of the same quad (DPP quad_perm: lane i of each group of
// 4 takes lane CTRL[2i+1:2i]).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_swap(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// A wave-uniform value moved to a scalar register (the compiler cannot tell
// that threadIdx.x / 64 is uniform).
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Horner combination of per-plane popcounts: sum_j c_j a_j.
__device__ __forceinline__ int combine_planes(const int (&a)[8]) {
    int r = -a[7];
#pragma unroll
    for (int j = 6; j >= 0; --j) r = 2 * r + a[j];
    return r;
}

// ================================= AND+popcount GEMV, whole k per workgroup
// No hand-off between workgroups: a workgroup (256 threads) owns RG rows
// (16 or 8) and the whole k range.  Thread (g, r) = (tid / RG, tid % RG)
// takes row r of the group and the k blocks b = g + G j (j < BPL, G = 256/RG
// k-groups) of each round of G BPL blocks; the RG lanes of a k-group read RG
// adjacent rows of a tile (16 RG contiguous bytes per load).  Activation
// planes and group sums of the round are staged once in LDS; the G k-groups'
// results for a row are added in a fixed order (lane exchanges, then four
// waves through LDS).
//
// HGF layers run the ternary loop and add, in the epilogue of each row, the
// correction's up projection gate sum_j h_j B[j][n] ([HGF] §4.1 asks for the
// ternary product and the correction in one kernel): the workgroup's RG rows
// of B^T (RG rank fp16) and the token's h (rank floats, written by the
// activation step) are copied into LDS ahead of the weight stream.
//
// XQ = 1 (bf16) or 2 (fp32): the activation quantizer runs in this kernel's
// prologue instead of a separate launch (one token, whole k range in one
// round).  `act` is then the raw x.  Every workgroup loads all of x (small,
// L2-resident) ahead of its weight stream, reduces amax, and quantizes it
// with the separate quantizer's arithmetic (s = fl32(Qm/amax), q =
// rint(fl32(x s)), d = fl32(amax/Qm)), so planes, group sums and d are the
// same bits as that quantizer's (and y the same bits as the two-launch path
// whenever both use the same rows per workgroup).  A lane takes 8 inputs (a
// chunk); fl32(x s) + 1.5 2^23 rounds to the nearest integer (ties to even,
// as rint) and leaves q in the low byte of the float's bits (|q| <= Qm <
// 2^22).  The 8 code bytes of a chunk are bit-transposed as an 8x8 bit matrix
// (byte j = plane j of the chunk), and the 4 lanes of a 32-input word
// assemble its 8 plane words with two byte-permute exchanges.  No clamp is
// needed: |x| <= amax gives |fl32(x s)| < Qm + 1/2.
template <int FMT, int P, bool ACC, int BPL, int RG, bool ONE, int XQ = 0>
__global__ __launch_bounds__(256) void gemv_bits_nr_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                           size_t off_c1, const uint8_t* __restrict__ act,
                                                           size_t act_off_S, size_t act_off_d, int M, int N, int K,
                                                           int Tb, int abits, size_t off_c2, size_t act_off_h,
                                                           int rank, float* __restrict__ y) {
    constexpr bool TERN = FMT == BITQ_TERNARY || FMT == BITQ_HGF;  // ternary planes
    constexpr bool LORA = FMT == BITQ_HGF && !ACC;                 // the correction epilogue
    constexpr int G = 256 / RG;    // k-groups: lanes that share a row
    constexpr int Q = 64 / RG;     // row groups per 64-row tile
    constexpr int NBW = G * BPL;   // k blocks per round
    constexpr int BSTR = 36;       // LDS words per block: 32 + 4 padding, so up to
                                   // 8 k-groups of a wave hit disjoint banks
    // Activation staging goes straight from global memory into LDS
    // (global_load_lds_dwordx4: lane l of a wave fills the 16-byte slot l of
    // the wave's destination), in whole passes of 256 lanes.  A block takes 9
    // slots: its 8 plane uint4 and one slot of padding.
    constexpr int SLOT_PASSES = (NBW * 9 + 255) / 256;
    constexpr int S_PASSES = (NBW + 255) / 256;
    __shared__ __attribute__((aligned(16))) uint32_t s_act[SLOT_PASSES * 256 * 4];
    __shared__ __attribute__((aligned(16))) int32_t s_S[S_PASSES * 256 * 4];
    __shared__ float4 s_cache[FMT == BITQ_BVSR4 ? 512 : 1];
    // HGF: B^T rows of the group (RG x rank fp16, rank <= 64: RG 8 slots of
    // 16 bytes) and h of the current token (rank floats; the copy fills one
    // 16-byte slot per lane of a wave: 64 slots).  Declared as one word
    // array: with vector-typed arrays of template-dependent size here, this
    // compiler drops the kernel's host-side stub.
    __shared__ __attribute__((aligned(16))) uint32_t s_lora[FMT == BITQ_HGF ? (RG * 8 + 64) * 4 : 4];
    uint4* const s_bt = reinterpret_cast<uint4*>(s_lora);
    float4* const s_h = reinterpret_cast<float4*>(s_lora + RG * 8 * 4);
    __shared__ float s_red[4][16];
    __shared__ int32_t s_redi[4][16];
    constexpr bool FQ = XQ != 0;   // fused activation quantizer
    static_assert(!FQ || (ONE && !ACC && FMT != BITQ_HGF), "fused quantizer: whole k in one round, y output");

    const int tid = threadIdx.x, r = tid % RG, g = tid / RG, wave = tid >> 6;
    // the wave index as a uniform value, for branches around the LDS copies
    // (their LDS destination must be uniform)
    const int wave_u = wave_uniform(wave);
    // Workgroup wg runs on XCD wg mod 8 (round-robin dispatch); the Q row
    // groups of a 64-row tile go to workgroups wg, wg+8, ..., wg+8(Q-1) of one
    // XCD, so the tile's coefficient lines (64 rows x 4 bytes) are fetched
    // into a single L2.
    const int wg = blockIdx.x;
    const int t = 8 * (wg / (8 * Q)) + (wg & 7);  // 64-row tile
    const int quarter = (wg >> 3) % Q;
    if (t >= (N + 63) / 64) return;               // padding workgroups of the last XCD round
    const int rowin = RG * quarter + r;           // row inside the tile
    const int n = 64 * t + rowin;
    const int NB = Tb;
    const int Kw = Tb * 4;
    const int rounds = (NB + NBW - 1) / NBW;
    const uint32_t* __restrict__ aplanes = reinterpret_cast<const uint32_t*>(act);
    const int32_t* __restrict__ aS = reinterpret_cast<const int32_t*>(act + act_off_S);
    const float* __restrict__ ad = reinterpret_cast<const float*>(act + act_off_d);

    uint4 wv[BPL][P];
    uint32_t coef[BPL];
    // uniform 64-bit bases of this tile; per-lane offsets fit in 32 bits
    const uint8_t* __restrict__ tile_planes = blob + kHeaderBytes + static_cast<size_t>(t) * Tb * P * 1024;
    const uint32_t* __restrict__ tile_coef = reinterpret_cast<const uint32_t*>(blob + off_c0) + static_cast<size_t>(t) * Tb * 64;
    auto load_weights = [&](int b_base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            const int b = min(b_base + g + G * j, NB - 1);  // in bounds; surplus skipped below
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const uint32_t off = static_cast<uint32_t>((b * P + p) * 1024 + rowin * 16);
                wv[j][p] = *reinterpret_cast<const uint4*>(tile_planes + off);
            }
            coef[j] = 0;
            if (FMT == BITQ_W2A8 || FMT == BITQ_BVSR4 || FMT == BITQ_WNAM)
                coef[j] = tile_coef[static_cast<uint32_t>(b * 64 + rowin)];
        }
    };
    // Staging of the activation planes and sums of blocks [b_base, b_base +
    // NBW) into LDS.  The copies complete asynchronously (counted like any
    // other load), so they are issued ahead of the weight stream and land
    // while it is still in flight.  Slots past the last real block receive
    // copies of it (clamped addresses); the compute loop skips those blocks.
    auto stage = [&](int m, int b_base) __attribute__((always_inline)) {
        const uint4* src = reinterpret_cast<const uint4*>(aplanes) + (static_cast<size_t>(m) * Kw + 4 * b_base) * 2;
        const int last = min(NBW, NB - b_base) - 1;  // last real block of the round
#pragma unroll
        for (int v = 0; v < SLOT_PASSES; ++v) {
            const int slot = tid + 256 * v;
            const int blk = slot / 9, part = slot - 9 * blk;
            __builtin_amdgcn_global_load_lds(src + 8 * min(blk, last) + min(part, 7),
                                             reinterpret_cast<uint4*>(s_act) + 256 * v + 64 * wave, 16, 0, 0);
        }
        const int4* srcS = reinterpret_cast<const int4*>(aS + static_cast<size_t>(m) * Kw + 4 * b_base);
#pragma unroll
        for (int v = 0; v < S_PASSES; ++v)
            __builtin_amdgcn_global_load_lds(srcS + min(tid + 256 * v, last),
                                             reinterpret_cast<int4*>(s_S) + 256 * v + 64 * wave, 16, 0, 0);
        if (LORA && b_base == 0 && wave_u == 0) {  // h[m]: rank / 4 16-byte slots
            const float4* hsrc = reinterpret_cast<const float4*>(act + act_off_h) + static_cast<size_t>(m) * (rank / 4);
            // (wave_u is 0 here; a destination computed from it, rather than
            // the constant s_h, avoids a crash of this compiler's SGPR-copy pass)
            __builtin_amdgcn_global_load_lds(hsrc + min(tid, rank / 4 - 1), s_h + 64 * wave_u, 16, 0, 0);
        }
    };

    // Issue order: coefficient cache (BVSR), activation copies, then the
    // weight stream; kWeightLoads loads follow the copies, so the barrier
    // below waits for the copies without waiting for the weights.
    constexpr int kWeightLoads = BPL * P + ((FMT == BITQ_W2A8 || FMT == BITQ_BVSR4 || FMT == BITQ_WNAM) ? BPL : 0);
    if (FMT == BITQ_BVSR4 && !ACC) {
        // cache entry e (c0..c3, b; 5 floats) -> LDS floats 8e..8e+4 by 4-byte
        // copies; floats 8e+5..8e+7 are never read (they get copies of b)
        const float* cache = reinterpret_cast<const float*>(blob + off_c1);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int slot = tid + 256 * v, e = slot >> 3, f = slot & 7;
            __builtin_amdgcn_global_load_lds(cache + 5 * e + min(f, 4),
                                             reinterpret_cast<float*>(s_cache) + 256 * v + 64 * wave, 4, 0, 0);
        }
    }
    if (LORA && wave_u < RG / 8) {
        // B^T rows 64t + RG quarter .. + RG - 1 are contiguous: RG rank / 8
        // 16-byte slots (<= 128, waves 0 and 1; the rows exist up to Np)
        const uint4* bsrc = reinterpret_cast<const uint4*>(blob + off_c2) +
                            static_cast<size_t>(64 * t + RG * quarter) * (rank / 8);
        __builtin_amdgcn_global_load_lds(bsrc + min(tid, RG * (rank / 8) - 1), s_bt + 64 * wave_u, 16, 0, 0);
    }
    // fused quantizer: chunks c = tid + 256 i of 8 inputs (word c / 4, byte
    // c % 4 of its plane words); XLPC 16-byte loads each
    constexpr int XCPT = FQ ? NBW * 16 / 256 : 1;
    constexpr int XLPC = XQ == 2 ? 2 : 1;
    static_assert(!FQ || (NBW * 16) % 256 == 0, "whole chunks per thread");
    uint4 xr[XCPT][XLPC];
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FQ) {
        // unconditional loads (clamped to the last chunk of x) through an
        // address without the argument's restrict provenance, kept ahead of
        // the weight stream by the memory clobber
        uintptr_t xaddr = reinterpret_cast<uintptr_t>(act);
        asm volatile("" : "+s"(xaddr));
        const int nch = K / 8;
#pragma unroll
        for (int i = 0; i < XCPT; ++i) {
            const int c = min(tid + 256 * i, nch - 1);
#pragma unroll
            for (int l = 0; l < XLPC; ++l) xr[i][l] = global_load16(xaddr, XLPC * c + l);
        }
        asm volatile("" ::: "memory");
    } else if (ONE) {
        stage(0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ONE) load_weights(0);
    __builtin_amdgcn_sched_barrier(0);

    float dq_fused = 0.0f;  // the token's d (fused quantizer)
    if constexpr (FQ) {
        __shared__ float s_amax[4];
        // 8 inputs of chunk i as floats (fp32: two 16-byte loads; the index
        // XLPC - 1 keeps the bf16 instantiation, which never takes that
        // branch, inside the array)
        auto chunk = [&](int i, float (&v)[8]) __attribute__((always_inline)) {
            if (XQ == 2) {
                v[0] = __uint_as_float(xr[i][0].x); v[1] = __uint_as_float(xr[i][0].y);
                v[2] = __uint_as_float(xr[i][0].z); v[3] = __uint_as_float(xr[i][0].w);
                v[4] = __uint_as_float(xr[i][XLPC - 1].x); v[5] = __uint_as_float(xr[i][XLPC - 1].y);
                v[6] = __uint_as_float(xr[i][XLPC - 1].z); v[7] = __uint_as_float(xr[i][XLPC - 1].w);
            } else {
                const uint32_t u[4] = {xr[i][0].x, xr[i][0].y, xr[i][0].z, xr[i][0].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(u[e] << 16);
                    v[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
                }
            }
        };
        // amax over x (clamped duplicates do not change it)
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < XCPT; ++i) {
            float v[8];
            chunk(i, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
        }
        am = wave_max(am);
        if ((tid & 63) == 0) s_amax[wave] = am;
        barrier_after_loads<kWeightLoads>();
        am = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
        const float qmax = FMT == BITQ_WNAM ? static_cast<float>((1 << (abits - 1)) - 1) : 127.0f;
        const float sx = am > 0.0f ? __fdiv_rn(qmax, am) : 0.0f;
        dq_fused = am > 0.0f ? __fdiv_rn(am, qmax) : 0.0f;
        constexpr uint32_t kMagic = 0x4B400000u;  // bits of 1.5 2^23
        // byte-permute selectors of the two exchanges, v_perm(partner, own)
        // (lane e = tid % 4 of the word; bytes 0-3 select own, 4-7 partner's):
        // after the first, even lanes hold 16-bit halves of planes (0, 1) of
        // lanes (e, e+1), odd lanes planes (2, 3) of lanes (e-1, e); after the
        // second, lane e holds the whole word of plane pl (and pl + 4 from hi)
        const uint32_t sel1 = (tid & 1) ? 0x03070206u : 0x05010400u;
        const uint32_t sel2 = (tid & 2) ? 0x03020706u : 0x05040100u;
        const int pl = ((tid & 1) << 1) | ((tid >> 1) & 1);
        const int nch = K / 8;
#pragma unroll
        for (int i = 0; i < XCPT; ++i) {
            const int c = tid + 256 * i;
            const float sc = c < nch ? sx : 0.0f;  // chunks past K quantize to 0
            float v[8];
            chunk(i, v);
            uint32_t b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = __float_as_uint(__fadd_rn(__fmul_rn(v[e], sc), 12582912.0f));
            // group sum of the chunk: sum (bits - magic) = sum q
            int S = static_cast<int>((b[0] + b[1] + b[2] + b[3]) + (b[4] + b[5] + b[6] + b[7]) - 8u * kMagic);
            // code bytes (input e in byte e % 4 of lo / hi)
            uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
            uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
            // 8x8 bit transpose of the 64-bit value hi:lo (bit 8e + j <-> 8j + e)
            uint32_t t;
            t = (lo ^ (lo >> 7)) & 0x00AA00AAu; lo = lo ^ t ^ (t << 7);
            t = (hi ^ (hi >> 7)) & 0x00AA00AAu; hi = hi ^ t ^ (t << 7);
            t = (lo ^ (lo >> 14)) & 0x0000CCCCu; lo = lo ^ t ^ (t << 14);
            t = (hi ^ (hi >> 14)) & 0x0000CCCCu; hi = hi ^ t ^ (t << 14);
            t = (lo ^ (hi << 4)) & 0xF0F0F0F0u; lo ^= t; hi ^= t >> 4;
            // exchange 1 with lane e ^ 1, exchange 2 with lane e ^ 2 (DPP quad
            // permutations 1,0,3,2 and 2,3,0,1)
            lo = __builtin_amdgcn_perm(quad_swap<0xB1>(lo), lo, sel1);
            hi = __builtin_amdgcn_perm(quad_swap<0xB1>(hi), hi, sel1);
            lo = __builtin_amdgcn_perm(quad_swap<0x4E>(lo), lo, sel2);
            hi = __builtin_amdgcn_perm(quad_swap<0x4E>(hi), hi, sel2);
            S += static_cast<int>(quad_swap<0xB1>(static_cast<uint32_t>(S)));
            S += static_cast<int>(quad_swap<0x4E>(static_cast<uint32_t>(S)));
            const int word = c >> 2;  // 32-input word of the round: block word / 4, its word word % 4
            uint32_t* dst = &s_act[(word >> 2) * BSTR + 8 * (word & 3)];
            dst[pl] = lo;
            dst[pl + 4] = hi;
            if ((tid & 3) == 0) s_S[word] = S;
        }
        barrier_after_loads<kWeightLoads>();
    }

    // one activation row; the first is peeled so that its loads need no wait
    // at a loop header
    auto pass = [&](int m, bool first) __attribute__((always_inline)) {
        // per-token (and per-tensor) scales: uniform loads issued now, long
        // before the epilogue needs them
        const float scale = (TERN && !ACC ? *reinterpret_cast<const float*>(blob + off_c0) : 1.0f) *
                            (ACC ? 1.0f : (FQ ? dq_fused : ad[m]));
        const float gate = LORA ? *reinterpret_cast<const float*>(blob + kHdrGate) : 0.0f;
        float yacc = 0.0f;
        int tacc[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) tacc[i][j] = 0;

        for (int rd = 0; rd < (ONE ? 1 : rounds); ++rd) {
            const int b_base = rd * NBW;
            if (!first || rd > 0) __syncthreads();  // previous readers of s_act are done
            if (!ONE) {
                stage(m, b_base);
                __builtin_amdgcn_sched_barrier(0);
                load_weights(b_base);
                __builtin_amdgcn_sched_barrier(0);
                barrier_after_loads<kWeightLoads>();
            } else if (first) {
                if (!FQ) barrier_after_loads<kWeightLoads>();  // copies issued in the prologue
            } else {
                stage(m, b_base);
                barrier_after_loads<0>();
            }
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const int bl = g + G * j;  // block inside the round
                const int b = b_base + bl;
                if (b >= NB) continue;
                const uint32_t* xa = &s_act[bl * BSTR];
                // Use of this block's coefficient word starts here: without the
                // empty asm the compiler hoists its decoding, and the wait for
                // it, above the barrier, ahead of the whole weight stream.
                uint32_t cw = coef[j];
                asm volatile("" : "+v"(cw));
                // ternary and W2A8: the block's 8 activation-plane reads are
                // issued together ahead of the popcounts (one LDS wait instead
                // of four; W2A8 11008x4096 5.18 -> 5.12 us).  Not for HGF and
                // BVSR4, whose extra registers cost more than the wait (BVSR
                // 28672x8192 30.4 -> 31.5 us).
                constexpr bool HOIST = FMT == BITQ_TERNARY || FMT == BITQ_W2A8;
                uint4 xq[4][2];
                if (HOIST) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        xq[w][0] = *reinterpret_cast<const uint4*>(xa + 8 * w);
                        xq[w][1] = *reinterpret_cast<const uint4*>(xa + 8 * w + 4);
                    }
                }
                if (TERN) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint4 x0 = HOIST ? xq[w][0] : *reinterpret_cast<const uint4*>(xa + 8 * w);
                        const uint4 x1 = HOIST ? xq[w][1] : *reinterpret_cast<const uint4*>(xa + 8 * w + 4);
                        const uint32_t xj[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                        const uint32_t wp = (&wv[j][0].x)[w], wm = (&wv[j][1].x)[w];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            tacc[0][jj] = bcnt_acc(wp & xj[jj], tacc[0][jj]);
                            tacc[1][jj] = bcnt_acc(wm & xj[jj], tacc[1][jj]);
                        }
                    }
                } else if (FMT == BITQ_W2A8) {
                    int a[2][8];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) a[i][jj] = 0;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint4 x0 = xq[w][0];
                        const uint4 x1 = xq[w][1];
                        const uint32_t xj[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                        const uint32_t w0 = (&wv[j][0].x)[w], w1 = (&wv[j][1].x)[w];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            a[0][jj] = bcnt_acc(w0 & xj[jj], a[0][jj]);
                            a[1][jj] = bcnt_acc(w1 & xj[jj], a[1][jj]);
                        }
                    }
                    int t8[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) t8[jj] = a[0][jj] + 2 * a[1][jj];
                    const int A = combine_planes(t8);
                    if (ACC) {
                        if (n < N) reinterpret_cast<int32_t*>(y)[(static_cast<size_t>(m) * N + n) * NB + b] = A;
                    } else {
                        const int4 S4 = *reinterpret_cast<const int4*>(&s_S[4 * bl]);
                        const int S128 = S4.x + S4.y + S4.z + S4.w;
                        const float delta = f16_bits_to_f32(cw);
                        const float z = f16_bits_to_f32(cw >> 16);
                        yacc += delta * (static_cast<float>(A) - z * static_cast<float>(S128));
                    }
                } else if (FMT == BITQ_WNAM) {
                    // n = P weight planes, m = abits activation planes: the sign
                    // plane 7 (weight -2^(m-1)), then planes m-2 .. 0 in a loop
                    // of m - 1 steps (bits m-1..6 of an m-bit code are sign
                    // copies), Horner-accumulated per weight plane:
                    //   r_i = -c_i7, then r_i = 2 r_i + c_ij,  c_ij = sum_w popc(W_i & X_j)
                    uint32_t wi[P][4];
#pragma unroll
                    for (int i = 0; i < P; ++i) {
                        wi[i][0] = wv[j][i].x; wi[i][1] = wv[j][i].y; wi[i][2] = wv[j][i].z; wi[i][3] = wv[j][i].w;
                    }
                    int r[P];
#pragma unroll
                    for (int i = 0; i < P; ++i) {
                        int c = 0;
#pragma unroll
                        for (int w = 0; w < 4; ++w) c = bcnt_acc(wi[i][w] & xa[8 * w + 7], c);
                        r[i] = -c;
                    }
                    for (int jj = abits - 2; jj >= 0; --jj) {
                        uint32_t xw[4];
#pragma unroll
                        for (int w = 0; w < 4; ++w) xw[w] = xa[8 * w + jj];
#pragma unroll
                        for (int i = 0; i < P; ++i) {
                            int c = 0;
#pragma unroll
                            for (int w = 0; w < 4; ++w) c = bcnt_acc(wi[i][w] & xw[w], c);
                            r[i] = 2 * r[i] + c;
                        }
                    }
                    int A = r[P - 1];
#pragma unroll
                    for (int i = P - 2; i >= 0; --i) A = 2 * A + r[i];
                    if (ACC) {
                        if (n < N) reinterpret_cast<int32_t*>(y)[(static_cast<size_t>(m) * N + n) * NB + b] = A;
                    } else {
                        const int4 S4 = *reinterpret_cast<const int4*>(&s_S[4 * bl]);
                        const int S128 = S4.x + S4.y + S4.z + S4.w;
                        const float delta = f16_bits_to_f32(cw);
                        const float z = f16_bits_to_f32(cw >> 16);
                        yacc += delta * (static_cast<float>(A) - z * static_cast<float>(S128));
                    }
                } else {  // BVSR4
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint4 x0 = *reinterpret_cast<const uint4*>(xa + 8 * w);
                        const uint4 x1 = *reinterpret_cast<const uint4*>(xa + 8 * w + 4);
                        const uint32_t xj[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                        int Pk[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t bk = (&wv[j][k].x)[w];
                            int a8[8];
#pragma unroll
                            for (int jj = 0; jj < 8; ++jj) a8[jj] = bcnt_acc(bk & xj[jj], 0);
                            Pk[k] = combine_planes(a8);
                        }
                        const int gi = 4 * b + w;
                        if (ACC) {
                            const int G = K / 32;  // groups of the real (unpadded) K
                            int4* dst = reinterpret_cast<int4*>(y) + (static_cast<size_t>(m) * N + n) * G + gi;
                            if (n < N && gi < G) *dst = make_int4(Pk[0], Pk[1], Pk[2], Pk[3]);
                        } else {
                            const int id = (cw >> (8 * w)) & 0xFF;
                            const float4 c = s_cache[2 * id];
                            const float bo = s_cache[2 * id + 1].x;
                            const float S32 = static_cast<float>(s_S[4 * bl + w]);
                            yacc += bo * S32 + c.x * static_cast<float>(Pk[0]) + c.y * static_cast<float>(Pk[1]) +
                                    c.z * static_cast<float>(Pk[2]) + c.w * static_cast<float>(Pk[3]);
                        }
                    }
                }
            }
        }
        if (ACC && !TERN) return;  // partials already written per group

        // ---- add the G k-groups of each row in a fixed order
        if (TERN && ACC) {
            int Y[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) Y[jj] = tacc[0][jj] - tacc[1][jj];
            int v = combine_planes(Y);
#pragma unroll
            for (int sh = RG; sh < 64; sh *= 2) v += __shfl_xor(v, sh, 64);
            if ((tid & 63) < RG) s_redi[wave][r] = v;
            __syncthreads();
            if (tid < RG && n < N)
                reinterpret_cast<int32_t*>(y)[static_cast<size_t>(m) * N + n] =
                    (s_redi[0][r] + s_redi[1][r]) + (s_redi[2][r] + s_redi[3][r]);
        } else {
            float v;
            if (TERN) {
                int Y[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) Y[jj] = tacc[0][jj] - tacc[1][jj];
                v = static_cast<float>(combine_planes(Y));  // exact while |Y| < 2^24 (K <= 2^17)
            } else {
                v = yacc;
            }
#pragma unroll
            for (int sh = RG; sh < 64; sh *= 2) v += __shfl_xor(v, sh, 64);
            if ((tid & 63) < RG) s_red[wave][r] = v;
            __syncthreads();
            if (tid < RG && n < N) {
                float tot = (s_red[0][r] + s_red[1][r]) + (s_red[2][r] + s_red[3][r]);
                tot = scale * tot;
                if (LORA) {  // gate sum_j h_j B[j][n], fp32 in j order
                    float l = 0.0f;
                    const uint4* bt = &s_bt[r * (rank / 8)];
                    for (int c = 0; c < rank / 8; ++c) {
                        const uint4 b = bt[c];
                        const float4 h0 = s_h[2 * c], h1 = s_h[2 * c + 1];
                        l = fmaf(h0.x, f16_bits_to_f32(b.x), l);
                        l = fmaf(h0.y, f16_bits_to_f32(b.x >> 16), l);
                        l = fmaf(h0.z, f16_bits_to_f32(b.y), l);
                        l = fmaf(h0.w, f16_bits_to_f32(b.y >> 16), l);
                        l = fmaf(h1.x, f16_bits_to_f32(b.z), l);
                        l = fmaf(h1.y, f16_bits_to_f32(b.z >> 16), l);
                        l = fmaf(h1.z, f16_bits_to_f32(b.w), l);
                        l = fmaf(h1.w, f16_bits_to_f32(b.w >> 16), l);
                    }
                    tot = fmaf(gate, l, tot);
                }
                y[static_cast<size_t>(m) * N + n] = tot;
            }
        }
    };
    pass(0, true);
    if (!FQ)
        for (int m = 1; m < M; ++m) pass(m, false);
}

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

// ================================================== binary activations (XNOR)
// [BitNet] §2.1 sign with the tie at 0 going to +1 (so -0.0 -> +1): one bit
// per input, 1 <-> +1, LSB first, zero bits past K.  beta = mean_k |x_k| is
// the per-token scale of the fully binary product (workgroup 0 of each token
// sums the row in a fixed order).  The 16-byte loads need x 16-byte aligned.  Grid (words / 8, M), 256 lanes: each wave
// turns 64 inputs into two words with one ballot.
template <int DT>
__global__ __launch_bounds__(256) void binarize_act_kernel(const void* __restrict__ x, int K, int Kw,
                                                           uint32_t* __restrict__ bits, float* __restrict__ beta) {
    __shared__ float s_sum[4];
    const int m = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row = static_cast<size_t>(m) * K;
    const int w0 = 8 * blockIdx.x + 2 * wave;
    const int k = 32 * w0 + lane;
    const bool pos = k < K && act_at<DT>(x, row + min(k, K - 1)) >= 0.0f;
    const uint64_t b = __ballot(pos);
    if (w0 < Kw) {
        if (lane == 0) bits[static_cast<size_t>(m) * Kw + w0] = static_cast<uint32_t>(b);
        if (lane == 32 && w0 + 1 < Kw) bits[static_cast<size_t>(m) * Kw + w0 + 1] = static_cast<uint32_t>(b >> 32);
    }
    if (blockIdx.x != 0) return;
    // sum |x| of the row: 16-byte loads, four in flight per lane, fixed order
    constexpr int VEC = (DT == BITQ_DT_F32) ? 4 : 8;
    const uint4* xv = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) + row * (DT == BITQ_DT_F32 ? 4 : 2));
    const int nvec = K / VEC;  // K is a multiple of 32
    float sum = 0.0f;
    for (int i0 = 0; i0 < nvec; i0 += 1024) {
        uint4 v[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) v[h] = xv[min(i0 + tid + 256 * h, nvec - 1)];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t keep = i0 + tid + 256 * h < nvec ? 0xFFFFFFFFu : 0u;  // clamped duplicates add 0
            const uint32_t a[4] = {v[h].x & keep, v[h].y & keep, v[h].z & keep, v[h].w & keep};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (DT == BITQ_DT_F32) sum += fabsf(__uint_as_float(a[e]));
                else sum += fabsf(__uint_as_float(a[e] << 16)) + fabsf(__uint_as_float(a[e] & 0xFFFF0000u));
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) beta[m] = ((s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3])) / static_cast<float>(K);
}

// ====================================================== XNOR+popcount GEMV
// [BitNet] §2.3: with both operands in {-1,+1} as sign bits (1 <-> +1),
//   Y[m,n] = sum_k B[n,k] x_b[m,k] = K - 2 popcount(bits(B_n) XOR bits(x_m))
// (the page prints popcount(xnor) times the scale; the affine map makes it
// the dot product), one XOR and one popcount-accumulate per 32 weights, and
// y = alpha_n beta_m Y.  Zero padding bits of both operands agree, so only
// the real K counts.  Workgroups as in the AND+popcount kernel (RG rows x
// 256/RG k-groups, row groups of a tile on one XCD), k in rounds of G BPL
// blocks; the sign words of x come straight from global memory (one 16-byte
// load per block, the same for the RG lanes of a k-group).  Per-token counts
// are added in LDS with integer atomics: exact and order-independent.
template <bool ACC, int BPL, int RG>
__global__ __launch_bounds__(256) void gemv_xnor_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                        const uint8_t* __restrict__ act, size_t act_off_beta, int M,
                                                        int N, int K, int Tb, float* __restrict__ y) {
    constexpr int G = 256 / RG;
    constexpr int Q = 64 / RG;
    constexpr int NBW = G * BPL;  // k blocks per round
    __shared__ int s_cnt[64][RG];
    const int tid = threadIdx.x, r = tid % RG, g = tid / RG;
    const int wg = blockIdx.x;
    const int t = 8 * (wg / (8 * Q)) + (wg & 7);  // 64-row tile (XCD-aware, see the AND+popcount kernel)
    const int quarter = (wg >> 3) % Q;
    if (t >= (N + 63) / 64) return;               // padding workgroups of the last XCD round
    const int rowin = RG * quarter + r;
    const int NB = Tb;
    // the epilogue's scales, loaded now rather than after the k loop: a
    // thread writes row r (256 is a multiple of RG) for tokens tid / RG and
    // (tid + 256) / RG
    const float* beta = reinterpret_cast<const float*>(act + act_off_beta);
    const float alpha_r = reinterpret_cast<const float*>(blob + off_c0)[min(64 * t + rowin, N - 1)];
    const float beta0 = beta[min(tid / RG, M - 1)], beta1 = beta[min((tid + 256) / RG, M - 1)];
    for (int i = tid; i < 64 * RG; i += 256) (&s_cnt[0][0])[i] = 0;  // visible after the barrier below
    const uint8_t* __restrict__ tile = blob + kHeaderBytes + static_cast<size_t>(t) * Tb * 1024;  // one plane
    const uint4* __restrict__ xw = reinterpret_cast<const uint4*>(act);  // [M][Kw] words = [M][NB] uint4
    const int rounds = (NB + NBW - 1) / NBW;
    for (int rd = 0; rd < rounds; ++rd) {
        const int b_base = rd * NBW;
        uint4 xv[BPL], wv[BPL];
#pragma unroll
        for (int j = 0; j < BPL; ++j) xv[j] = xw[min(b_base + g + G * j, NB - 1)];  // token 0
#pragma unroll
        for (int j = 0; j < BPL; ++j)
            wv[j] = *reinterpret_cast<const uint4*>(tile + static_cast<uint32_t>(min(b_base + g + G * j, NB - 1) * 1024 +
                                                                                 rowin * 16));
        for (int m = 0; m < M; ++m) {
            if (m > 0) {
#pragma unroll
                for (int j = 0; j < BPL; ++j) xv[j] = xw[static_cast<size_t>(m) * NB + min(b_base + g + G * j, NB - 1)];
            }
            int c = 0;
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const uint32_t keep = b_base + g + G * j < NB ? 0xFFFFFFFFu : 0u;  // clamped duplicates add 0
                c = bcnt_acc((wv[j].x ^ xv[j].x) & keep, c);
                c = bcnt_acc((wv[j].y ^ xv[j].y) & keep, c);
                c = bcnt_acc((wv[j].z ^ xv[j].z) & keep, c);
                c = bcnt_acc((wv[j].w ^ xv[j].w) & keep, c);
            }
#pragma unroll
            for (int sh = RG; sh < 64; sh *= 2) c += __shfl_xor(c, sh, 64);
            if (rd == 0 && m == 0) {
                // the empty asm keeps the scale loads up here (they have
                // landed: loads complete in order and the k loads above were
                // issued after them), instead of letting the compiler sink
                // them into the epilogue
                asm volatile("" ::"v"(alpha_r), "v"(beta0), "v"(beta1));
                __syncthreads();  // the zeroed counters, before the first add
            }
            if ((tid & 63) < RG) atomicAdd(&s_cnt[m][r], c);
        }
    }
    __syncthreads();
    for (int i = tid; i < M * RG; i += 256) {
        const int m = i / RG, rr = i % RG;  // rr == r
        const int n = 64 * t + RG * quarter + rr;
        if (n >= N) continue;
        const int Y = K - 2 * s_cnt[m][rr];
        if (ACC) {
            reinterpret_cast<int32_t*>(y)[static_cast<size_t>(m) * N + n] = Y;
        } else {
            y[static_cast<size_t>(m) * N + n] = (alpha_r * (i < 256 ? beta0 : beta1)) * static_cast<float>(Y);
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

int launch_quantize_act(const void* x, int x_dtype, int M, int K, int abits, void* act, void* stream) {
    ActLayout A = act_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    auto* planes = reinterpret_cast<uint32_t*>(base + A.off_planes);
    auto* S = reinterpret_cast<int32_t*>(base + A.off_S);
    auto* q = reinterpret_cast<int8_t*>(base + A.off_q);
    auto* d = reinterpret_cast<float*>(base + A.off_d);
    const int Kw = static_cast<int>(A.Kw);
    const dim3 grid((Kw + 7) / 8, M);
    const float qmax = static_cast<float>((1 << (abits - 1)) - 1);  // 127 for int8
    if (x_dtype == BITQ_DT_F32)
        hipLaunchKernelGGL((quant_act_kernel<BITQ_DT_F32, 0>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           x, K, Kw, qmax, planes, S, q, d, nullptr, 0, 0, nullptr, nullptr);
    else
        hipLaunchKernelGGL((quant_act_kernel<BITQ_DT_BF16, 0>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           x, K, Kw, qmax, planes, S, q, d, nullptr, 0, 0, nullptr, nullptr);
    return static_cast<int>(hipGetLastError());
}

template <int DT, int RANK>
static void launch_quant_hgf(dim3 grid, hipStream_t st, const void* x, int K, int Kw, uint32_t* planes, int32_t* S,
                             int8_t* q, float* d, const uint8_t* blob, size_t off_at, int Kp,
                             unsigned long long* ws, float* h) {
    hipLaunchKernelGGL((quant_act_kernel<DT, RANK>), grid, dim3(256), 0, st, x, K, Kw, 127.0f, planes, S, q, d, blob,
                       off_at, Kp, ws, h);
}

template <int DT>
static void launch_quant_hgf_rank(int rank, dim3 grid, hipStream_t st, const void* x, int K, int Kw,
                                  uint32_t* planes, int32_t* S, int8_t* q, float* d, const uint8_t* blob,
                                  size_t off_at, int Kp, unsigned long long* ws, float* h) {
    switch (rank) {
        case 8: launch_quant_hgf<DT, 8>(grid, st, x, K, Kw, planes, S, q, d, blob, off_at, Kp, ws, h); break;
        case 16: launch_quant_hgf<DT, 16>(grid, st, x, K, Kw, planes, S, q, d, blob, off_at, Kp, ws, h); break;
        case 32: launch_quant_hgf<DT, 32>(grid, st, x, K, Kw, planes, S, q, d, blob, off_at, Kp, ws, h); break;
        default: launch_quant_hgf<DT, 64>(grid, st, x, K, Kw, planes, S, q, d, blob, off_at, Kp, ws, h); break;
    }
}

int launch_quantize_act_hgf(const void* x, int x_dtype, int M, int K, int rank, const void* w, const BlobLayout& L,
                            void* act, void* ws, void* stream) {
    ActLayout A = act_layout(M, K, rank);
    uint8_t* base = static_cast<uint8_t*>(act);
    auto* planes = reinterpret_cast<uint32_t*>(base + A.off_planes);
    auto* S = reinterpret_cast<int32_t*>(base + A.off_S);
    auto* q = reinterpret_cast<int8_t*>(base + A.off_q);
    auto* d = reinterpret_cast<float*>(base + A.off_d);
    auto* h = reinterpret_cast<float*>(base + A.off_h);
    const int Kw = static_cast<int>(A.Kw);
    const dim3 grid((Kw + 7) / 8, M);
    const uint8_t* blob = static_cast<const uint8_t*>(w);  // A^T and amax_a are read by the kernel
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* wsw = static_cast<unsigned long long*>(ws);
    const int Kp = static_cast<int>(L.Kp);
    if (x_dtype == BITQ_DT_F32)
        launch_quant_hgf_rank<BITQ_DT_F32>(rank, grid, st, x, K, Kw, planes, S, q, d, blob, L.off_c1, Kp, wsw, h);
    else
        launch_quant_hgf_rank<BITQ_DT_BF16>(rank, grid, st, x, K, Kw, planes, S, q, d, blob, L.off_c1, Kp, wsw, h);
    return static_cast<int>(hipGetLastError());
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

template <int FMT, int P, bool ACC, int BPL, int RG>
static void launch_nr_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M,
                          float* y, hipStream_t st) {
    ActLayout A = act_layout(M, d.K, d.rank);
    // 64/RG row groups per 64-row tile, tiles dealt round-robin to the 8 XCDs:
    // the grid is padded to whole rounds of 8 tiles (extra workgroups exit)
    const int tiles = static_cast<int>(L.Tn);
    const int groups = 8 * (64 / RG) * ((tiles + 7) / 8);
    const bool one = L.Tb <= (256 / RG) * BPL;  // the whole k range in one round
    auto kern = one ? gemv_bits_nr_kernel<FMT, P, ACC, BPL, RG, true> : gemv_bits_nr_kernel<FMT, P, ACC, BPL, RG, false>;
    const int abits = d.fmt == BITQ_WNAM ? d.abits : 8;
    hipLaunchKernelGGL(kern, dim3(groups), dim3(256), 0, st, static_cast<const uint8_t*>(w), L.off_c0, L.off_c1,
                       static_cast<const uint8_t*>(act), A.off_S, A.off_d, M, d.N, d.K, static_cast<int>(L.Tb),
                       abits, L.off_c2, A.off_h, d.rank, y);
}

template <int FMT, int P, bool ACC, int RG>
static void launch_nr_rg(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w,
                         const void* act, int M, float* y, hipStream_t st) {
    if constexpr (FMT == BITQ_WNAM) {  // blocks per lane 1, 2, 4 or 8 (the plan rounds up)
        switch (pl.blocks_per_split) {
            case 1: launch_nr_bpl<FMT, P, ACC, 1, RG>(d, L, w, act, M, y, st); break;
            case 2: launch_nr_bpl<FMT, P, ACC, 2, RG>(d, L, w, act, M, y, st); break;
            case 4: launch_nr_bpl<FMT, P, ACC, 4, RG>(d, L, w, act, M, y, st); break;
            default: launch_nr_bpl<FMT, P, ACC, 8, RG>(d, L, w, act, M, y, st); break;
        }
    } else {
        switch (pl.blocks_per_split) {  // blocks per lane
            case 1: launch_nr_bpl<FMT, P, ACC, 1, RG>(d, L, w, act, M, y, st); break;
            case 2: launch_nr_bpl<FMT, P, ACC, 2, RG>(d, L, w, act, M, y, st); break;
            case 3: launch_nr_bpl<FMT, P, ACC, 3, RG>(d, L, w, act, M, y, st); break;
            case 4: launch_nr_bpl<FMT, P, ACC, 4, RG>(d, L, w, act, M, y, st); break;
            case 6: launch_nr_bpl<FMT, P, ACC, 6, RG>(d, L, w, act, M, y, st); break;
            default: launch_nr_bpl<FMT, P, ACC, 8, RG>(d, L, w, act, M, y, st); break;
        }
    }
}

template <int FMT, int P, bool ACC>
static void launch_nr(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* act,
                      int M, float* y, hipStream_t st) {
    if constexpr (FMT == BITQ_WNAM) {  // 8 rows per workgroup only
        launch_nr_rg<FMT, P, ACC, 8>(d, pl, L, w, act, M, y, st);
    } else {
        switch (pl.rows_per_wg) {  // rows per workgroup
            case 8: launch_nr_rg<FMT, P, ACC, 8>(d, pl, L, w, act, M, y, st); break;
            default: launch_nr_rg<FMT, P, ACC, 16>(d, pl, L, w, act, M, y, st); break;
        }
    }
}

template <bool ACC>
static void launch_wnam(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* act,
                        int M, float* y, hipStream_t st) {
    switch (d.planes) {
        case 1: launch_nr<BITQ_WNAM, 1, ACC>(d, pl, L, w, act, M, y, st); break;
        case 2: launch_nr<BITQ_WNAM, 2, ACC>(d, pl, L, w, act, M, y, st); break;
        case 3: launch_nr<BITQ_WNAM, 3, ACC>(d, pl, L, w, act, M, y, st); break;
        default: launch_nr<BITQ_WNAM, 4, ACC>(d, pl, L, w, act, M, y, st); break;
    }
}

int launch_binarize_act(const void* x, int x_dtype, int M, int K, void* act, void* stream) {
    BinActLayout A = binact_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    auto* bits = reinterpret_cast<uint32_t*>(base);
    auto* beta = reinterpret_cast<float*>(base + A.off_beta);
    const int Kw = static_cast<int>(A.Kw);
    const dim3 grid((Kw + 7) / 8, M);
    if (x_dtype == BITQ_DT_F32)
        hipLaunchKernelGGL(binarize_act_kernel<BITQ_DT_F32>, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           x, K, Kw, bits, beta);
    else
        hipLaunchKernelGGL(binarize_act_kernel<BITQ_DT_BF16>, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           x, K, Kw, bits, beta);
    return static_cast<int>(hipGetLastError());
}

template <bool ACC, int BPL>
static void launch_xnor_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M,
                            float* y, hipStream_t st) {
    constexpr int RG = 8;
    BinActLayout A = binact_layout(M, d.K);
    const int tiles = static_cast<int>(L.Tn);
    const int groups = 8 * (64 / RG) * ((tiles + 7) / 8);
    hipLaunchKernelGGL((gemv_xnor_kernel<ACC, BPL, RG>), dim3(groups), dim3(256), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, static_cast<const uint8_t*>(act), A.off_beta, M,
                       d.N, d.K, static_cast<int>(L.Tb), y);
}

int launch_gemv_xnor(const bitq_wdesc& d, const void* w, const void* act, int M, float* y, uint32_t flags,
                     void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool acc = (flags & BITQ_F_ACC_INT32) != 0;
    const int64_t need = (L.Tb + 31) / 32;  // blocks per lane with 32 k-groups (8 rows per workgroup)
    const int bpl = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;  // more k: rounds
    switch (bpl) {
        case 1: acc ? launch_xnor_bpl<true, 1>(d, L, w, act, M, y, st) : launch_xnor_bpl<false, 1>(d, L, w, act, M, y, st); break;
        case 2: acc ? launch_xnor_bpl<true, 2>(d, L, w, act, M, y, st) : launch_xnor_bpl<false, 2>(d, L, w, act, M, y, st); break;
        case 4: acc ? launch_xnor_bpl<true, 4>(d, L, w, act, M, y, st) : launch_xnor_bpl<false, 4>(d, L, w, act, M, y, st); break;
        default: acc ? launch_xnor_bpl<true, 8>(d, L, w, act, M, y, st) : launch_xnor_bpl<false, 8>(d, L, w, act, M, y, st); break;
    }
    return static_cast<int>(hipGetLastError());
}

template <int FMT, int P, bool ACC>
static void launch_mfma(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M, float* y,
                        hipStream_t st) {
    ActLayout A = act_layout(M, d.K, d.rank);
    const auto* wb = static_cast<const uint8_t*>(w);
    const auto* ab = static_cast<const uint8_t*>(act);
    const int Tb = static_cast<int>(L.Tb);
    const unsigned tiles = static_cast<unsigned>(L.Tn);
    // Launch shape (measured on 11008x4096 and 4096x11008 W2A8 and 4096^2
    // ternary layers, M = 2..64): 16 rows per workgroup and 8 or 16 waves
    // over k (about 4-8k waves in flight, each with one or two load chunks
    // of 2 blocks), except that on layers of 8192+ rows the q operands are
    // worth sharing by 64-row workgroups from 8 tokens on (16 waves, one
    // block per chunk, up to 16 tokens; 8 waves, two blocks, beyond).
    const int TT = (M + 15) / 16;  // token tiles of 16
    const bool wide = TT >= 2 && d.N >= 8192;
    const bool tall16 = TT == 1 && M >= 8 && d.N >= 8192;
    const bool kw16 = d.N <= 8192;
#define BITQ_MFMA(TT_, RS, KW, CH)                                                                               \
    hipLaunchKernelGGL((gemm_mfma_kernel<FMT, P, ACC, TT_, RS, KW, CH>), dim3(tiles * (4 / RS)), dim3(64 * KW), 0, \
                       st, wb, L.off_c0, ab, A.off_S, A.off_q, A.off_d, M, d.N, Tb, y)
#define BITQ_MFMA_TT(TT_)                      \
    do {                                       \
        if (wide)                              \
            BITQ_MFMA(TT_, 4, 8, 2);           \
        else if (kw16)                         \
            BITQ_MFMA(TT_, 1, 16, 2);          \
        else                                   \
            BITQ_MFMA(TT_, 1, 8, 2);           \
    } while (0)
    switch (TT) {
        case 1:
            if (tall16)
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

// Fused quantizer + GEMV of one token (XQ = 1: bf16 x, 2: fp32 x).  The host
// admits K <= kMaxFusedK, so the plan's blocks per lane (at most 4 with 8 rows
// per workgroup, 8 with 16) keep the whole k range in one round; other
// combinations are not built and return false.
template <int FMT, int P, int BPL, int RG, int XQ>
static void launch_fq_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* x, float* y,
                          hipStream_t st) {
    const int tiles = static_cast<int>(L.Tn);
    const int groups = 8 * (64 / RG) * ((tiles + 7) / 8);  // as launch_nr_bpl
    const int abits = d.fmt == BITQ_WNAM ? d.abits : 8;
    hipLaunchKernelGGL((gemv_bits_nr_kernel<FMT, P, false, BPL, RG, true, XQ>), dim3(groups), dim3(256), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, L.off_c1, static_cast<const uint8_t*>(x),
                       static_cast<size_t>(0), static_cast<size_t>(0), 1, d.N, d.K, static_cast<int>(L.Tb), abits,
                       L.off_c2, static_cast<size_t>(0), 0, y);
}

template <int FMT, int P, int RG, int XQ>
static bool launch_fq_rg(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                         float* y, hipStream_t st) {
    if (L.Tb > static_cast<size_t>(256 / RG) * pl.blocks_per_split) return false;  // not one round
    constexpr bool wnam = FMT == BITQ_WNAM;
    switch (pl.blocks_per_split) {
        case 1: launch_fq_bpl<FMT, P, 1, RG, XQ>(d, L, w, x, y, st); return true;
        case 2: launch_fq_bpl<FMT, P, 2, RG, XQ>(d, L, w, x, y, st); return true;
        case 3:
            if constexpr (!wnam) {
                launch_fq_bpl<FMT, P, 3, RG, XQ>(d, L, w, x, y, st);
                return true;
            }
            return false;
        case 4: launch_fq_bpl<FMT, P, 4, RG, XQ>(d, L, w, x, y, st); return true;
        case 6:
            if constexpr (!wnam && RG == 16) {
                launch_fq_bpl<FMT, P, 6, RG, XQ>(d, L, w, x, y, st);
                return true;
            }
            return false;
        case 8:
            if constexpr (RG == 16) {
                launch_fq_bpl<FMT, P, 8, RG, XQ>(d, L, w, x, y, st);
                return true;
            }
            return false;
        default: return false;
    }
}

template <int FMT, int P, int XQ>
static bool launch_fq_fmt(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                          float* y, hipStream_t st) {
    return pl.rows_per_wg == 8 ? launch_fq_rg<FMT, P, 8, XQ>(d, pl, L, w, x, y, st)
                               : launch_fq_rg<FMT, P, 16, XQ>(d, pl, L, w, x, y, st);
}

template <int XQ>
static bool launch_fq(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                      float* y, hipStream_t st) {
    switch (d.fmt) {
        case BITQ_TERNARY: return launch_fq_fmt<BITQ_TERNARY, 2, XQ>(d, pl, L, w, x, y, st);
        case BITQ_W2A8: return launch_fq_fmt<BITQ_W2A8, 2, XQ>(d, pl, L, w, x, y, st);
        case BITQ_BVSR4: return launch_fq_fmt<BITQ_BVSR4, 4, XQ>(d, pl, L, w, x, y, st);
        case BITQ_WNAM:
            switch (d.planes) {
                case 1: return launch_fq_fmt<BITQ_WNAM, 1, XQ>(d, pl, L, w, x, y, st);
                case 2: return launch_fq_fmt<BITQ_WNAM, 2, XQ>(d, pl, L, w, x, y, st);
                case 3: return launch_fq_fmt<BITQ_WNAM, 3, XQ>(d, pl, L, w, x, y, st);
                case 4: return launch_fq_fmt<BITQ_WNAM, 4, XQ>(d, pl, L, w, x, y, st);
                default: return false;
            }
        default: return false;
    }
}

int launch_gemv_fused(const bitq_wdesc& d, const Plan& pl, const void* w, const void* x, int x_dtype, float* y,
                      void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool built = x_dtype == BITQ_DT_BF16 ? launch_fq<1>(d, pl, L, w, x, y, st) : launch_fq<2>(d, pl, L, w, x, y, st);
    if (!built) return kLaunchNotBuilt;
    return static_cast<int>(hipGetLastError());
}

int launch_gemv_int(const bitq_wdesc& d, const Plan& pl, const void* w, const void* act, int M, float* y,
                    void* ws, uint32_t flags, void* stream) {
    BlobLayout L = blob_layout(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool acc = (flags & BITQ_F_ACC_INT32) != 0;
    (void)ws;
    if (pl.mfma) {
        acc ? launch_mfma_fmt<true>(d, L, w, act, M, y, st) : launch_mfma_fmt<false>(d, L, w, act, M, y, st);
        return static_cast<int>(hipGetLastError());
    }
    switch (d.fmt) {
        case BITQ_TERNARY:
            acc ? launch_nr<BITQ_TERNARY, 2, true>(d, pl, L, w, act, M, y, st)
                : launch_nr<BITQ_TERNARY, 2, false>(d, pl, L, w, act, M, y, st);
            break;
        case BITQ_HGF:  // the exact partials Y are the ternary kernel's
            acc ? launch_nr<BITQ_TERNARY, 2, true>(d, pl, L, w, act, M, y, st)
                : launch_nr<BITQ_HGF, 2, false>(d, pl, L, w, act, M, y, st);
            break;
        case BITQ_W2A8:
            acc ? launch_nr<BITQ_W2A8, 2, true>(d, pl, L, w, act, M, y, st)
                : launch_nr<BITQ_W2A8, 2, false>(d, pl, L, w, act, M, y, st);
            break;
        case BITQ_WNAM:
            acc ? launch_wnam<true>(d, pl, L, w, act, M, y, st) : launch_wnam<false>(d, pl, L, w, act, M, y, st);
            break;
        default:
            acc ? launch_nr<BITQ_BVSR4, 4, true>(d, pl, L, w, act, M, y, st)
                : launch_nr<BITQ_BVSR4, 4, false>(d, pl, L, w, act, M, y, st);
            break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace bitq
