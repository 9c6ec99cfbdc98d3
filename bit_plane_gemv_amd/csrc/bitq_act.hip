// Activation kernels of libbitq: the per-token int8 / m-bit quantizer (with
// the HGF correction's down projection) and the sign binarizer of the fully
// binary path.  Also the per-device gfx950 check used by the host code.
#include <atomic>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "bitq_device.h"

namespace bitq {

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

// Where the matrix-core kernel reads input i of word w (inputs 32w ..
// 32w + 31) of token m = 16t + j in the permuted copy qm of q, with T token
// tiles of 16: in block b = w / 4, word g = w % 4 of the block, input
// 8e + 2c + s of the word sits at byte
//   ((b T + t) 2 + s) 1024 + (16 g + j) 16 + 4c + e,
// so a wave's operand load for one block, token tile and k step (lane
// 16 g + j taking 16 bytes) is 1 KB contiguous.
__device__ __forceinline__ size_t qm_off(int m, int w, int i, int T) {
    const int b = w >> 2, g = w & 3, t = m >> 4, j = m & 15;
    return (static_cast<size_t>(b * T + t) * 2 + (i & 1)) * 1024 + static_cast<size_t>(16 * g + j) * 16 +
           4 * ((i >> 1) & 3) + (i >> 3);
}

// amax of a long row (K > kAmaxOnePassK) in a launch of its own: one
// workgroup of 1024 lanes per token, four 16-byte loads in flight per lane.
// The quantizer then reads only its own inputs instead of the whole row.
template <int DT>
__global__ __launch_bounds__(1024) void act_amax_kernel(const void* __restrict__ x, int K, float* __restrict__ amax) {
    constexpr int VEC = (DT == BITQ_DT_F32) ? 4 : 8;
    __shared__ float s_red[16];
    const int m = blockIdx.x, tid = threadIdx.x;
    const uint4* xv = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                     static_cast<size_t>(m) * K * (DT == BITQ_DT_F32 ? 4 : 2));
    const int nvec = K / VEC;
    float a = 0.0f;
    for (int i0 = 0; i0 < nvec; i0 += 4096) {
        uint4 v[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int i = i0 + tid + 1024 * h;
            v[h] = i < nvec ? xv[i] : make_uint4(0, 0, 0, 0);   // zeros do not change the max of |x|
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t u[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (DT == BITQ_DT_F32)
                    a = fmaxf(a, fabsf(__uint_as_float(u[e])));
                else
                    a = fmaxf(a, fmaxf(fabsf(__uint_as_float(u[e] << 16)), fabsf(__uint_as_float(u[e] & 0xFFFF0000u))));
            }
        }
    }
    a = wave_max(a);
    if ((tid & 63) == 0) s_red[tid >> 6] = a;
    __syncthreads();
    if (tid == 0) {
        float t = s_red[0];
        for (int w = 1; w < 16; ++w) t = fmaxf(t, s_red[w]);
        amax[m] = t;
    }
}

// Pointers to the sections of an activation buffer (include/bitq.h).
struct ActOut {
    uint32_t* planes;
    int32_t* S;
    int8_t* q;
    int8_t* qm;
    float* d;
    float* amax;
    float* h;
};

// PRE: amax comes from act_amax_kernel (out.amax, written by the previous
// launch on the stream) and the workgroup reads only its own 256 inputs.
template <int DT, int RANK, bool PRE, int HOLD = 4>
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ x, int K, int Kw, float qmax,
                                                        ActOut out, const uint8_t* __restrict__ blob, size_t off_at,
                                                        int Kp, unsigned long long* __restrict__ ws) {
    static_assert(!(PRE && RANK > 0), "the HGF activation step has K <= 16128: one pass");
    constexpr int VEC = (DT == BITQ_DT_F32) ? 4 : 8;  // inputs per 16-byte load
    // HOLD: 16-byte loads per thread in flight together in the one-pass amax
    // (8 for rows of more than 1024 of them: the whole row in one batch
    // instead of a batch of 4 and a loop of dependent loads)
    __shared__ float s_red[4];
    __shared__ float s_slice[256];                     // this workgroup's 256 inputs
    const int m = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t xrow = static_cast<size_t>(m) * K;
    const uint4* xv = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                     xrow * (DT == BITQ_DT_F32 ? 4 : 2));
    const int nvec = K / VEC;           // K is a multiple of 32
    const int lo = 256 * blockIdx.x;    // first input of this workgroup

    float amax = 0.0f;
    auto take = [&](int i, const uint4& u, bool reduce) {
        const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v0, v1;
            if (DT == BITQ_DT_F32) {
                v0 = __uint_as_float(a[e]);
                if (reduce) amax = fmaxf(amax, fabsf(v0));
                const int k = i * VEC + e;
                if (k >= lo && k < lo + 256) s_slice[k - lo] = v0;
            } else {
                v0 = __uint_as_float(a[e] << 16);
                v1 = __uint_as_float(a[e] & 0xFFFF0000u);
                if (reduce) amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
                const int k = i * VEC + 2 * e;
                if (k >= lo && k < lo + 256) {
                    s_slice[k - lo] = v0;
                    s_slice[k + 1 - lo] = v1;
                }
            }
        }
    };
    if constexpr (PRE) {
        // ---- amax from the separate pass; this workgroup's inputs to LDS
        const int i = lo / VEC + tid;
        if (tid < 256 / VEC && i < nvec) take(i, xv[i], false);
        amax = out.amax[m];
        __syncthreads();
    } else {
        // ---- one pass over the row: amax, and this workgroup's inputs to LDS
        {
            uint4 hold[HOLD];
#pragma unroll
            for (int h = 0; h < HOLD; ++h) {  // all loads of the first pass in flight together
                const int i = tid + 256 * h;
                hold[h] = (i < nvec) ? xv[i] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int h = 0; h < HOLD; ++h)
                if (tid + 256 * h < nvec) take(tid + 256 * h, hold[h], true);
        }
        for (int i = tid + 256 * HOLD; i < nvec; i += 256) take(i, xv[i], true);
        amax = wave_max(amax);
        if (lane == 0) s_red[wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        if (blockIdx.x == 0 && tid == 0) out.amax[m] = amax;
    }
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
                        &out.h[static_cast<size_t>(m) * RANK + tid]);
        }
    }
    float s = 0.0f;
    if (amax > 0.0f) s = __fdiv_rn(qmax, amax);
    if (blockIdx.x == 0 && tid == 0) out.d[m] = (amax > 0.0f) ? __fdiv_rn(amax, qmax) : 0.0f;

    // ---- this wave's 64 inputs = words w0 and w0 + 1
    const int w0 = 8 * blockIdx.x + 2 * wave;
    if (w0 >= Kw) return;
    const int k = 32 * w0 + lane;
    int qi = 0;
    if (k < K && amax > 0.0f) {
        const float r = rintf(__fmul_rn(s_slice[k - lo], s));
        qi = static_cast<int>(fminf(fmaxf(r, -qmax), qmax));
    }
    out.q[static_cast<size_t>(m) * (Kw * 32) + k] = static_cast<int8_t>(qi);
    out.qm[qm_off(m, w0 + (lane >> 5), lane & 31, (static_cast<int>(gridDim.y) + 15) >> 4)] = static_cast<int8_t>(qi);
    // planes: lane j (< 8) keeps plane j of word w0, lane 8 + j of word w0 + 1
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t b = __ballot((qi >> j) & 1);
        if (lane == j) mine = static_cast<uint32_t>(b);
        if (lane == 8 + j) mine = static_cast<uint32_t>(b >> 32);
    }
    if (lane < 16) out.planes[(static_cast<size_t>(m) * Kw + w0) * 8 + lane] = mine;
    // group sums of the two words: reductions inside each half of the wave
    int sum = qi;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) out.S[static_cast<size_t>(m) * Kw + w0] = sum;
    if (lane == 32) out.S[static_cast<size_t>(m) * Kw + w0 + 1] = sum;
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

static ActOut act_out(void* act, const ActLayout& A) {
    uint8_t* base = static_cast<uint8_t*>(act);
    ActOut o;
    o.planes = reinterpret_cast<uint32_t*>(base + A.off_planes);
    o.S = reinterpret_cast<int32_t*>(base + A.off_S);
    o.q = reinterpret_cast<int8_t*>(base + A.off_q);
    o.qm = reinterpret_cast<int8_t*>(base + A.off_qm);
    o.d = reinterpret_cast<float*>(base + A.off_d);
    o.amax = reinterpret_cast<float*>(base + A.off_amax);
    o.h = reinterpret_cast<float*>(base + A.off_h);
    return o;
}

// Workgroups from which the amax of each token is taken by a launch of its
// own (one read of the row) rather than by every workgroup of the token:
// 64 tokens x 11008 inputs (2752 workgroups) 25.8 -> 23.9 us per W2A8
// 4096x11008 step; with 64 x 4096 (1024 workgroups) the extra launch costs
// more than the repeated reads save (14.7 -> 16.9 us).
constexpr int64_t kAmaxPassMinWorkgroups = 2048;

template <int DT>
static void launch_quant_plain(const void* x, int M, int K, int Kw, float qmax, const ActOut& o, hipStream_t st) {
    const dim3 grid((Kw + 7) / 8, M);
    if (K > kAmaxOnePassK || static_cast<int64_t>(grid.x) * M >= kAmaxPassMinWorkgroups) {
        hipLaunchKernelGGL((act_amax_kernel<DT>), dim3(M), dim3(1024), 0, st, x, K, o.amax);
        hipLaunchKernelGGL((quant_act_kernel<DT, 0, true>), grid, dim3(256), 0, st, x, K, Kw, qmax, o,
                           static_cast<const uint8_t*>(nullptr), static_cast<size_t>(0), 0,
                           static_cast<unsigned long long*>(nullptr));
    } else if (K / (DT == BITQ_DT_F32 ? 4 : 8) > 1024) {
        hipLaunchKernelGGL((quant_act_kernel<DT, 0, false, 8>), grid, dim3(256), 0, st, x, K, Kw, qmax, o,
                           static_cast<const uint8_t*>(nullptr), static_cast<size_t>(0), 0,
                           static_cast<unsigned long long*>(nullptr));
    } else {
        hipLaunchKernelGGL((quant_act_kernel<DT, 0, false>), grid, dim3(256), 0, st, x, K, Kw, qmax, o,
                           static_cast<const uint8_t*>(nullptr), static_cast<size_t>(0), 0,
                           static_cast<unsigned long long*>(nullptr));
    }
}

int launch_quantize_act(const void* x, int x_dtype, int M, int K, int abits, void* act, void* stream) {
    ActLayout A = act_layout(M, K);
    const ActOut o = act_out(act, A);
    const int Kw = static_cast<int>(A.Kw);
    const float qmax = static_cast<float>((1 << (abits - 1)) - 1);  // 127 for int8
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == BITQ_DT_F32)
        launch_quant_plain<BITQ_DT_F32>(x, M, K, Kw, qmax, o, st);
    else
        launch_quant_plain<BITQ_DT_BF16>(x, M, K, Kw, qmax, o, st);
    return static_cast<int>(hipGetLastError());
}

template <int DT, int RANK>
static void launch_quant_hgf(dim3 grid, hipStream_t st, const void* x, int K, int Kw, const ActOut& o,
                             const uint8_t* blob, size_t off_at, int Kp, unsigned long long* ws) {
    hipLaunchKernelGGL((quant_act_kernel<DT, RANK, false>), grid, dim3(256), 0, st, x, K, Kw, 127.0f, o, blob,
                       off_at, Kp, ws);
}

template <int DT>
static void launch_quant_hgf_rank(int rank, dim3 grid, hipStream_t st, const void* x, int K, int Kw,
                                  const ActOut& o, const uint8_t* blob, size_t off_at, int Kp,
                                  unsigned long long* ws) {
    switch (rank) {
        case 8: launch_quant_hgf<DT, 8>(grid, st, x, K, Kw, o, blob, off_at, Kp, ws); break;
        case 16: launch_quant_hgf<DT, 16>(grid, st, x, K, Kw, o, blob, off_at, Kp, ws); break;
        case 32: launch_quant_hgf<DT, 32>(grid, st, x, K, Kw, o, blob, off_at, Kp, ws); break;
        default: launch_quant_hgf<DT, 64>(grid, st, x, K, Kw, o, blob, off_at, Kp, ws); break;
    }
}

int launch_quantize_act_hgf(const void* x, int x_dtype, int M, int K, int rank, const void* w, const BlobLayout& L,
                            void* act, void* ws, void* stream) {
    ActLayout A = act_layout(M, K, rank);
    const ActOut o = act_out(act, A);
    const int Kw = static_cast<int>(A.Kw);
    const dim3 grid((Kw + 7) / 8, M);
    const uint8_t* blob = static_cast<const uint8_t*>(w);  // A^T and amax_a are read by the kernel
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* wsw = static_cast<unsigned long long*>(ws);
    const int Kp = static_cast<int>(L.Kp);
    if (x_dtype == BITQ_DT_F32)
        launch_quant_hgf_rank<BITQ_DT_F32>(rank, grid, st, x, K, Kw, o, blob, L.off_c1, Kp, wsw);
    else
        launch_quant_hgf_rank<BITQ_DT_BF16>(rank, grid, st, x, K, Kw, o, blob, L.off_c1, Kp, wsw);
    return static_cast<int>(hipGetLastError());
}

// ------------------------------------------- the no-allocation activation step
// Scratch of bitq_quantize_act_hgf_noalloc: the 64-bit fixed-point words of
// the HGF down projection (one per token and rank column), for the largest
// call (64 tokens x rank 64 = 32 KB).  Each GPU the library runs on holds
// its own copy until the process ends.  In host code the name `scratch` is
// not a device address: the address comes from hipGetSymbolAddress, once
// per device, and only that address is passed to kernels.
static __device__ __align__(256) unsigned long long scratch[kNoAllocScratchWords];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device: the device address of `scratch`, or null before set-up
}  // namespace

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned long long* __restrict__ w, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) w[i] = 0ull;
}

int noalloc_scratch(void** ptr, void* stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= 64) return static_cast<int>(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
        // The words start at zero (device globals are zero-initialized, and
        // every completed call leaves them zero); cleared once more here at
        // set-up with a fill kernel, which is also valid under graph capture.
        hipLaunchKernelGGL(zero_words_kernel, dim3((kNoAllocScratchWords + 255) / 256), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<unsigned long long*>(p),
                           kNoAllocScratchWords);
        e = hipGetLastError();
        if (e != hipSuccess) return static_cast<int>(e);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int launch_quantize_act_hgf_noalloc(const void* x, int x_dtype, int M, int K, int rank, const void* w,
                                    const BlobLayout& L, void* act, void* stream) {
    void* ws = nullptr;
    const int e = noalloc_scratch(&ws, stream);
    if (e) return e;
    return launch_quantize_act_hgf(x, x_dtype, M, K, rank, w, L, act, ws, stream);
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

}  // namespace bitq
