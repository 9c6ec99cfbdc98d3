// XNOR+popcount GEMV of libbitq: SIGN1 weights times binary activations.
#include <hip/hip_runtime.h>

#include "bitq_device.h"

namespace bitq {

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

template <bool ACC, int BPL>
static void launch_xnor_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M,
                            float* y, hipStream_t st) {
    constexpr int RG = 8;
    BinActLayout A = binact_layout(M, d.K);
    const int tiles = static_cast<int>(L.Tn);
    const int groups = xcd_row_groups(tiles, RG);
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

}  // namespace bitq
