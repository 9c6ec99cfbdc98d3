// AND+popcount GEMV of libbitq for integer activations (TERNARY, W2A8,
// BVSR4, WNAM, HGF): M = 1, the VALU small-M path, and the variant with the
// activation quantizer fused into the prologue.
#include <hip/hip_runtime.h>

#include "bitq_device.h"

namespace bitq {

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
//   BVSR4 ([BVSR]): per 32-group P_k = sum_i beta_k[i] q_i (below: 4-bit
//           dot products), y += b S32 + sum_k c_k P_k with (c, b) = cache[idx]

// BVSR4 on the 4-bit dot products of gfx950 instead.  P_k = sum_i beta_k[i]
// q_i is a masked sum of the group's activations; with q = 16 (q >> 4) +
// (q & 15) split into a signed high and an unsigned low nibble, and the four
// bitvectors stored nibble-interleaved (plane word s of a group: nibble e =
// the 4 bits beta_0..3 of one of its inputs 8 s .. 8 s + 7), the mask
// W & (0x11111111 << k) holds 2^k beta_k per nibble, and one v_dot8_u32_u4
// (low nibbles) plus one v_dot8_i32_i4 (high nibbles) take 8 inputs of
// bitvector k: 2^k P_k = lo + 16 hi (k = 3: lo - 16 hi, the signed nibble
// 8 being -8).  Per group and bitvector 4 masks and 8 dot products replace
// the 8 ANDs, 8 popcounts and plane combine of the AND+popcount form; the
// same integer P_k comes out exactly.
//
// Low- and high-nibble words of 8 inputs from two words of 4 activation bytes
// (inputs 0..3 in a, 4..7 in b): nibble e holds input (e >> 1) + 4 (e & 1).
// v_dot8_i32_i4 in its three-operand form (the compiler's accumulate-in-place
// form needs a register zeroed first for each chain)
__device__ __forceinline__ int sdot8_acc(uint32_t a, uint32_t b, int c) {
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ int sdot8_first(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ void nibble_words(uint32_t a, uint32_t b, uint32_t& lo, uint32_t& hi) {
    lo = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
    hi = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
}

// The waves' partials of row r added in a fixed order (pairs, then pairs of
// pairs, then the two halves of eight waves).
template <typename T, int W>
__device__ __forceinline__ T wave_sum(const T (&s)[W][16], int r) {
    T v = (s[0][r] + s[1][r]) + (s[2][r] + s[3][r]);
    if constexpr (W == 8) v += (s[4][r] + s[5][r]) + (s[6][r] + s[7][r]);
    return v;
}

// ================================= AND+popcount GEMV, whole k per workgroup
// No hand-off between workgroups: a workgroup (NT = 256 threads; 512 for the
// fused quantizer with 16 rows and a long k range) owns RG rows
// (16 or 8) and the whole k range.  Thread (g, r) = (tid / RG, tid % RG)
// takes row r of the group and the k blocks b = g + G j (j < BPL, G = NT/RG
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
//
// Arguments: what the prologue needs comes first (the first 56 bytes arrive
// preloaded in scalar registers); activation-buffer offsets are 32-bit (the
// host bounds that buffer far below 4 GB).
template <int FMT, int P, bool ACC, int BPL, int RG, bool ONE, int XQ = 0, int NT = 256>
__global__ __launch_bounds__(NT) void gemv_bits_nr_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                           size_t off_c1, const uint8_t* __restrict__ act,
                                                           uint32_t act_off_S, uint32_t act_off_q, int N, int Tb, int M,
                                                           int K, uint32_t act_off_d, int abits, size_t off_c2,
                                                           uint32_t act_off_h, int rank, float* __restrict__ y) {
    constexpr bool TERN = FMT == BITQ_TERNARY || FMT == BITQ_HGF;  // ternary planes
    constexpr bool LORA = FMT == BITQ_HGF && !ACC;                 // the correction epilogue
    constexpr int G = NT / RG;     // k-groups: lanes that share a row
    constexpr int NWV = NT / 64;   // waves
    static_assert(NT == 256 || (NT == 512 && RG == 16 && (XQ != 0 || FMT == BITQ_BVSR4)),
                  "512 lanes: 16 rows, fused quantizer or BVSR4");
    constexpr int Q = 64 / RG;     // row groups per 64-row tile
    constexpr int NBW = G * BPL;   // k blocks per round
    constexpr int BSTR = 36;       // LDS words per block: 32 + 4 padding, so up to
                                   // 8 k-groups of a wave hit disjoint banks
    // Activation staging goes straight from global memory into LDS
    // (global_load_lds_dwordx4: lane l of a wave fills the 16-byte slot l of
    // the wave's destination), in whole passes of 256 lanes.  A block takes 9
    // slots: its 8 plane uint4 and one slot of padding.
    constexpr int SLOT_PASSES = (NBW * 9 + NT - 1) / NT;
    constexpr int S_PASSES = (NBW + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) uint32_t s_act[SLOT_PASSES * NT * 4];
    __shared__ __attribute__((aligned(16))) int32_t s_S[S_PASSES * NT * 4];
    __shared__ float4 s_cache[FMT == BITQ_BVSR4 ? 512 : 1];
    // HGF: B^T rows of the group (RG x rank fp16, rank <= 64: RG 8 slots of
    // 16 bytes) and h of the current token (rank floats; the copy fills one
    // 16-byte slot per lane of a wave: 64 slots).  Declared as one word
    // array: with vector-typed arrays of template-dependent size here, this
    // compiler drops the kernel's host-side stub.
    __shared__ __attribute__((aligned(16))) uint32_t s_lora[FMT == BITQ_HGF ? (RG * 8 + 64) * 4 : 4];
    uint4* const s_bt = reinterpret_cast<uint4*>(s_lora);
    float4* const s_h = reinterpret_cast<float4*>(s_lora + RG * 8 * 4);
    __shared__ float s_red[NWV][16];
    __shared__ int32_t s_redi[NWV][16];
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
    constexpr bool NIBX = FMT == BITQ_BVSR4;
    constexpr int XST = NIBX && !FQ ? (NBW * 8 + NT - 1) / NT : 1;  // q loads per lane and round
    uint4 xs[XST];
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
    //
    // BVSR4 stages nibble words instead of planes: q of the round goes into
    // registers (16 inputs per lane and load) and, once it has landed,
    // store_nibbles writes each 8 inputs' low-nibble word (unsigned q & 15)
    // and high-nibble word (signed q >> 4) to the block's LDS words
    // 8 w + s and 8 w + 4 + s (32-group w, sub-word s).
    auto stage = [&](int m, int b_base) __attribute__((always_inline)) {
        const int last = min(NBW, NB - b_base) - 1;  // last real block of the round
        if constexpr (NIBX) {
            const uint4* qsrc = reinterpret_cast<const uint4*>(act + act_off_q) +
                                (static_cast<size_t>(m) * NB + b_base) * 8;  // q [M][Kp]
#pragma unroll
            for (int v = 0; v < XST; ++v) {
                const int ch = tid + NT * v;
                xs[v] = qsrc[8 * min(ch >> 3, last) + (ch & 7)];
            }
        } else {
            const uint4* src = reinterpret_cast<const uint4*>(aplanes) + (static_cast<size_t>(m) * Kw + 4 * b_base) * 2;
#pragma unroll
            for (int v = 0; v < SLOT_PASSES; ++v) {
                const int slot = tid + NT * v;
                const int blk = slot / 9, part = slot - 9 * blk;
                __builtin_amdgcn_global_load_lds(src + 8 * min(blk, last) + min(part, 7),
                                                 reinterpret_cast<uint4*>(s_act) + NT * v + 64 * wave, 16, 0, 0);
            }
        }
        const int4* srcS = reinterpret_cast<const int4*>(aS + static_cast<size_t>(m) * Kw + 4 * b_base);
#pragma unroll
        for (int v = 0; v < S_PASSES; ++v)
            __builtin_amdgcn_global_load_lds(srcS + min(tid + NT * v, last),
                                             reinterpret_cast<int4*>(s_S) + NT * v + 64 * wave, 16, 0, 0);
        if (LORA && b_base == 0 && wave_u == 0) {  // h[m]: rank / 4 16-byte slots
            const float4* hsrc = reinterpret_cast<const float4*>(act + act_off_h) + static_cast<size_t>(m) * (rank / 4);
            // (wave_u is 0 here; a destination computed from it, rather than
            // the constant s_h, avoids a crash of this compiler's SGPR-copy pass)
            __builtin_amdgcn_global_load_lds(hsrc + min(tid, rank / 4 - 1), s_h + 64 * wave_u, 16, 0, 0);
        }
    };

    // (the use of xs waits for its loads, and only for them: they are issued
    // ahead of the weight stream)
    auto store_nibbles = [&]() __attribute__((always_inline)) {
        if constexpr (NIBX) {
#pragma unroll
            for (int v = 0; v < XST; ++v) {
                const int ch = tid + NT * v;
                if (XST * NT == NBW * 8 || ch < NBW * 8) {
                    const int blk = ch >> 3, w = (ch & 7) >> 1, s0 = 2 * (ch & 1);
                    uint32_t lo0, hi0, lo1, hi1;
                    nibble_words(xs[v].x, xs[v].y, lo0, hi0);
                    nibble_words(xs[v].z, xs[v].w, lo1, hi1);
                    uint32_t* dst = &s_act[blk * BSTR + 8 * w + s0];
                    *reinterpret_cast<uint2*>(dst) = make_uint2(lo0, lo1);
                    *reinterpret_cast<uint2*>(dst + 4) = make_uint2(hi0, hi1);
                }
            }
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
            if (NT == 256 || wave_u < 4)  // 2048 4-byte slots: the first four waves
                __builtin_amdgcn_global_load_lds(cache + 5 * e + min(f, 4),
                                                 reinterpret_cast<float*>(s_cache) + 256 * v + 64 * wave_u, 4, 0, 0);
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
    constexpr int XCPT = FQ ? NBW * 16 / NT : 1;
    constexpr int XLPC = XQ == 2 ? 2 : 1;
    static_assert(!FQ || (NBW * 16) % NT == 0, "whole chunks per thread");
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
            const int c = min(tid + NT * i, nch - 1);
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
        __shared__ float s_amax[NWV];
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
        if constexpr (NWV == 8) am = fmaxf(am, fmaxf(fmaxf(s_amax[4], s_amax[5]), fmaxf(s_amax[6], s_amax[7])));
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
            const int c = tid + NT * i;
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
            S += static_cast<int>(quad_swap<0xB1>(static_cast<uint32_t>(S)));
            S += static_cast<int>(quad_swap<0x4E>(static_cast<uint32_t>(S)));
            const int word = c >> 2;  // 32-input word of the round: block word / 4, its word word % 4
            uint32_t* dst = &s_act[(word >> 2) * BSTR + 8 * (word & 3)];
            if ((tid & 3) == 0) s_S[word] = S;
            if constexpr (NIBX) {  // chunk c = sub-word c % 4 of its word
                uint32_t nlo, nhi;
                nibble_words(lo, hi, nlo, nhi);
                dst[c & 3] = nlo;
                dst[4 + (c & 3)] = nhi;
                continue;
            }
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
            dst[pl] = lo;
            dst[pl + 4] = hi;
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
        if constexpr (NIBX && ONE) {
            // the weights stay in registers across the tokens: without this
            // empty asm the compiler hoists every bitvector mask out of the
            // token loop (256 registers) and spills
#pragma unroll
            for (int j = 0; j < BPL; ++j)
#pragma unroll
                for (int p = 0; p < P; ++p)
                    asm volatile("" : "+v"(wv[j][p].x), "+v"(wv[j][p].y), "+v"(wv[j][p].z), "+v"(wv[j][p].w));
        }
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
                store_nibbles();
                barrier_after_loads<kWeightLoads>();
            } else if (first) {
                if (!FQ) {  // copies issued in the prologue
                    store_nibbles();
                    barrier_after_loads<kWeightLoads>();
                }
            } else {
                stage(m, b_base);
                store_nibbles();
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
                        // nibble words of the group's sub-words sw = 0..3
                        const uint4 x0 = *reinterpret_cast<const uint4*>(xa + 8 * w);      // q & 15
                        const uint4 x1 = *reinterpret_cast<const uint4*>(xa + 8 * w + 4);  // q >> 4
                        const uint32_t xl[4] = {x0.x, x0.y, x0.z, x0.w}, xh[4] = {x1.x, x1.y, x1.z, x1.w};
                        uint32_t tl[4] = {0u, 0u, 0u, 0u};
                        int th[4] = {0, 0, 0, 0};
#pragma unroll
                        for (int sw = 0; sw < 4; ++sw) {
                            const uint32_t ws = (&wv[j][sw].x)[w];
#pragma unroll
                            for (int k = 0; k < 4; ++k) {
                                const uint32_t mk = ws & (0x11111111u << k);  // nibbles 2^k beta_k
                                tl[k] = __builtin_amdgcn_udot8(mk, xl[sw], tl[k], false);
                                th[k] = sw == 0 ? sdot8_first(mk, xh[sw]) : sdot8_acc(mk, xh[sw], th[k]);
                            }
                        }
                        // T_k = 2^k P_k (as a signed nibble, 2^3 reads -8)
                        int Tk[4];
#pragma unroll
                        for (int k = 0; k < 3; ++k) Tk[k] = static_cast<int>(tl[k]) + 16 * th[k];
                        Tk[3] = static_cast<int>(tl[3]) - 16 * th[3];
                        const int gi = 4 * b + w;
                        if (ACC) {
                            const int G = K / 32;  // groups of the real (unpadded) K
                            int4* dst = reinterpret_cast<int4*>(y) + (static_cast<size_t>(m) * N + n) * G + gi;
                            if (n < N && gi < G) *dst = make_int4(Tk[0], Tk[1] >> 1, Tk[2] >> 2, Tk[3] >> 3);
                        } else {
                            // the packed cache holds c_k 2^-k: c_k P_k exactly as (c_k 2^-k) T_k
                            const int id = (cw >> (8 * w)) & 0xFF;
                            const float4 c = s_cache[2 * id];
                            const float bo = s_cache[2 * id + 1].x;
                            const float S32 = static_cast<float>(s_S[4 * bl + w]);
                            yacc += bo * S32 + c.x * static_cast<float>(Tk[0]) + c.y * static_cast<float>(Tk[1]) +
                                    c.z * static_cast<float>(Tk[2]) + c.w * static_cast<float>(Tk[3]);
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
                    wave_sum(s_redi, r);
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
                float tot = wave_sum(s_red, r);
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

template <int FMT, int P, bool ACC, int BPL, int RG, int NT = 256>
static void launch_nr_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M,
                          float* y, hipStream_t st) {
    ActLayout A = act_layout(M, d.K, d.rank);
    // 64/RG row groups per 64-row tile, tiles dealt round-robin to the 8 XCDs:
    // the grid is padded to whole rounds of 8 tiles (extra workgroups exit)
    const int tiles = static_cast<int>(L.Tn);
    const int groups = xcd_row_groups(tiles, RG);
    const bool one = L.Tb <= (NT / RG) * BPL;  // the whole k range in one round
    auto kern = one ? gemv_bits_nr_kernel<FMT, P, ACC, BPL, RG, true, 0, NT>
                    : gemv_bits_nr_kernel<FMT, P, ACC, BPL, RG, false, 0, NT>;
    const int abits = d.fmt == BITQ_WNAM ? d.abits : 8;
    hipLaunchKernelGGL(kern, dim3(groups), dim3(NT), 0, st, static_cast<const uint8_t*>(w), L.off_c0, L.off_c1,
                       static_cast<const uint8_t*>(act), static_cast<uint32_t>(A.off_S), static_cast<uint32_t>(A.off_q),
                       d.N, static_cast<int>(L.Tb), M, d.K, static_cast<uint32_t>(A.off_d), abits, L.off_c2,
                       static_cast<uint32_t>(A.off_h), d.rank, y);
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
        if constexpr (FMT == BITQ_BVSR4 && RG == 16) {
            if (pl.waves_per_wg == 8) {  // 512 lanes, one round: 2 to 4 blocks per lane
                switch (pl.blocks_per_split) {
                    case 2: launch_nr_bpl<FMT, P, ACC, 2, RG, 512>(d, L, w, act, M, y, st); return;
                    case 3: launch_nr_bpl<FMT, P, ACC, 3, RG, 512>(d, L, w, act, M, y, st); return;
                    case 4: launch_nr_bpl<FMT, P, ACC, 4, RG, 512>(d, L, w, act, M, y, st); return;
                    default: break;
                }
            }
        }
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

// Fused quantizer + GEMV of one token (XQ = 1: bf16 x, 2: fp32 x).  The host
// admits K <= kMaxFusedK, so the plan's blocks per lane (at most 4 with 8 rows
// per workgroup, 8 with 16) keep the whole k range in one round; other
// combinations are not built and return false.
template <int FMT, int P, int BPL, int RG, int XQ, int NT = 256>
static void launch_fq_bpl(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* x, float* y,
                          hipStream_t st) {
    const int tiles = static_cast<int>(L.Tn);
    const int groups = xcd_row_groups(tiles, RG);  // as launch_nr_bpl
    const int abits = d.fmt == BITQ_WNAM ? d.abits : 8;
    hipLaunchKernelGGL((gemv_bits_nr_kernel<FMT, P, false, BPL, RG, true, XQ, NT>), dim3(groups), dim3(NT), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, L.off_c1, static_cast<const uint8_t*>(x), 0u, 0u, d.N,
                       static_cast<int>(L.Tb), 1, d.K, 0u, abits, L.off_c2, 0u, 0, y);
}

template <int FMT, int P, int RG, int XQ>
static bool launch_fq_rg(const bitq_wdesc& d, const Plan& pl, const BlobLayout& L, const void* w, const void* x,
                         float* y, hipStream_t st) {
    constexpr bool wnam = FMT == BITQ_WNAM;
    if constexpr (RG == 16) {
        if (pl.waves_per_wg == 8) {  // 512 lanes, 2 to 4 blocks per lane
            if (L.Tb > static_cast<size_t>(512 / RG) * pl.blocks_per_split) return false;
            switch (pl.blocks_per_split) {
                case 2: launch_fq_bpl<FMT, P, 2, RG, XQ, 512>(d, L, w, x, y, st); return true;
                case 3:
                    if constexpr (!wnam) {
                        launch_fq_bpl<FMT, P, 3, RG, XQ, 512>(d, L, w, x, y, st);
                        return true;
                    }
                    return false;
                case 4: launch_fq_bpl<FMT, P, 4, RG, XQ, 512>(d, L, w, x, y, st); return true;
                default: return false;
            }
        }
    }
    if (L.Tb > static_cast<size_t>(256 / RG) * pl.blocks_per_split) return false;  // not one round
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
    if (pl.mfma) return launch_gemm_mfma(d, w, act, M, y, flags, stream);
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
