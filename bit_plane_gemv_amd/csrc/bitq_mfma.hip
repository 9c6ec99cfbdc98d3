// Small-M GEMM of libbitq on the int8 matrix cores (TERNARY, W2A8, WNAM).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bitq_device.h"

namespace bitq {

// ============================== small-M GEMM on the int8 matrix cores
// With M tokens the AND+popcount work of the VALU kernel grows M-fold, so
// from two tokens on the contraction is compute-bound there.  The same
// integer contraction then goes to v_mfma_i32_16x16x64_i8:
//   D[16 rows][16 tokens] += A[16][64] B[64][16]
// with A = the weight codes unpacked from their bit planes to int8 and B =
// the int8 activations q ([ABQ] computes with the binary decomposition
// because its target has 1-bit tensor cores; gfx950 has int8 ones, so the
// planes are recombined into codes instead, each weight once per launch).
//
// Operand layout of the instruction (checked on the device): lane l holds 16
// int8 of A for row l % 16 and 16 int8 of B for column l % 16; byte e of the
// lanes with l / 16 = g meets byte e of the B lanes with the same g (one k
// position); D element i of lane l is row 4 (l / 16) + i, column l % 16.
// The k position of (g, e) is free as long as A and B agree.  Lane group g
// takes plane word g of each 128-input block (inputs 32 g .. 32 g + 31), so
// every lane loads one 4-byte word per plane and block and the 64 lanes read
// 256 contiguous bytes.
//
// Unpack.  The planes of the word are interleaved into 2-bit fields with
// one bit-field insert each: Z_s = (P0 >> s) with (P1 << (1 - s)) in the odd
// bits, so field f of Z_s holds the two low code bits of input 2 f + s.  Then
// register c of k-step s is (Z_s >> 2c) & 0x03030303, whose byte j is the
// code of input 8 j + 2 c + s (three and four planes: nibble fields built
// the same way, (Q >> 4i) & 0x0F0F0F0F).  A byte permute through a table
// maps each code to its operand byte: c - z of the row's zero point (W2A8,
// WNAM; the matrix cores then return A - z S128 itself, exactly), or the
// ternary value (fields p + 2m: 0 -> 0, 1 -> +1, 2 -> -1).  So a code costs
// about one VALU operation.  The activation buffer's qm section holds q in
// the same order (input 8j + 2c + s of a word at byte 4c + j of its half s),
// tiled so that the B operands of a wave's block, token tile and k step are
// one contiguous 16-byte-per-lane load.
//
// Work decomposition.  One workgroup per CU (grid = 256) owns a contiguous
// range of 16-row sub-tiles over the whole k range, up to kMfmaSubs of them
// per pass, and all M <= 16 TT tokens; its KW waves take the k blocks
// w, w + KW, ...  A workgroup reads q (M K bytes, from L2) once per pass
// and applies it to all its sub-tiles, so q costs about 256 M K bytes of L2
// reads per launch; the weights are read once.  Ranges are dealt so that
// the workgroups of one XCD (round-robin dispatch) hold adjacent rows and
// share their coefficient lines in one L2.  A wave issues the loads of C
// blocks together before computing them.  Per 128-group (W2A8, WNAM) the
// exact group sum becomes delta (A - z S128) in fp32, added in block order;
// TERNARY keeps int32 sums over all of k.  The waves' partials are then
// added in wave order through LDS: y does not depend on scheduling.
typedef int v4i32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (mask & a) | (~mask & b); }

// Code bytes of the 32 inputs of one plane word: r[4 s + c] byte j = code
// of input 8 j + 2 c + s.  TERNARY: w = (plus, minus), code p + 2m.
template <int P>
__device__ __forceinline__ void unpack_codes(const uint32_t (&w)[P], uint32_t (&r)[8]) {
    if constexpr (P <= 2) {
        const uint32_t hi = P == 2 ? w[1] : 0u;
        uint32_t z[2] = {bfi(0x55555555u, w[0], hi << 1), bfi(0x55555555u, w[0] >> 1, hi)};
        // (materialized here: otherwise the compiler folds the first mask
        // into the interleave and computes it twice)
        asm volatile("" : "+v"(z[0]), "+v"(z[1]));
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c) r[4 * s + c] = (z[s] >> (2 * c)) & 0x03030303u;
    } else {
        const uint32_t w3 = P == 4 ? w[3] : 0u;
        const uint32_t z[2] = {bfi(0x55555555u, w[0], w[1] << 1), bfi(0x55555555u, w[0] >> 1, w[1])};
        const uint32_t yv[2] = {bfi(0x55555555u, w[2], w3 << 1), bfi(0x55555555u, w[2] >> 1, w3)};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // nibble a of q[h] = code of input 4a + 2h + s (low two bits from
            // Z_s field 2a + h, high two from the same field of Y_s)
            const uint32_t q[2] = {bfi(0x33333333u, z[s], yv[s] << 2), bfi(0x33333333u, z[s] >> 2, yv[s])};
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i) r[4 * s + 2 * i + h] = (q[h] >> (4 * i)) & 0x0F0F0F0Fu;
        }
    }
}

// What one wave reads for one 128-input block besides its weights.
template <int P, int S, int TT, bool LOADC>
struct MfmaBlock {
    v4i32_t qv[2][TT];          // B operands of the two k steps
    uint32_t zr[LOADC ? S : 1];  // coefficient word of row li (its zero point)
    uint4 cz[LOADC ? S : 1];    // coefficient words of rows 4 g .. 4 g + 3 (their delta)
};

template <int FMT, int P, bool ACC, int TT, int KW, int C, int S>
__global__ __launch_bounds__(64 * KW) void gemm_mfma_kernel(const uint8_t* __restrict__ blob, size_t off_c0,
                                                            const uint8_t* __restrict__ act, size_t act_off_qm,
                                                            size_t act_off_d, int M, int N, int Tb, int nsub,
                                                            float* __restrict__ y) {
    static_assert(S == 1 || S == kMfmaSubs, "sub-tiles per pass");
    constexpr bool GRP = FMT != BITQ_TERNARY;  // per-128-group epilogue (W2A8, WNAM)
    constexpr bool LOADC = GRP && !ACC;        // coefficients needed (fold + delta)
    constexpr bool PERM = FMT == BITQ_TERNARY || (LOADC && P <= 3);  // codes through a byte table
    constexpr int NV = S * TT * 4;             // partial outputs per lane
    // the waves' partials; at least kOneWgPerCuLds bytes, so that no CU
    // holds a second workgroup while another CU holds none
    // (rows of 68 floats: the reads of the reduction below, 4 tokens x 16
    // consecutive rows per wave instruction, then hit 64 distinct banks)
    constexpr int KST = 68;
    constexpr int PART = KW * NV * KST;
    __shared__ float s_part_mem[PART * 4 > kOneWgPerCuLds ? PART : kOneWgPerCuLds / 4];
    float (*s_part)[NV][KST] = reinterpret_cast<float (*)[NV][KST]>(s_part_mem);

    // (the wave index through readfirstlane: the compiler then knows it is
    // uniform and keeps the block and tile arithmetic in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    // sub-tile range: the workgroups of XCD x (blockIdx % 8 = x) take the
    // ranges 32 x .. 32 x + 31 in order (nsub <= 2^16, grid <= 256)
    const uint32_t G = gridDim.x, ns_u = static_cast<uint32_t>(nsub);
    const uint32_t per = G / 8, rid = G % 8 == 0 ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    const int s_beg = static_cast<int>(ns_u * rid / G), s_end = static_cast<int>(ns_u * (rid + 1) / G);
    const int nbw = wave < Tb ? (Tb - wave + KW - 1) / KW : 0;  // k blocks of this wave
    const int Np = 16 * nsub;
    const int8_t* qm = reinterpret_cast<const int8_t*>(act + act_off_qm);
    const float* ad = reinterpret_cast<const float*>(act + act_off_d);
    // The step d of this thread's token of each tile in the final reduction
    // (token 16 tt + (tid / 16) % 16), loaded once instead of once per output
    // there (a dependent L2 round trip in every iteration).  With one token
    // tile it is loaded just before the reduction: loaded here, its register
    // made the first block's loads wait for it (1.05x slower at 4-16
    // tokens); with more tiles, here (1.02x faster than there at 64 tokens).
    float dtok[TT];
    if constexpr (TT > 1) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) dtok[tt] = ad[min(16 * tt + ((tid >> 4) & 15), M - 1)];
    }
    const float gamma = (FMT == BITQ_TERNARY && !ACC) ? *reinterpret_cast<const float*>(blob + off_c0) : 1.0f;
    const uint32_t* coef = reinterpret_cast<const uint32_t*>(blob + off_c0);
    // q is tiled for these loads (include/bitq.h): the operand of block b,
    // token tile tt and k step s2 is the 1 KB at ((b TT + tt) 2 + s2) 1024,
    // lane l taking bytes 16 l .. 16 l + 15, so every q load of a wave is
    // one contiguous KB.  (The earlier layout, token rows of Kp + 128 bytes,
    // made each load touch 16 cache lines, half of each: W2A8 11008x4096
    // took 15.9 us at M = 64, 9.6 us at M = 32, against 11.4 and 8.4 us.)
    // Loads go through buffer descriptors: the per-lane part of each offset
    // is computed once, the per-block part is a scalar offset, so the loads
    // take no vector address arithmetic (four token tiles: plain loads,
    // measured faster there).  Token slots past M hold no codes; their
    // products land in outputs that are not stored.
    constexpr bool kQDesc = TT <= 2;
    const auto rq = buffer_rsrc(qm, static_cast<uint32_t>(TT) * 2048u * static_cast<uint32_t>(Tb));
    const size_t coef_words = static_cast<size_t>(Np) * Tb, planes_bytes = static_cast<size_t>(Np / 64) * Tb * P * 1024;

    for (int sb = s_beg; sb < s_end; sb += S) {
        const int ns = min(S, s_end - sb);
        // per sub-tile: its 64-row tile and first row inside it (surplus
        // sub-tiles re-read the last one and store nothing)
        int tl[S], r0[S];
#pragma unroll
        for (int R = 0; R < S; ++R) {
            const int sg = sb + min(R, ns - 1);
            tl[R] = sg >> 2;
            r0[R] = 16 * (sg & 3);
        }
        // descriptors over the coefficients and planes from this pass's first
        // tile (offsets inside a pass span at most two tiles: 32 bits)
        const size_t cw0 = static_cast<size_t>(sb >> 2) * Tb * 64, pb0 = static_cast<size_t>(sb >> 2) * Tb * P * 1024;
        const auto rc = buffer_rsrc(coef + cw0, range_u32((coef_words - cw0) * 4));
        const auto rw = buffer_rsrc(blob + kHeaderBytes + pb0, range_u32(planes_bytes - pb0));
        uint32_t csub[S];  // scalar byte offset of sub-tile R's coefficient words in block 0
#pragma unroll
        for (int R = 0; R < S; ++R) csub[R] = static_cast<uint32_t>(((tl[R] - (sb >> 2)) * Tb) * 256 + r0[R] * 4);
        // weight pieces of a round of CC blocks: lane part of slot t's offset
        auto woff = [&](int CC, int t) __attribute__((always_inline)) {
            const int m = min(4 * t + g, CC * S * P - 1);  // (surplus slots re-read the last piece)
            const int i = m / (S * P), R = (m / P) % S, p = m % P;
            const int sg = sb + min(R, ns - 1);
            return static_cast<uint32_t>((((sg >> 2) - (sb >> 2)) * Tb + KW * i) * P + p) * 1024u +
                   static_cast<uint32_t>(16 * (sg & 3) + li) * 16u;
        };
        constexpr int NIC = (C * S * P + 3) / 4, NI1 = (S * P + 3) / 4;
        uint32_t woC[NIC], wo1[NI1];
#pragma unroll
        for (int t = 0; t < NIC; ++t) woC[t] = woff(C, t);
#pragma unroll
        for (int t = 0; t < NI1; ++t) wo1[t] = woff(1, t);
        v4i32_t acc[S][TT];
        float yacc[S][TT][4];
#pragma unroll
        for (int R = 0; R < S; ++R)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                acc[R][tt] = v4i32_t{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 4; ++i) yacc[R][tt][i] = 0.0f;
            }

        using Blk = MfmaBlock<P, S, TT, LOADC>;
        auto load = [&](Blk& L, int b) __attribute__((always_inline)) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const uint32_t qo = static_cast<uint32_t>(lane) * 16u + static_cast<uint32_t>(tt * 2 + s2) * 1024u;
                    if constexpr (kQDesc) {
                        const uint4 v = buffer_load_u128(rq, qo, static_cast<uint32_t>(b) * (TT * 2048u));
                        L.qv[s2][tt] = v4i32_t{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                                               static_cast<int>(v.w)};
                    } else {
                        L.qv[s2][tt] = *reinterpret_cast<const v4i32_t*>(qm + static_cast<size_t>(b) * (TT * 2048) + qo);
                    }
                }
            if constexpr (LOADC) {
#pragma unroll
                for (int R = 0; R < S; ++R) {
                    const uint32_t so = csub[R] + 256u * static_cast<uint32_t>(b);
                    L.zr[R] = buffer_load_u32(rc, 4 * li, so);
                    L.cz[R] = buffer_load_u128(rc, 16 * g, so);
                }
            }
        };

        auto compute = [&](Blk& L, int b, auto word) __attribute__((always_inline)) {
            // every loaded value passes an empty asm here, so no use of this
            // block's data (and no wait for it) moves above the previous block's
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) asm volatile("" : "+v"(L.qv[s2][tt]));
            if constexpr (LOADC) {
#pragma unroll
                for (int R = 0; R < S; ++R) asm volatile("" : "+v"(L.zr[R]), "+v"(L.cz[R].x), "+v"(L.cz[R].y),
                                                         "+v"(L.cz[R].z), "+v"(L.cz[R].w));
            }
#pragma unroll
            for (int R = 0; R < S; ++R) {
                uint32_t r[8];
                uint32_t wq[P];
#pragma unroll
                for (int p = 0; p < P; ++p) wq[p] = word(R, p);
                unpack_codes<P>(wq, r);
                if constexpr (PERM) {
                    // operand byte of each code through a byte table (v_perm_b32)
                    uint32_t tlo, thi = 0u;
                    if constexpr (FMT == BITQ_TERNARY) {
                        tlo = 0x00FF0100u;  // p + 2m = 0, 1, 2 -> 0, +1, -1
                    } else {
                        // bytes e - z for e = 0..7 ((e | 0x80) - z cannot borrow; ^ 0x80 takes 0x80 off);
                        // z in every byte by a byte permute; codes of one or two planes are below 4
                        const uint32_t z = static_cast<uint32_t>(f16_bits_to_f32(L.zr[R] >> 16));
                        const uint32_t zb = __builtin_amdgcn_perm(0u, z, 0x00000000u);
                        tlo = (0x83828180u - zb) ^ 0x80808080u;
                        if constexpr (P >= 3) thi = (0x87868584u - zb) ^ 0x80808080u;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = __builtin_amdgcn_perm(thi, tlo, r[e]);
                } else if constexpr (LOADC) {  // four planes: codes up to 15, c - z by arithmetic
                    const uint32_t z = static_cast<uint32_t>(f16_bits_to_f32(L.zr[R] >> 16));
                    const uint32_t zb = __builtin_amdgcn_perm(0u, z, 0x00000000u);
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = ((r[e] | 0x80808080u) - zb) ^ 0x80808080u;
                }
                // (ACC: the unshifted codes, so the int32 output is A itself)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const v4i32_t a = v4i32_t{static_cast<int>(r[4 * s2]), static_cast<int>(r[4 * s2 + 1]),
                                              static_cast<int>(r[4 * s2 + 2]), static_cast<int>(r[4 * s2 + 3])};
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
                        acc[R][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, L.qv[s2][tt], acc[R][tt], 0, 0, 0);
                }
            }
            if constexpr (GRP) {
                if constexpr (ACC) {  // exact group sums A[m][n][b]
#pragma unroll
                    for (int R = 0; R < S; ++R)
#pragma unroll
                        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int n = 16 * (sb + R) + 4 * g + i, m = 16 * tt + li;
                                if (R < ns && n < N && m < M)
                                    reinterpret_cast<int32_t*>(y)[(static_cast<size_t>(m) * N + n) * Tb + b] =
                                        acc[R][tt][i];
                            }
                } else {
#pragma unroll
                    for (int R = 0; R < S; ++R) {
                        const uint32_t c[4] = {L.cz[R].x, L.cz[R].y, L.cz[R].z, L.cz[R].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float delta = f16_bits_to_f32(c[i]);
#pragma unroll
                            for (int tt = 0; tt < TT; ++tt)  // acc = A - z S128 (one fused multiply-add)
                                yacc[R][tt][i] = __builtin_fmaf(delta, static_cast<float>(acc[R][tt][i]), yacc[R][tt][i]);
                        }
                    }
                }
#pragma unroll
                for (int R = 0; R < S; ++R)
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) acc[R][tt] = v4i32_t{0, 0, 0, 0};
            }
        };

        // Weights as 16-byte loads: the pieces (block i of the round, sub-tile
        // R, plane p), m = (i S + R) P + p, go 4 to a load, lane (j, r) taking
        // row r of piece 4 t + j (its 4 plane words).  A 4 x 4 transpose across
        // the lane groups (two 32-lane and two 16-lane swaps) then gives lane
        // (g, li) word g of row li of each of the 4 pieces: the operand layout.
        auto round = [&](auto cint, int i0) __attribute__((always_inline)) {
            constexpr int CC = decltype(cint)::value;
            constexpr int NPC = CC * S * P, NI = (NPC + 3) / 4;
            // loads, all unconditional: each block's q and coefficients
            // (L2-resident, small) first, then the weight stream
            Blk L[CC];
#pragma unroll
            for (int i = 0; i < CC; ++i) load(L[i], wave + KW * (i0 + i));
            uint4 wr[NI];
            const uint32_t wso = static_cast<uint32_t>(wave + KW * i0) * P * 1024u;  // the round's first block
#pragma unroll
            for (int t = 0; t < NI; ++t) wr[t] = buffer_load_u128(rw, CC == C ? woC[t] : wo1[t], wso);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t wt[NI][4];
#pragma unroll
            for (int i = 0; i < CC; ++i) {
                // transpose the loads whose first piece belongs to block i
                // (the wait for them is here)
#pragma unroll
                for (int t = 0; t < NI; ++t) {
                    if ((4 * t) / (S * P) != i) continue;
                    uint32_t a0 = wr[t].x, a1 = wr[t].y, a2 = wr[t].z, a3 = wr[t].w;
                    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
                    const auto s02 = __builtin_amdgcn_permlane32_swap(a0, a2, false, false);
                    const auto s13 = __builtin_amdgcn_permlane32_swap(a1, a3, false, false);
                    const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
                    const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
                    wt[t][0] = s01[0];
                    wt[t][1] = s01[1];
                    wt[t][2] = s23[0];
                    wt[t][3] = s23[1];
                }
                compute(L[i], wave + KW * (i0 + i), [&](int R, int p) __attribute__((always_inline)) {
                    const int m = (i * S + R) * P + p;
                    return wt[m / 4][m % 4];
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // whole rounds of C blocks, then the wave's remaining blocks one at
        // a time: no slot is ever surplus, so nothing is predicated
        int i0 = 0;
        for (; i0 + C <= nbw; i0 += C) round(std::integral_constant<int, C>{}, i0);
        for (; i0 < nbw; ++i0) round(std::integral_constant<int, 1>{}, i0);

        if constexpr (!(GRP && ACC)) {
            if constexpr (TT == 1) dtok[0] = ad[min((tid >> 4) & 15, M - 1)];
            // ---- the waves' partials, added in wave order
#pragma unroll
            for (int R = 0; R < S; ++R)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s_part[wave][(R * TT + tt) * 4 + i][lane] =
                            GRP ? yacc[R][tt][i] : __int_as_float(acc[R][tt][i]);
            __syncthreads();
            // Output (row n, token m) of the pass is summed over the waves in
            // wave order.  Thread idx takes n16 = idx % 16 (n = 16 (sb + R) +
            // n16, held by lane 16 (n16 / 4) + li as element n16 % 4), token
            // m = 16 tt + li with li = idx / 16 % 16, and the sub-tile and
            // tile rt = idx / 256: a wave's stores are 4 tokens x 64
            // contiguous bytes of y.
            for (int idx = tid; idx < NV * 64; idx += 64 * KW) {
                const int n16 = idx & 15, li2 = (idx >> 4) & 15, rt = idx >> 8;
                const int R = rt / TT, tt = rt % TT;
                const int k = 4 * rt + (n16 & 3), l = 16 * (n16 >> 2) + li2;
                const int n = 16 * (sb + R) + n16, m = 16 * tt + li2;
                float vf = 0.0f;
                int vi = 0;
#pragma unroll
                for (int w = 0; w < KW; ++w) {
                    if (GRP)
                        vf += s_part[w][k][l];
                    else
                        vi += __float_as_int(s_part[w][k][l]);
                }
                if (R < ns && n < N && m < M) {
                    float dm = dtok[0];
#pragma unroll
                    for (int t2 = 1; t2 < TT; ++t2)
                        if (tt == t2) dm = dtok[t2];
                    if (GRP)
                        y[static_cast<size_t>(m) * N + n] = dm * vf;
                    else if (ACC)
                        reinterpret_cast<int32_t*>(y)[static_cast<size_t>(m) * N + n] = vi;
                    else
                        y[static_cast<size_t>(m) * N + n] = gamma * dm * static_cast<float>(vi);
                }
            }
            __syncthreads();
        }
    }
}

template <int FMT, int P, bool ACC, int TT, int KW, int C>
static void launch_mfma_1(const bitq_wdesc& d, const BlobLayout& L, const MfmaShape& sh, const void* w,
                          const void* act, int M, float* y, hipStream_t st) {
    ActLayout A = act_layout(M, d.K, d.rank);
    // one sub-tile per workgroup when the sub-tiles do not outnumber the CUs
    // (up to 4096 rows): no surplus slots
    auto kern = sh.RS == 1 ? gemm_mfma_kernel<FMT, P, ACC, TT, KW, C, 1> : gemm_mfma_kernel<FMT, P, ACC, TT, KW, C, kMfmaSubs>;
    hipLaunchKernelGGL(kern, dim3(sh.grid), dim3(64 * KW), 0, st,
                       static_cast<const uint8_t*>(w), L.off_c0, static_cast<const uint8_t*>(act), A.off_qm, A.off_d,
                       M, d.N, static_cast<int>(L.Tb), static_cast<int>(L.Np / 16), y);
}

// The (KW, C) pairs built for each token-tile count; mfma_shape picks one.
template <int FMT, int P, bool ACC, int TT>
static void launch_mfma_kw(const bitq_wdesc& d, const BlobLayout& L, const MfmaShape& sh, const void* w,
                           const void* act, int M, float* y, hipStream_t st) {
#define BITQ_MFMA_CASE(KW_, C_) \
    if (sh.KW == KW_ && sh.CH == C_) return launch_mfma_1<FMT, P, ACC, TT, KW_, C_>(d, L, sh, w, act, M, y, st)
    if constexpr (TT == 1) {
        BITQ_MFMA_CASE(16, 1);
        launch_mfma_1<FMT, P, ACC, TT, 16, 2>(d, L, sh, w, act, M, y, st);
    } else {
        BITQ_MFMA_CASE(8, 1);
        launch_mfma_1<FMT, P, ACC, TT, 8, 2>(d, L, sh, w, act, M, y, st);
    }
#undef BITQ_MFMA_CASE
}

template <int FMT, int P, bool ACC>
static void launch_mfma(const bitq_wdesc& d, const BlobLayout& L, const void* w, const void* act, int M, float* y,
                        hipStream_t st) {
    const MfmaShape sh = mfma_shape(d, M);
    switch (sh.TT) {
        case 1: launch_mfma_kw<FMT, P, ACC, 1>(d, L, sh, w, act, M, y, st); break;
        case 2: launch_mfma_kw<FMT, P, ACC, 2>(d, L, sh, w, act, M, y, st); break;
        case 3: launch_mfma_kw<FMT, P, ACC, 3>(d, L, sh, w, act, M, y, st); break;
        default: launch_mfma_kw<FMT, P, ACC, 4>(d, L, sh, w, act, M, y, st); break;
    }
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
