/*
 * bitq.h -- C ABI of libbitq: decode-time linear layers y = W x on AMD MI355X
 * (gfx950) with W stored as packed binary bit-planes and small float
 * coefficients.
 *
 * Sources (cited below by the short name in brackets):
 *   [RaBiT]  "RaBiT框架：突破2比特量化性能瓶颈的LLM部署方案"
 *            (2-path residual binarization W^ = g1.B1.h1 + g2.B2.h2)
 *   [HGF]    "1.58位LLM混合门控流优化技术解析"
 *            (ternary weights with absmean gamma, int8 activations, a gated
 *             low-rank fp16 correction path)
 *   [ABQ]    "ABQ-LLM：用于大語言模型的任意比特量化推理加速"
 *            (arbitrary-bit weight/activation planes, binary-TensorCore-
 *             equivalent integer GEMV)
 *   [BVSR]   "BVSR：面向分布感知的大语言模型权重量化的比特向量求和表示"
 *            (bitvector-sum representation, AND+popcount GEMV)
 *   [BitNet] "1-bit LLM的端侧推理革命" (sign() binarization, scale alpha,
 *            XNOR+popcount, the weight-parameter struct of §3.2)
 *
 * Conventions for every entry point
 *   - Shapes: W is [N, K] (N outputs, K inputs); activations are [M, K]
 *     row-major; outputs y are [M, N] row-major fp32.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     memory (host or device) and keeps no state between calls other than a
 *     per-thread error string, a per-device "is gfx950" check and the static
 *     device scratch of bitq_quantize_act_hgf_noalloc.
 *   - Validation: every argument is checked before anything is enqueued or
 *     written.  On error nothing is written, a negative bitq_status is
 *     returned and bitq_last_error() describes it.  No C++ exception crosses
 *     the ABI; the library never aborts or exits.
 *   - Device calls are asynchronous on the given stream (a hipStream_t passed
 *     as void*, NULL = the null stream) and never synchronize.  A launch
 *     failure reported by the HIP runtime maps to BITQ_E_DEVICE.
 *   - Device pointers must satisfy the alignments stated per call
 *     (BITQ_E_ALIGN otherwise); host pointers need natural alignment only.
 */
#ifndef BITQ_H
#define BITQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITQ_VERSION 1

typedef enum {
    BITQ_OK = 0,
    BITQ_E_ARG = -1,          /* null pointer, bad enum, bad value in a logical form */
    BITQ_E_SHAPE = -2,        /* N, K, M or planes/group out of range or misaligned */
    BITQ_E_ALIGN = -3,        /* device pointer alignment */
    BITQ_E_UNSUPPORTED = -4,  /* format/flag combination not implemented, non-gfx950 device */
    BITQ_E_CAPACITY = -5,     /* destination or workspace smaller than required */
    BITQ_E_DEVICE = -6        /* error reported by the HIP runtime */
} bitq_status;

/* Weight formats. */
typedef enum {
    BITQ_SIGN1 = 1,    /* [BitNet] §2.1-2.2: W^ = alpha_n * B, B = sign(W) in {-1,+1},
                          one fp32 alpha per output row. planes = 1, group = 0. */
    BITQ_RABIT = 2,    /* [RaBiT] §2.1-2.2: W^ = sum_p g_p (.) B_p (.) h_p with B_p in
                          {-1,+1}, g_p fp16 per row, h_p fp16 per column.
                          planes = number of paths (1..3), group = 0. */
    BITQ_TERNARY = 3,  /* [HGF] §1.2: W^ = gamma * T, T in {-1,0,1} stored as a
                          plus plane and a minus plane (2 bits/weight), one fp32
                          gamma per tensor. planes = 2, group = 0. */
    BITQ_W2A8 = 4,     /* [ABQ] §3.2 Eq. (3): 2-bit asymmetric codes q in 0..3,
                          W^ = delta * (q - z) per group of 128 consecutive inputs,
                          delta and z fp16; the two bits are two binary planes.
                          planes = 2, group = 128. */
    BITQ_BVSR4 = 5,    /* [BVSR] introduction: per group of 32 consecutive inputs,
                          W^ = b + sum_k c_k beta_k with 4 {0,1} bitvectors
                          beta_0..3 and a coefficient set (c_0..c_3, b) picked by
                          a u8 index from a shared 256-entry cache of fp32 sets.
                          planes = 4, group = 32. */
    BITQ_WNAM = 6,     /* [ABQ] §1 arbitrary-bit WnAm: n-bit asymmetric codes
                          q in 0..2^n-1, W^ = delta * (q - z) per group of 128
                          inputs (delta, z fp16; the W2A8 arithmetic with
                          2^n - 1 steps), times m-bit symmetric activations.
                          planes = n (1..4), group = 128, abits = m (2..8). */
    BITQ_HGF = 7       /* [HGF] §2.1 and §4.1: the TERNARY layer plus a gated
                          low-rank correction of its unquantized input x:
                          y = gamma d (T q) + tanh(alpha) (silu(x A) B), with
                          A [K][r] and B [r][N] in fp16 and the gate parameter
                          alpha in fp32.  planes = 2, group = 0, rank = r
                          (8, 16, 32 or 64), K <= 16128. */
} bitq_format;

/* Activation dtypes accepted by bitq_quantize_act / bitq_gemv. */
typedef enum {
    BITQ_DT_F32 = 0,   /* raw fp32 activations [M, K] */
    BITQ_DT_BF16 = 1,  /* raw bf16 activations [M, K] (uint16 bit patterns) */
    BITQ_DT_ACT = 2,   /* an activation buffer written by bitq_quantize_act */
    BITQ_DT_BINARY = 3 /* a binary activation buffer written by bitq_binarize_act
                          (SIGN1 weights only: the fully binary XNOR path) */
} bitq_dtype;

/* Flags of bitq_gemv / bitq_gemm_smallM. */
#define BITQ_F_ACC_INT32 1u  /* integer formats only: the production main loop
                                writes its exact int32 partial sums to y instead
                                of the fp32 output (see bitq_gemv). */
#define BITQ_F_FUSE_QUANT 2u /* bitq_gemv with TERNARY/W2A8/BVSR4/WNAM weights:
                                x_dev is the raw token (BITQ_DT_BF16 or
                                BITQ_DT_F32) and the activation quantizer runs
                                in the GEMV kernel (see bitq_gemv). */

/* Shape/format descriptor of one weight matrix. */
typedef struct {
    int32_t fmt;      /* bitq_format */
    int32_t N;        /* outputs, 1 .. 2^24 */
    int32_t K;        /* inputs, multiple of 32 (of 128 for BITQ_W2A8/WNAM),
                         <= 2^20 (SIGN1/RABIT: <= 64512) */
    int32_t planes;   /* see bitq_format */
    int32_t group;    /* see bitq_format */
    int32_t abits;    /* activation bits of the integer GEMV: WNAM 2..8; the
                         other integer formats 0 or 8 (int8); float formats 0.
                         Activation buffers passed to the GEMV must have been
                         written with the same bit count. */
    int32_t rank;     /* HGF: rank r of the correction path (8, 16, 32, 64);
                         0 for every other format */
} bitq_wdesc;

/*
 * Logical (unpacked) quantized form of one weight matrix, host memory,
 * row-major.  Only the fields of the descriptor's format are read; the rest
 * may be NULL.  fp16 values are passed as their IEEE binary16 bit patterns.
 *
 *   BITQ_SIGN1   sign [N][K] (+1/-1), alpha [N]
 *   BITQ_RABIT   sign [P][N][K] (+1/-1), g [P][N], h [P][K]
 *   BITQ_TERNARY tern [N][K] (-1/0/+1), gamma
 *   BITQ_W2A8    code [N][K] (0..3), delta [N][K/128], zero [N][K/128]
 *                (zero must hold an integer 0..3)
 *   BITQ_BVSR4   code [N][K] (0..15, bit k = bitvector beta_k), idx [N][K/32],
 *                cache [256][5] as (c0, c1, c2, c3, b)
 *   BITQ_WNAM    code [N][K] (0..2^n-1), delta [N][K/128], zero [N][K/128]
 *                (zero must hold an integer 0..2^n-1)
 *   BITQ_HGF     tern [N][K] (-1/0/+1), gamma, lora_a [K][r], lora_b [r][N]
 *                (finite fp16), lora_alpha (finite)
 *
 * This mirrors the weight-parameter struct of [BitNet] §3.2 (binary weights,
 * scales, optional zero points) generalized to the six formats.
 */
typedef struct {
    const int8_t*   sign;
    const int8_t*   tern;
    const uint8_t*  code;
    const float*    alpha;
    const uint16_t* g;
    const uint16_t* h;
    float           gamma;
    const uint16_t* delta;
    const uint16_t* zero;
    const uint8_t*  idx;
    const float*    cache;
    const uint16_t* lora_a;
    const uint16_t* lora_b;
    float           lora_alpha;
} bitq_logical;

/*
 * Packed blob layout (what bitq_pack_weights writes and the kernels read).
 * Little-endian.  Np = N rounded up to 64, Kp = K rounded up to 128.
 *
 *   header, 256 bytes: u32 magic 0x51544942 ("BITQ"), u32 version (1),
 *     u32 fmt, u32 N, u32 K, u32 P (planes), u32 group, u32 Np, u32 Kp,
 *     u32 reserved (0), u64 off_planes, u64 off_c0, u64 off_c1,
 *     u64 total_bytes, then at byte 72 f32 hbound[3]: SIGN1 1, RABIT
 *     max_k |h_p[k]| for p < P (the float GEMV bounds its split-k sums with
 *     it); HGF only, from byte 88: u64 off_c2, u32 rank, f32 alpha,
 *     f32 gate = tanh(alpha) (fp64, rounded to fp32), f32 amax_a =
 *     max |A|; the rest is zero.
 *   planes section: tiles of 64 rows x 128 inputs x 1 plane = 1024 bytes,
 *     ordered [row tile t][k block b][plane p].  Inside a tile, row
 *     r = n - 64t owns 16 contiguous bytes = 4 uint32 words; word w holds
 *     inputs k = 128b + 32w + i at bit i (LSB first).  So the 64 rows of a
 *     tile are adjacent: one 16-byte load per lane, 1 KB per 64-lane wave,
 *     is fully coalesced ([BVSR] introduction: bitvectors of consecutive
 *     output rows stored next to each other).  Rows >= N and inputs >= K are
 *     zero bits.
 *   plane meaning: SIGN1/RABIT bit 1 <-> +1, 0 <-> -1 (one plane per path);
 *     TERNARY and HGF plane 0 = [T == +1], plane 1 = [T == -1]; W2A8 plane i = bit i
 *     of q; BVSR4 planes hold the four bitvectors nibble-interleaved: plane s
 *     of a 32-input word carries its inputs 8s .. 8s+7, one per nibble, bits
 *     4e .. 4e+3 for input 8s + (e >> 1) + 4 (e & 1) with bit 4e + j =
 *     beta_j (the kernel masks one bitvector and takes 8 inputs per 4-bit
 *     dot product).
 *   coefficient sections (zero-padded):
 *     SIGN1   c0 = alpha f32 [Np]
 *     RABIT   c0 = g f16 [P][Np];  c1 = h f16 [P][Kp]
 *     TERNARY c0 = gamma f32 [1]
 *     W2A8    c0 = u32 [Np/64][Kp/128][64]: low 16 bits delta, high 16 bits z
 *     BVSR4   c0 = idx u8 [Np/64][Kp/128][64][4] (byte j: group 4b + j);
 *             c1 = cache f32 [256][5], entry (c_0, c_1/2, c_2/4, c_3/8, b)
 *             (the dot products of bitvector j carry the factor 2^j)
 *     HGF     c0 = gamma f32 [1];  c1 = A transposed, f16 [r][Kp] (row j
 *             holds A[k][j] for every k);  c2 = B transposed, f16 [Np][r]
 *             (row n holds B[j][n] for every j)
 *   Every section starts at a multiple of 256 bytes; off_c1 = total_bytes
 *   when a format has no c1 section.
 */

/*
 * Bytes of the packed blob for a descriptor: the header, the plane tiles and
 * the coefficient sections of the layout above, each section rounded up to
 * 256 bytes.  The plane tiles keep the bitvectors of consecutive output rows
 * next to each other, the coalesced layout of [BVSR] introduction; the
 * coefficient sections are those of each format's definition (see
 * bitq_format).  Host only; BITQ_E_SHAPE / BITQ_E_ARG for a bad descriptor.
 */
bitq_status bitq_packed_size(const bitq_wdesc* desc, size_t* bytes);

/*
 * Host packer: logical form -> packed blob (host memory, dst_bytes >=
 * bitq_packed_size).  Rejects codes outside their range (BITQ_E_ARG).
 * The blob is then copied to device memory by the caller (256-byte aligned).
 */
bitq_status bitq_pack_weights(const bitq_wdesc* desc, const bitq_logical* src,
                              void* dst, size_t dst_bytes);

/*
 * Host quantizer + packer: fp32 W [N][K] (host) -> packed blob, using the
 * library's own offline quantizer for the format:
 *   SIGN1   B = sign(W) (sign(0) = +1, [BitNet] §2.1), alpha_n = mean_k |W|
 *   RABIT   per path ([RaBiT] §2.2): B_p = sign(R_p), (g_p, h_p) = leading
 *           singular pair of |R_p| by 30 power iterations (fp64, sigma split
 *           evenly), stored fp16; R_{p+1} = R_p - g_p.B_p.h_p from the stored
 *           fp16 values; R_0 = W
 *   TERNARY gamma = mean|W| (fp32), T = clamp(rint(W/gamma), -1, 1) ([HGF] §1.2)
 *   W2A8    per 128-group min/max RTN ([ABQ] Eq. 3, no compensation)
 *   BVSR4   256-set cache from the group-range quantiles, exhaustive
 *           nearest-point / least-SSE search per 32-group ([BVSR] intro)
 * nthreads <= 0 uses all hardware threads.  W must be finite.
 */
bitq_status bitq_quantize_weights(const bitq_wdesc* desc, const float* W, void* dst,
                                  size_t dst_bytes, int32_t nthreads);

/*
 * HGF host quantizer + packer: the TERNARY quantizer of bitq_quantize_weights
 * for the backbone W (fp32 [N][K], host), together with the trained
 * correction parameters ([HGF] §2.1) lora_a [K][r] and lora_b [r][N] (fp16
 * bit patterns, finite, host) and the gate parameter lora_alpha (finite).
 * desc must be an HGF descriptor.
 */
bitq_status bitq_quantize_weights_hgf(const bitq_wdesc* desc, const float* W, const uint16_t* lora_a,
                                      const uint16_t* lora_b, float lora_alpha, void* dst,
                                      size_t dst_bytes, int32_t nthreads);

/* Options of the offline quantizer (zero-initialize; reserved must stay 0). */
typedef struct {
    int32_t rabit_svid_sweeps;  /* RABIT: Gauss-Seidel sweeps of [RaBiT] §2.2's
                                   iterative residual SVID after the greedy
                                   pass (0 = greedy only; the page's default
                                   is 20).  Path p is refitted to
                                   T = W - sum_{q != p} g_q B_q h_q (stored fp16
                                   scales): B_p = sign(T), (g_p, h_p) = rank-1
                                   fit of |T|.  0..1000 */
    int32_t wnam_bit_balance;   /* WNAM with planes = 3: [ABQ] §3.3 bit balance,
                                   the 2-bit grid widened to the symmetric
                                   {-2,-1,0,1,2}: per 128-group
                                   delta = fl16(max|W| / 2),
                                   code = clamp(rint(W / delta), -2, 2) + 2,
                                   z = 2 (a zero step gives delta = 1, code 2).
                                   0 or 1 */
    int32_t reserved[6];
} bitq_quant_opts;

/* bitq_quantize_weights with options (NULL opts: BITQ_E_ARG). */
bitq_status bitq_quantize_weights_opts(const bitq_wdesc* desc, const float* W,
                                       const bitq_quant_opts* opts, void* dst,
                                       size_t dst_bytes, int32_t nthreads);

/*
 * Activation buffer (written by bitq_quantize_act, read by the integer
 * formats).  Kp = K rounded up to 128, Kw = Kp / 32.  Sections, each at a
 * multiple of 256 bytes, in this order:
 *   planes u32 [M][Kw][8]  plane j of word w = bit j of the two's-complement
 *                          byte of q[m][32w + i] at bit i
 *   S      i32 [M][Kw]     sum of q over each run of 32 inputs
 *   q      i8  [M][Kp]     quantized activations (0 beyond K)
 *   qm     i8  [Kp/128][T][2][64][16]  the same codes in the order the
 *                          matrix-core kernel reads them, T = ceil(M/16) tiles
 *                          of 16 tokens: input 8e + 2c + s of word g (inputs
 *                          32g .. 32g + 31) of 128-input block b, token
 *                          m = 16t + j, at byte ((b T + t) 2 + s) 1024 +
 *                          (16 g + j) 16 + 4c + e (token slots past M unused)
 *   d      f32 [M]         dequantization step amax/Qm (Qm = 127 for int8)
 *   amax   f32 [M]         max_k |x[m][k]|
 * With m-bit activations (bitq_quantize_act_bits) q lies in [-Qm, Qm],
 * Qm = 2^(m-1) - 1; the byte's bits m-1..7 then all equal the sign, and the
 * GEMV uses planes 0..m-2 and plane 7 (weight -2^(m-1)).
 */
bitq_status bitq_act_size(int32_t M, int32_t K, size_t* bytes);

/*
 * Per-token int8 quantization ([HGF] §1.2: int8 activations rescaled by
 * gamma_x/127; [BVSR] intro: online conversion of activations to bit-planes).
 * For each token m: amax = max_k |x|; if amax = 0 then q = 0 and d = 0, else
 * s = fl32(127/amax) (correctly rounded), q = clamp(rint(fl32(x*s)), -127,
 * 127) (round half to even), d = fl32(amax/127).  Bit-exact.
 *   x_dev   device [M][K] fp32 or bf16 (x_dtype BITQ_DT_F32/BF16), 16-byte
 *           aligned, finite values
 *   act_dev device buffer of bitq_act_size bytes, 256-byte aligned
 * 1 <= M <= 64.
 */
bitq_status bitq_quantize_act(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K,
                              void* act_dev, size_t act_bytes, void* stream);

/*
 * The same per-token quantization to m = abits bits ([ABQ] §1: arbitrary
 * activation precision, e.g. A4, A6): Qm = 2^(m-1) - 1 replaces 127, i.e.
 * s = fl32(Qm/amax), q = clamp(rint(fl32(x*s)), -Qm, Qm), d = fl32(amax/Qm).
 * abits 2..8; abits = 8 is bitq_quantize_act.  Same buffer layout.
 */
bitq_status bitq_quantize_act_bits(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K,
                                   int32_t abits, void* act_dev, size_t act_bytes, void* stream);

/*
 * HGF activation buffer: the sections of bitq_act_size(M, K), then, at the
 * next multiple of 256 bytes,
 *   h  f32 [M][r]   h[m] = silu(x[m] A), the correction path's hidden vector.
 * ws_bytes is the workspace of bitq_quantize_act_hgf: M*r 64-bit words.  The
 * caller zero-fills it once before its first use; every completed call
 * leaves it zero again, so it is reused without clearing.  Calls that share
 * a workspace must be ordered (same stream).
 */
bitq_status bitq_hgf_act_size(const bitq_wdesc* desc, int32_t M, size_t* act_bytes, size_t* ws_bytes);

/*
 * Activation step of an HGF layer: the int8 quantization of
 * bitq_quantize_act ([HGF] §1.2; bit-exact, the same sections), and from the
 * same unquantized input the correction's down projection ([HGF] §2.1)
 *   h[m][j] = silu(z), z = sum_k x[m][k] A[k][j], silu(z) = z / (1 + exp(-z)).
 * z is summed in fp32 over each run of 256 inputs.  The runs are then added
 * exactly as 64-bit fixed-point integers, scaled to the bound
 * K max_k|x[m][k]| amax_a, so h does not depend on workgroup order; the
 * arrival count shares the word, and the run that completes a sum applies
 * silu in fp32.
 *   desc    an HGF descriptor; w_dev its packed blob (device, 256-byte aligned)
 *   x_dev   device [M][K] fp32 or bf16, 16-byte aligned, finite values
 *   act_dev device, >= act_bytes of bitq_hgf_act_size, 256-byte aligned
 *   ws_dev  device, >= ws_bytes of bitq_hgf_act_size, 256-byte aligned
 * 1 <= M <= 64.
 */
bitq_status bitq_quantize_act_hgf(const bitq_wdesc* desc, const void* w_dev, const void* x_dev,
                                  int32_t x_dtype, int32_t M, void* act_dev, size_t act_bytes,
                                  void* ws_dev, size_t ws_bytes, void* stream);

/*
 * bitq_quantize_act_hgf without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, arithmetic and outputs
 * as bitq_quantize_act_hgf; the fixed-point words of the down projection live
 * in the library's own static device array of 64 x 64 words (32 KB per GPU,
 * held until the process ends), which covers every valid call
 * (M * rank <= 4096; larger gives BITQ_E_CAPACITY).  Nothing is allocated:
 * the array's device address is looked up on the first call on each device,
 * which also clears it with a small kernel on the given stream; every
 * completed call leaves it zero again.  All calls on one GPU share the array:
 * calls that may overlap in time on one GPU (different streams without
 * ordering, concurrent graphs) race and give wrong h; order them.
 */
bitq_status bitq_quantize_act_hgf_noalloc(const bitq_wdesc* desc, const void* w_dev, const void* x_dev,
                                          int32_t x_dtype, int32_t M, void* act_dev, size_t act_bytes,
                                          void* stream);

/*
 * Binary activation buffer (written by bitq_binarize_act, read by the SIGN1
 * XNOR path).  Kp = K rounded up to 128, Kw = Kp / 32.  Sections, each at a
 * multiple of 256 bytes:
 *   bits u32 [M][Kw]  bit i of word w = [x[m][32w + i] >= 0] (1 <-> +1; zero
 *                     past K)
 *   beta f32 [M]      mean_k |x[m][k]| (fp32 sum in a fixed order, / K)
 */
bitq_status bitq_binact_size(int32_t M, int32_t K, size_t* bytes);

/*
 * Binary activations of the fully binary path ([BitNet] §2.1: sign(x) = +1
 * for x >= 0, else -1; §2.3 XNOR+popcount product): the sign bits of every
 * input and the per-token scale beta = mean |x| (the page gives the weight
 * scale only; beta is the reading taken, so that beta sign(x) approximates x).
 *   x_dev   device [M][K] fp32 or bf16, 16-byte aligned
 *   act_dev device buffer of bitq_binact_size bytes, 256-byte aligned
 * 1 <= M <= 64.  The bits are exact; beta is an fp32 sum.
 */
bitq_status bitq_binarize_act(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K,
                              void* act_dev, size_t act_bytes, void* stream);

/*
 * Workspace for one bitq_gemv / bitq_gemm_smallM call (device memory, 256-byte
 * aligned).  SIGN1/RABIT layers whose k range is split over several
 * workgroups need one 64-bit word per row (Np words), in which the splits
 * add their fixed-point partial sums together with an arrival count.  The
 * size is 0 when the call needs none (the integer formats, whose workgroups
 * each cover the whole k range, and float layers with a single split);
 * ws_dev may then be NULL.  The caller zero-fills it once before its first
 * use; every completed call leaves the words at zero again, so the same
 * workspace is reused without clearing.  Calls that share a workspace must
 * be ordered (same stream); concurrent calls need distinct workspaces.
 */
bitq_status bitq_workspace_size(const bitq_wdesc* desc, int32_t M, size_t* bytes);

/*
 * Batch-1 GEMV y[N] = W^ x.
 *   w_dev  packed blob in device memory (256-byte aligned)
 *   x_dev  SIGN1/RABIT: raw activations, BITQ_DT_F32 or BITQ_DT_BF16, 16-byte
 *          aligned.  TERNARY/W2A8/BVSR4/WNAM: an activation buffer from
 *          bitq_quantize_act (WNAM: bitq_quantize_act_bits with desc->abits)
 *          with M = 1 (x_dtype = BITQ_DT_ACT); HGF: the buffer of
 *          bitq_quantize_act_hgf with M = 1.  SIGN1 with x_dtype =
 *          BITQ_DT_BINARY: a binary activation buffer from bitq_binarize_act
 *          with M = 1 (the XNOR path; no workspace needed, ws_dev may be
 *          NULL).
 *   y_dev  fp32 [N], 4-byte aligned.
 * Float formats ([RaBiT] §3.2 sign-apply instead of multiplies): y_n =
 *   sum_p g_p[n] sum_k B_p[n,k] h_p[k] x_k (SIGN1: alpha_n sum_k B[n,k] x_k),
 *   accumulated in fp32 per k slice; the slices are added exactly in 64-bit
 *   fixed point scaled to the bound sum_p |g_p[n]| max|h_p| sum_k |x_k|, so
 *   y does not depend on the order of the workgroups.  A row whose bound is
 *   not finite (inf/NaN in x, g or h) comes out NaN.
 * Integer formats (AND+popcount of weight planes with activation planes,
 *   [ABQ] abstract/§1, [BVSR] intro; exact int32 partial sums):
 *   TERNARY y_n = gamma d Y_n, Y_n = sum_k T[n,k] q_k
 *   W2A8    y_n = d sum_g delta[n,g] (A[n,g] - z[n,g] S128[g]),
 *           A[n,g] = sum_{k in g} q[n,k] q_k
 *   BVSR4   y_n = d sum_g (b S32[g] + sum_j c_j P[n,g,j]),
 *           P[n,g,j] = sum_{k in g} beta_j[n,k] q_k, (c, b) = cache[idx[n,g]]
 *   WNAM    as W2A8 with n-bit codes and m-bit q: the AND+popcount runs over
 *           n weight planes and m activation planes only
 *   HGF     y_n = gamma d Y_n + gate sum_j h_j B[j][n] ([HGF] §4.1: the
 *           ternary product and the correction in one kernel), Y_n as
 *           TERNARY, the correction's up projection in fp32
 * Fully binary path (SIGN1, BITQ_DT_BINARY; [BitNet] §2.3 XNOR+popcount):
 *   y_n = alpha_n beta Y_n, Y_n = sum_k B[n,k] sign(x_k)
 *       = K - 2 popcount(bits(B_n) XOR bits(x)), exact
 * flags & BITQ_F_ACC_INT32 (integer formats): y_dev receives, as int32,
 *   TERNARY/HGF Y [N]; W2A8/WNAM A [N][K/128]; BVSR4 P [N][K/32][4]; SIGN1 with
 *   binary activations Y [N]; the buffer must hold that many int32 values.
 * flags & BITQ_F_FUSE_QUANT (TERNARY, W2A8, BVSR4, WNAM; K <= 16384): x_dev
 *   is the raw token, x_dtype BITQ_DT_BF16 or BITQ_DT_F32, 16-byte aligned,
 *   finite values.  The activation quantizer ([HGF] §1.2 absmax int8; [ABQ]
 *   m-bit for WNAM with desc->abits) runs in the GEMV kernel's prologue
 *   instead of a separate bitq_quantize_act launch, with the same arithmetic
 *   (the same q, planes, group sums and d).  TERNARY y is bit-identical to
 *   bitq_quantize_act followed by bitq_gemv (exact integer sums); so is the
 *   y of the other formats on layers below 4096 rows.  From 4096 rows on the
 *   fused kernel takes 16 rows per workgroup (the two-launch kernel 8 below
 *   16384 rows, and WNAM always 8), so its fp32 group terms are added in
 *   another order and y may differ in the last bits, within the tolerance.
 *   Nothing but y is written (no activation buffer, no workspace).  Errors:
 *   BITQ_E_UNSUPPORTED for other formats (HGF included), K > 16384, or
 *   together with BITQ_F_ACC_INT32; BITQ_E_ARG for another x_dtype.
 */
bitq_status bitq_gemv(const bitq_wdesc* desc, const void* w_dev, const void* x_dev,
                      int32_t x_dtype, float* y_dev, void* ws_dev, size_t ws_bytes,
                      uint32_t flags, void* stream);

/*
 * Small-batch GEMM y[M][N] = x W^T for 2 <= M <= 64, integer formats
 * (TERNARY, W2A8, BVSR4, WNAM, HGF) and SIGN1 with binary activations,
 * reading every weight once for all M tokens.  [ABQ] §1: in decoding the
 * GEMM degenerates into a GEMV and small batches (fewer than 8 tokens) are
 * padded on matrix units, wasting most of the multiply; here a batch of M
 * tokens is one pass over the weights, on the VALU for the fewest tokens
 * and on the int8 matrix cores once the contraction is compute-bound.
 *   act_dev activation buffer from bitq_quantize_act(_bits) with this M
 *           (SIGN1: from bitq_binarize_act; HGF: from bitq_quantize_act_hgf).
 * W2A8 and WNAM (from 2 tokens) and TERNARY (from 3) run on the int8 matrix cores
 * (codes recombined from the planes, exact int32 sums): the integer partials
 * equal those of bitq_gemv, the fp32 outputs agree within the tolerance
 * (another summation order), and a token's output does not depend on the
 * other tokens of the batch.
 *   y_dev   fp32 [M][N].  BITQ_F_ACC_INT32 writes [M][...] int32 partials
 *           laid out as in bitq_gemv, one block per token.
 */
bitq_status bitq_gemm_smallM(const bitq_wdesc* desc, const void* w_dev, const void* act_dev,
                             int32_t M, float* y_dev, void* ws_dev, size_t ws_bytes,
                             uint32_t flags, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* bitq_last_error(void);

/* BITQ_VERSION of the built library. */
int32_t bitq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITQ_H */
