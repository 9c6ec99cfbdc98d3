// Host side of libbitq: argument validation, blob/activation layouts, the
// host packer, the offline weight quantizers and the C ABI entry points.
//
// Sources are cited by the short names defined in include/bitq.h:
// [RaBiT], [HGF], [ABQ], [BVSR], [BitNet].

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "bitq_internal.h"

namespace bitq {
namespace {

thread_local std::string g_error;

bitq_status fail(bitq_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return s;
}

bitq_status ok() {
    g_error.clear();
    return BITQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------- fp16 helpers
// IEEE binary16 from a double, round-half-to-even, with subnormals and
// overflow to infinity.
uint16_t f64_to_f16(double x) {
    uint16_t sign = std::signbit(x) ? 0x8000 : 0;
    double a = std::fabs(x);
    if (std::isnan(a)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;  // halfway above 65504 rounds to inf
    if (a < std::ldexp(1.0, -14)) {           // subnormal range, ulp = 2^-24
        double r = std::nearbyint(std::ldexp(a, 24));
        return sign | static_cast<uint16_t>(r);  // r == 1024 encodes 2^-14
    }
    int e;
    std::frexp(a, &e);  // a = m 2^e, m in [0.5, 1)
    e -= 1;             // a in [2^e, 2^(e+1))
    double r = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    if (e > 15) return sign | 0x7C00;
    return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(r) - 1024));
}

double f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = std::ldexp(static_cast<double>(m), -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = std::ldexp(static_cast<double>(m + 1024), e - 25);
    return s ? -v : v;
}

// --------------------------------------------------------------- threading
template <class F>
void parallel_for(int64_t n, int nthreads, F&& body) {
    if (nthreads <= 0) nthreads = std::max(1u, std::thread::hardware_concurrency());
    nthreads = static_cast<int>(std::min<int64_t>(nthreads, std::max<int64_t>(n, 1)));
    if (nthreads <= 1) {
        for (int64_t i = 0; i < n; ++i) body(i);
        return;
    }
    std::atomic<int64_t> next{0};
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; ++t)
        th.emplace_back([&] {
            for (;;) {
                int64_t i = next.fetch_add(1);
                if (i >= n) break;
                body(i);
            }
        });
    for (auto& x : th) x.join();
}

// ------------------------------------------------------------- validation
bitq_status check_desc(const bitq_wdesc* d) {
    if (!d) return fail(BITQ_E_ARG, "desc is NULL");
    if (d->fmt < BITQ_SIGN1 || d->fmt > BITQ_HGF) return fail(BITQ_E_ARG, "unknown format %d", d->fmt);
    if (d->N < 1 || d->N > (1 << 24)) return fail(BITQ_E_SHAPE, "N=%d out of range [1, 2^24]", d->N);
    if (d->K < 32 || d->K > (1 << 20)) return fail(BITQ_E_SHAPE, "K=%d out of range [32, 2^20]", d->K);
    if (d->K % 32) return fail(BITQ_E_SHAPE, "K=%d is not a multiple of 32", d->K);
    if ((d->fmt == BITQ_SIGN1 || d->fmt == BITQ_RABIT) && d->K > kMaxFloatK)
        return fail(BITQ_E_SHAPE, "K=%d: SIGN1/RABIT support K <= %d", d->K, kMaxFloatK);
    switch (d->fmt) {
        case BITQ_SIGN1:
            if (d->planes != 1 || d->group != 0)
                return fail(BITQ_E_SHAPE, "SIGN1 needs planes=1, group=0");
            break;
        case BITQ_RABIT:
            if (d->planes < 1 || d->planes > 3 || d->group != 0)
                return fail(BITQ_E_SHAPE, "RABIT needs planes in 1..3, group=0");
            break;
        case BITQ_TERNARY:
            if (d->planes != 2 || d->group != 0)
                return fail(BITQ_E_SHAPE, "TERNARY needs planes=2, group=0");
            break;
        case BITQ_W2A8:
            if (d->planes != 2 || d->group != 128)
                return fail(BITQ_E_SHAPE, "W2A8 needs planes=2, group=128");
            if (d->K % 128) return fail(BITQ_E_SHAPE, "W2A8 needs K %% 128 == 0 (K=%d)", d->K);
            break;
        case BITQ_BVSR4:
            if (d->planes != 4 || d->group != 32)
                return fail(BITQ_E_SHAPE, "BVSR4 needs planes=4, group=32");
            break;
        case BITQ_WNAM:
            if (d->planes < 1 || d->planes > 4 || d->group != 128)
                return fail(BITQ_E_SHAPE, "WNAM needs planes in 1..4, group=128");
            if (d->K % 128) return fail(BITQ_E_SHAPE, "WNAM needs K %% 128 == 0 (K=%d)", d->K);
            if (d->abits < 2 || d->abits > 8) return fail(BITQ_E_SHAPE, "WNAM needs abits in 2..8 (abits=%d)", d->abits);
            break;
        case BITQ_HGF:
            if (d->planes != 2 || d->group != 0) return fail(BITQ_E_SHAPE, "HGF needs planes=2, group=0");
            if (d->rank != 8 && d->rank != 16 && d->rank != 32 && d->rank != 64)
                return fail(BITQ_E_SHAPE, "HGF needs rank 8, 16, 32 or 64 (rank=%d)", d->rank);
            if (d->K > kMaxHgfK) return fail(BITQ_E_SHAPE, "K=%d: HGF supports K <= %d", d->K, kMaxHgfK);
            break;
    }
    if (d->fmt != BITQ_HGF && d->rank != 0)
        return fail(BITQ_E_SHAPE, "rank=%d: only HGF has a correction rank (use 0)", d->rank);
    const bool intfmt = d->fmt == BITQ_TERNARY || d->fmt == BITQ_W2A8 || d->fmt == BITQ_BVSR4 || d->fmt == BITQ_HGF;
    if (intfmt && d->abits != 0 && d->abits != 8)
        return fail(BITQ_E_SHAPE, "abits=%d: TERNARY/W2A8/BVSR4/HGF use 8-bit activations (abits 0 or 8)", d->abits);
    if ((d->fmt == BITQ_SIGN1 || d->fmt == BITQ_RABIT) && d->abits != 0)
        return fail(BITQ_E_SHAPE, "abits=%d: SIGN1/RABIT take raw activations (abits 0)", d->abits);
    return BITQ_OK;
}

// ------------------------------------------------------------------ packer
void write_header(const bitq_wdesc& d, const BlobLayout& L, uint8_t* dst) {
    std::memset(dst, 0, kHeaderBytes);
    uint32_t u[10] = {kMagic,
                      1u,
                      static_cast<uint32_t>(d.fmt),
                      static_cast<uint32_t>(d.N),
                      static_cast<uint32_t>(d.K),
                      static_cast<uint32_t>(L.P),
                      static_cast<uint32_t>(d.group),
                      static_cast<uint32_t>(L.Np),
                      static_cast<uint32_t>(L.Kp),
                      0u};
    uint64_t v[4] = {L.off_planes, L.off_c0, L.off_c1, L.total};
    std::memcpy(dst, u, sizeof(u));
    std::memcpy(dst + 40, v, sizeof(v));
    if (d.fmt == BITQ_HGF) {
        const uint64_t off_c2 = L.off_c2;
        const uint32_t rank = static_cast<uint32_t>(d.rank);
        std::memcpy(dst + kHdrOffC2, &off_c2, 8);
        std::memcpy(dst + kHdrRank, &rank, 4);
    }
}

// Offset in bytes of the word (plane p, row n, word kw) inside the blob.
inline size_t plane_word_offset(const BlobLayout& L, int64_t p, int64_t n, int64_t kw) {
    int64_t t = n / kRowTile, r = n % kRowTile;
    int64_t b = kw / 4, w = kw % 4;
    return L.off_planes + static_cast<size_t>(((t * L.Tb + b) * L.P + p) * 1024 + r * 16 + w * 4);
}

// Fill all planes from a per-element bit extractor bit(p, n, k) -> 0/1.
template <class BitFn>
void pack_planes(const bitq_wdesc& d, const BlobLayout& L, uint8_t* dst, int nthreads, BitFn bit) {
    const int64_t Kw = d.K / 32;
    parallel_for(d.N, nthreads, [&](int64_t n) {
        for (int64_t p = 0; p < L.P; ++p)
            for (int64_t kw = 0; kw < Kw; ++kw) {
                uint32_t word = 0;
                for (int i = 0; i < 32; ++i) word |= static_cast<uint32_t>(bit(p, n, kw * 32 + i)) << i;
                std::memcpy(dst + plane_word_offset(L, p, n, kw), &word, 4);
            }
    });
}

bitq_status check_logical(const bitq_wdesc& d, const bitq_logical* s) {
    const int64_t N = d.N, K = d.K, P = d.planes;
    auto need = [&](const void* p, const char* name) -> bitq_status {
        return p ? BITQ_OK : fail(BITQ_E_ARG, "logical.%s is NULL", name);
    };
    bitq_status st = BITQ_OK;
    switch (d.fmt) {
        case BITQ_SIGN1:
        case BITQ_RABIT: {
            if ((st = need(s->sign, "sign"))) return st;
            if (d.fmt == BITQ_SIGN1) {
                if ((st = need(s->alpha, "alpha"))) return st;
            } else {
                if ((st = need(s->g, "g")) || (st = need(s->h, "h"))) return st;
            }
            const int64_t cnt = (d.fmt == BITQ_RABIT ? P : 1) * N * K;
            for (int64_t i = 0; i < cnt; ++i)
                if (s->sign[i] != 1 && s->sign[i] != -1)
                    return fail(BITQ_E_ARG, "sign[%lld]=%d is not +-1", (long long)i, s->sign[i]);
            break;
        }
        case BITQ_TERNARY:
        case BITQ_HGF:
            if ((st = need(s->tern, "tern"))) return st;
            for (int64_t i = 0; i < N * K; ++i)
                if (s->tern[i] < -1 || s->tern[i] > 1)
                    return fail(BITQ_E_ARG, "tern[%lld]=%d not in {-1,0,1}", (long long)i, s->tern[i]);
            if (d.fmt == BITQ_HGF) {
                if ((st = need(s->lora_a, "lora_a")) || (st = need(s->lora_b, "lora_b"))) return st;
                const int64_t r = d.rank;
                for (int64_t i = 0; i < K * r; ++i)
                    if ((s->lora_a[i] & 0x7C00u) == 0x7C00u)
                        return fail(BITQ_E_ARG, "lora_a[%lld] is not finite", (long long)i);
                for (int64_t i = 0; i < r * N; ++i)
                    if ((s->lora_b[i] & 0x7C00u) == 0x7C00u)
                        return fail(BITQ_E_ARG, "lora_b[%lld] is not finite", (long long)i);
                if (!std::isfinite(s->lora_alpha)) return fail(BITQ_E_ARG, "lora_alpha is not finite");
            }
            break;
        case BITQ_W2A8:
        case BITQ_WNAM: {
            if ((st = need(s->code, "code")) || (st = need(s->delta, "delta")) || (st = need(s->zero, "zero")))
                return st;
            const int top = (1 << d.planes) - 1;  // W2A8: planes = 2
            for (int64_t i = 0; i < N * K; ++i)
                if (s->code[i] > top)
                    return fail(BITQ_E_ARG, "code[%lld]=%d > %d", (long long)i, s->code[i], top);
            for (int64_t i = 0; i < N * (K / 128); ++i) {
                const double z = f16_to_f64(s->zero[i]);
                if (!(z >= 0 && z <= top && z == std::floor(z)))
                    return fail(BITQ_E_ARG, "zero[%lld] is not an integer in 0..%d", (long long)i, top);
            }
            break;
        }
        case BITQ_BVSR4:
            if ((st = need(s->code, "code")) || (st = need(s->idx, "idx")) || (st = need(s->cache, "cache")))
                return st;
            for (int64_t i = 0; i < N * K; ++i)
                if (s->code[i] > 15) return fail(BITQ_E_ARG, "code[%lld]=%d > 15", (long long)i, s->code[i]);
            break;
    }
    return BITQ_OK;
}

void pack_coefficients(const bitq_wdesc& d, const BlobLayout& L, const bitq_logical* s, uint8_t* dst) {
    const int64_t N = d.N, K = d.K, P = L.P, Np = L.Np, Kp = L.Kp;
    switch (d.fmt) {
        case BITQ_SIGN1:
            std::memcpy(dst + L.off_c0, s->alpha, 4 * N);
            break;
        case BITQ_RABIT:
            for (int64_t p = 0; p < P; ++p) {
                std::memcpy(dst + L.off_c0 + 2 * (p * Np), s->g + p * N, 2 * N);
                std::memcpy(dst + L.off_c1 + 2 * (p * Kp), s->h + p * K, 2 * K);
            }
            break;
        case BITQ_TERNARY: {
            float gmm = s->gamma;
            std::memcpy(dst + L.off_c0, &gmm, 4);
            break;
        }
        case BITQ_HGF: {
            float gmm = s->gamma;
            std::memcpy(dst + L.off_c0, &gmm, 4);
            const int64_t r = d.rank;
            uint16_t* at = reinterpret_cast<uint16_t*>(dst + L.off_c1);  // [r][Kp]
            uint16_t* bt = reinterpret_cast<uint16_t*>(dst + L.off_c2);  // [Np][r]
            for (int64_t k = 0; k < K; ++k)
                for (int64_t j = 0; j < r; ++j) at[j * Kp + k] = s->lora_a[k * r + j];
            for (int64_t j = 0; j < r; ++j)
                for (int64_t n = 0; n < N; ++n) bt[n * r + j] = s->lora_b[j * N + n];
            break;
        }
        case BITQ_W2A8:
        case BITQ_WNAM: {
            const int64_t G = K / 128;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t g = 0; g < G; ++g) {
                    uint32_t v = static_cast<uint32_t>(s->delta[n * G + g]) |
                                 (static_cast<uint32_t>(s->zero[n * G + g]) << 16);
                    size_t off = L.off_c0 + 4 * static_cast<size_t>(((n / 64) * L.Tb + g) * 64 + n % 64);
                    std::memcpy(dst + off, &v, 4);
                }
            break;
        }
        case BITQ_BVSR4: {
            const int64_t G = K / 32;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t g = 0; g < G; ++g) {
                    size_t off = L.off_c0 + static_cast<size_t>((((n / 64) * L.Tb + g / 4) * 64 + n % 64) * 4 + g % 4);
                    dst[off] = s->idx[n * G + g];
                }
            // c_j 2^-j (exact), then b: the kernel's products of sub-word j
            // carry the factor 2^j
            float* cache = reinterpret_cast<float*>(dst + L.off_c1);
            for (int e = 0; e < 256; ++e) {
                for (int j = 0; j < 4; ++j) cache[5 * e + j] = std::ldexp(s->cache[5 * e + j], -j);
                cache[5 * e + 4] = s->cache[5 * e + 4];
            }
            break;
        }
    }
}

bitq_status pack_impl(const bitq_wdesc& d, const bitq_logical* s, void* dstv, size_t dst_bytes, int nthreads) {
    BlobLayout L = blob_layout(d);
    if (dst_bytes < L.total)
        return fail(BITQ_E_CAPACITY, "dst has %zu bytes, blob needs %zu", dst_bytes, L.total);
    uint8_t* dst = static_cast<uint8_t*>(dstv);
    std::memset(dst, 0, L.total);
    write_header(d, L, dst);
    const int64_t N = d.N, K = d.K;
    switch (d.fmt) {
        case BITQ_SIGN1:
        case BITQ_RABIT:
            pack_planes(d, L, dst, nthreads,
                        [&](int64_t p, int64_t n, int64_t k) { return s->sign[(p * N + n) * K + k] > 0; });
            break;
        case BITQ_TERNARY:
        case BITQ_HGF:
            pack_planes(d, L, dst, nthreads, [&](int64_t p, int64_t n, int64_t k) {
                int8_t t = s->tern[n * K + k];
                return p == 0 ? t == 1 : t == -1;
            });
            break;
        case BITQ_W2A8:
        case BITQ_WNAM:
            pack_planes(d, L, dst, nthreads,
                        [&](int64_t p, int64_t n, int64_t k) { return (s->code[n * K + k] >> p) & 1; });
            break;
        case BITQ_BVSR4:
            // plane p of a 32-group holds its inputs 8p .. 8p + 7, one per
            // nibble: bit 4e + j of the word = beta_j of input 8p + bvsr_nibble_input(e)
            pack_planes(d, L, dst, nthreads, [&](int64_t p, int64_t n, int64_t k) {
                const int64_t i = k & 31, in = (k & ~int64_t(31)) + 8 * p + bvsr_nibble_input(static_cast<int>(i >> 2));
                return (s->code[n * K + in] >> (i & 3)) & 1;
            });
            break;
    }
    pack_coefficients(d, L, s, dst);
    if (d.fmt == BITQ_SIGN1 || d.fmt == BITQ_RABIT) {
        // header bound max_k |h_p[k]| (1 for SIGN1): the float GEMV scales its
        // split-k fixed-point sums from it
        float hb[3] = {0.0f, 0.0f, 0.0f};
        for (int64_t p = 0; p < L.P; ++p) {
            double m = d.fmt == BITQ_SIGN1 ? 1.0 : 0.0;
            if (d.fmt == BITQ_RABIT)
                for (int64_t k = 0; k < K; ++k) {
                    const double a = std::fabs(f16_to_f64(s->h[p * K + k]));
                    m = (a > m || a != a) ? a : m;  // NaN propagates
                }
            hb[p] = static_cast<float>(m);
        }
        std::memcpy(dst + kHdrHBound, hb, sizeof(hb));
    }
    if (d.fmt == BITQ_HGF) {
        // the gate tanh(alpha) is a property of the weights: computed here
        // once (fp64, rounded to fp32); amax_a bounds the activation step's
        // fixed-point sums
        const float alpha = s->lora_alpha;
        const float gate = static_cast<float>(std::tanh(static_cast<double>(alpha)));
        double am = 0.0;
        for (int64_t i = 0; i < K * d.rank; ++i) am = std::max(am, std::fabs(f16_to_f64(s->lora_a[i])));
        const float amax_a = static_cast<float>(am);
        std::memcpy(dst + kHdrAlpha, &alpha, 4);
        std::memcpy(dst + kHdrGate, &gate, 4);
        std::memcpy(dst + kHdrAmaxA, &amax_a, 4);
    }
    return ok();
}

// -------------------------------------------------------------- quantizers
// [HGF] §1.2 ternary quantizer: gamma = mean |W| (fp64 sum, stored fp32),
// T = clamp(rint(W / gamma), -1, 1) with the division in fp32.
float quantize_ternary(const float* W, int64_t count, std::vector<int8_t>& T) {
    double sabs = 0.0;
    for (int64_t i = 0; i < count; ++i) sabs += std::fabs(static_cast<double>(W[i]));
    const float gamma = static_cast<float>(sabs / static_cast<double>(count));
    T.assign(count, 0);
    if (gamma > 0.0f) {
        for (int64_t i = 0; i < count; ++i) {
            float r = std::nearbyint(W[i] / gamma);  // fp32 division, then RNE
            T[i] = static_cast<int8_t>(std::min(1.0f, std::max(-1.0f, r)));
        }
    }
    return gamma;
}

// [BitNet] §2.1: sign(x) = +1 if x >= 0 else -1.
inline int8_t sign_pm1(double v) { return v >= 0 ? 1 : -1; }

// Leading singular pair of a non-negative N x K matrix (row-major fp64) by
// power iteration: v0 = 1/sqrt(K); u = Av/|Av|; v = A^T u/|A^T u|; 30 times;
// sigma = u^T A v.  Returns false for a zero matrix.
bool rank1_fit(const std::vector<double>& A, int64_t N, int64_t K, int iters, int nthreads,
               std::vector<double>& u, std::vector<double>& v, double& sigma) {
    u.assign(N, 0.0);
    v.assign(K, 1.0 / std::sqrt(static_cast<double>(K)));
    std::vector<double> Av(N);
    const int64_t chunk = 256;
    const int64_t nch = (N + chunk - 1) / chunk;
    std::vector<std::vector<double>> part(nch, std::vector<double>(K));
    auto matvec = [&](const std::vector<double>& x, std::vector<double>& y) {  // y = A x
        parallel_for(N, nthreads, [&](int64_t n) {
            double s = 0.0;
            const double* a = &A[n * K];
            for (int64_t k = 0; k < K; ++k) s += a[k] * x[k];
            y[n] = s;
        });
    };
    auto matvec_t = [&](const std::vector<double>& x, std::vector<double>& y) {  // y = A^T x
        parallel_for(nch, nthreads, [&](int64_t c) {
            std::vector<double>& pp = part[c];
            std::fill(pp.begin(), pp.end(), 0.0);
            for (int64_t n = c * chunk; n < std::min(N, (c + 1) * chunk); ++n) {
                const double* a = &A[n * K];
                const double xn = x[n];
                for (int64_t k = 0; k < K; ++k) pp[k] += a[k] * xn;
            }
        });
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t c = 0; c < nch; ++c) s += part[c][k];
            y[k] = s;
        }
    };
    auto norm = [](const std::vector<double>& x) {
        double s = 0.0;
        for (double t : x) s += t * t;
        return std::sqrt(s);
    };
    for (int it = 0; it < iters; ++it) {
        matvec(v, u);
        double nu = norm(u);
        if (nu == 0.0) return false;
        for (auto& t : u) t /= nu;
        matvec_t(u, v);
        double nv = norm(v);
        if (nv == 0.0) return false;
        for (auto& t : v) t /= nv;
    }
    matvec(v, Av);
    double s = 0.0;
    for (int64_t n = 0; n < N; ++n) s += u[n] * Av[n];
    sigma = s;
    return true;
}

bitq_status quantize_rabit(const bitq_wdesc& d, const float* W, std::vector<int8_t>& B,
                           std::vector<uint16_t>& g, std::vector<uint16_t>& h, int nthreads) {
    const int64_t N = d.N, K = d.K, P = d.planes;
    std::vector<double> R(N * K), A(N * K);
    for (int64_t i = 0; i < N * K; ++i) R[i] = W[i];
    B.assign(P * N * K, 0);
    g.assign(P * N, 0);
    h.assign(P * K, 0);
    std::vector<double> u, v;
    for (int64_t p = 0; p < P; ++p) {
        int8_t* Bp = &B[p * N * K];
        for (int64_t i = 0; i < N * K; ++i) {
            Bp[i] = sign_pm1(R[i]);
            A[i] = std::fabs(R[i]);
        }
        double sigma = 0.0;
        if (rank1_fit(A, N, K, 30, nthreads, u, v, sigma)) {
            double r = std::sqrt(std::max(sigma, 0.0));
            for (int64_t n = 0; n < N; ++n) g[p * N + n] = f64_to_f16(r * u[n]);
            for (int64_t k = 0; k < K; ++k) h[p * K + k] = f64_to_f16(r * v[k]);
        }
        // next residual from the stored fp16 scales: R -= (g B) h
        for (int64_t n = 0; n < N; ++n) {
            const double gn = f16_to_f64(g[p * N + n]);
            for (int64_t k = 0; k < K; ++k)
                R[n * K + k] = R[n * K + k] - (gn * Bp[n * K + k]) * f16_to_f64(h[p * K + k]);
        }
    }
    return BITQ_OK;
}

// [RaBiT] §2.2 iterative residual SVID: Gauss-Seidel sweeps over the paths.
// Path p is refitted to what the other paths leave,
//   T = W - sum_{q != p} (g_q B_q) h_q   (stored fp16 scales, paths in order),
//   B_p = sign(T), (g_p, h_p) = rank-1 fit of |T|,
// the exact minimizer for that path, so the error does not grow except by
// the fp16 rounding of g and h.  T is rebuilt from the int8 signs and the fp16
// scales each time (no fp64 copy of the paths is kept).
void refine_rabit_svid(const bitq_wdesc& d, const float* W, std::vector<int8_t>& B, std::vector<uint16_t>& g,
                       std::vector<uint16_t>& h, int sweeps, int nthreads) {
    const int64_t N = d.N, K = d.K, P = d.planes;
    std::vector<double> A(N * K), hq(P * K);
    std::vector<double> u, v;
    for (int s = 0; s < sweeps; ++s)
        for (int64_t p = 0; p < P; ++p) {
            for (int64_t i = 0; i < P * K; ++i) hq[i] = f16_to_f64(h[i]);
            int8_t* Bp = &B[p * N * K];
            parallel_for(N, nthreads, [&](int64_t n) {
                for (int64_t k = 0; k < K; ++k) {
                    double t = W[n * K + k];
                    for (int64_t q = 0; q < P; ++q)
                        if (q != p)
                            t = t - (f16_to_f64(g[q * N + n]) * B[(q * N + n) * K + k]) * hq[q * K + k];
                    Bp[n * K + k] = sign_pm1(t);
                    A[n * K + k] = std::fabs(t);
                }
            });
            double sigma = 0.0;
            if (rank1_fit(A, N, K, 30, nthreads, u, v, sigma)) {
                const double r = std::sqrt(std::max(sigma, 0.0));
                for (int64_t n = 0; n < N; ++n) g[p * N + n] = f64_to_f16(r * u[n]);
                for (int64_t k = 0; k < K; ++k) h[p * K + k] = f64_to_f16(r * v[k]);
            } else {
                for (int64_t n = 0; n < N; ++n) g[p * N + n] = 0;
                for (int64_t k = 0; k < K; ++k) h[p * K + k] = 0;
            }
        }
}

// [ABQ] §3.2 Eq. (3) with gamma = 0 and clip factors 1: asymmetric min/max
// round-to-nearest per group of 128 inputs on L = 2^planes - 1 steps (W2A8:
// 2 planes, L = 3; WNAM: 1..4 planes).  delta = fl16((hi - lo)/L),
// z = clamp(rint(-lo/delta), 0, L), q = clamp(rint(W/delta) + z, 0, L); a
// group with a zero step gets delta = 1, z = 0, q = 0.
void quantize_w2a8(const bitq_wdesc& d, const float* W, std::vector<uint8_t>& q, std::vector<uint16_t>& delta,
                   std::vector<uint16_t>& zero, int nthreads) {
    const int64_t N = d.N, K = d.K, G = K / 128;
    const double L = static_cast<double>((1 << d.planes) - 1);
    q.assign(N * K, 0);
    delta.assign(N * G, 0);
    zero.assign(N * G, 0);
    parallel_for(N, nthreads, [&](int64_t n) {
        for (int64_t gi = 0; gi < G; ++gi) {
            const float* w = W + n * K + gi * 128;
            double lo = w[0], hi = w[0];
            for (int i = 1; i < 128; ++i) {
                lo = std::min(lo, static_cast<double>(w[i]));
                hi = std::max(hi, static_cast<double>(w[i]));
            }
            uint16_t d16 = f64_to_f16((hi - lo) / L);
            double dl = f16_to_f64(d16);
            if (dl == 0.0) {  // degenerate group: delta = 1, z = 0, q = 0
                delta[n * G + gi] = 0x3C00;
                zero[n * G + gi] = 0;
                continue;
            }
            double z = std::min(L, std::max(0.0, std::nearbyint(-lo / dl)));
            delta[n * G + gi] = d16;
            zero[n * G + gi] = f64_to_f16(z);
            for (int i = 0; i < 128; ++i) {
                double t = std::nearbyint(static_cast<double>(w[i]) / dl) + z;
                q[n * K + gi * 128 + i] = static_cast<uint8_t>(std::min(L, std::max(0.0, t)));
            }
        }
    });
}

// [ABQ] §3.3 bit balance: symmetric five-level grid {-2..2} per 128-group,
// delta = fl16(max|W| / 2), code = clamp(rint(W / delta), -2, 2) + 2, z = 2;
// a zero step gives delta = 1 and code 2.  fp64 arithmetic from the fp32
// weights and the fp16 step.
void quantize_bit_balance(const bitq_wdesc& d, const float* W, std::vector<uint8_t>& q,
                          std::vector<uint16_t>& delta, std::vector<uint16_t>& zero, int nthreads) {
    const int64_t N = d.N, K = d.K, G = K / 128;
    q.assign(N * K, 2);
    delta.assign(N * G, 0x3C00);
    zero.assign(N * G, 0x4000);  // fp16 2.0
    parallel_for(N, nthreads, [&](int64_t n) {
        for (int64_t gi = 0; gi < G; ++gi) {
            const float* w = W + n * K + gi * 128;
            double amax = 0.0;
            for (int i = 0; i < 128; ++i) amax = std::max(amax, std::fabs(static_cast<double>(w[i])));
            const uint16_t d16 = f64_to_f16(amax / 2.0);
            const double dl = f16_to_f64(d16);
            if (dl == 0.0) continue;  // degenerate group: delta = 1, code 2
            delta[n * G + gi] = d16;
            for (int i = 0; i < 128; ++i) {
                const double t = std::min(2.0, std::max(-2.0, std::nearbyint(static_cast<double>(w[i]) / dl)));
                q[n * K + gi * 128 + i] = static_cast<uint8_t>(t + 2.0);
            }
        }
    });
}

// [BVSR] introduction: coefficient sets are scaled/shifted subset sums of a
// geometric series; 256 sets from 16 ratios x 16 spans (group-range quantiles).
void bvsr_cache(const bitq_wdesc& d, const float* W, float* cache) {
    const int64_t NG = static_cast<int64_t>(d.N) * (d.K / 32);
    std::vector<double> spans(NG);
    for (int64_t gi = 0; gi < NG; ++gi) {
        const float* w = W + gi * 32;
        double lo = w[0], hi = w[0];
        for (int i = 1; i < 32; ++i) {
            lo = std::min(lo, static_cast<double>(w[i]));
            hi = std::max(hi, static_cast<double>(w[i]));
        }
        spans[gi] = hi - lo;
    }
    std::sort(spans.begin(), spans.end());
    auto quantile = [&](double qf) {  // linear interpolation, fixed arithmetic order
        double pos = qf * static_cast<double>(NG - 1);
        int64_t i = static_cast<int64_t>(std::floor(pos));
        if (i >= NG - 1) return spans[NG - 1];
        double frac = pos - static_cast<double>(i);
        return spans[i] + frac * (spans[i + 1] - spans[i]);
    };
    for (int i = 0; i < 16; ++i) {
        double r = 1.6 + (0.8 * i) / 15.0;
        double r2 = r * r, r3 = r2 * r;
        double denom = 1.0 + r + r2 + r3;
        for (int j = 0; j < 16; ++j) {
            double L = quantile((j + 0.5) / 16.0);
            double a = L / denom;
            float* c = cache + 5 * (16 * i + j);
            c[0] = static_cast<float>(a);
            c[1] = static_cast<float>(a * r);
            c[2] = static_cast<float>(a * r2);
            c[3] = static_cast<float>(a * r3);
            c[4] = static_cast<float>(-L / 2.0);
        }
    }
}

// Exhaustive per-group search over the 256 sets: each weight takes the nearest
// of the set's 16 points (ties -> smaller code), the set of least group SSE
// wins (ties -> lower id).  Nearest points come from the sorted point list
// (only the two bracketing values can be nearest); a set is abandoned as soon
// as its running SSE exceeds the best one, which cannot change the result.
void bvsr_search(const bitq_wdesc& d, const float* W, const float* cache, std::vector<uint8_t>& code,
                 std::vector<uint8_t>& idx, int nthreads) {
    const int64_t N = d.N, K = d.K, G = K / 32;
    struct Set {
        double val[16];   // sorted point values
        uint8_t code[16]; // their codes (ties in value sorted by code)
    };
    std::vector<Set> sets(256);
    for (int s = 0; s < 256; ++s) {
        const float* c = cache + 5 * s;
        std::pair<double, int> pts[16];
        for (int cd = 0; cd < 16; ++cd) {
            double v = static_cast<double>(c[4]);
            for (int k = 0; k < 4; ++k)
                if ((cd >> k) & 1) v = v + static_cast<double>(c[k]);
            pts[cd] = {v, cd};
        }
        std::sort(pts, pts + 16);
        for (int t = 0; t < 16; ++t) {
            sets[s].val[t] = pts[t].first;
            sets[s].code[t] = static_cast<uint8_t>(pts[t].second);
        }
    }
    code.assign(N * K, 0);
    idx.assign(N * G, 0);
    auto nearest = [](const Set& S, double w, double& d2out) -> uint8_t {
        // first index with val > w
        int lo = 0, hi = 16;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (S.val[mid] > w) hi = mid; else lo = mid + 1;
        }
        double bd = INFINITY;
        int bc = 16;
        auto consider = [&](int t) {
            // lowest code among equal values is the first of the run
            while (t > 0 && S.val[t - 1] == S.val[t]) --t;
            double df = w - S.val[t];
            double d2 = df * df;
            int c = S.code[t];
            if (d2 < bd || (d2 == bd && c < bc)) {
                bd = d2;
                bc = c;
            }
        };
        if (lo > 0) consider(lo - 1);
        if (lo < 16) consider(lo);
        d2out = bd;
        return static_cast<uint8_t>(bc);
    };
    parallel_for(N, nthreads, [&](int64_t n) {
        uint8_t cbuf[32], best_codes[32];
        for (int64_t gi = 0; gi < G; ++gi) {
            const float* w = W + n * K + gi * 32;
            double best = INFINITY;
            int best_id = 0;
            for (int s = 0; s < 256; ++s) {
                double sse = 0.0;
                bool abandoned = false;
                for (int e = 0; e < 32; ++e) {
                    double d2;
                    cbuf[e] = nearest(sets[s], static_cast<double>(w[e]), d2);
                    sse = sse + d2;
                    if (sse > best) {
                        abandoned = true;
                        break;
                    }
                }
                if (abandoned) continue;
                if (sse < best) {  // equal SSE keeps the lower id found first
                    best = sse;
                    best_id = s;
                    std::memcpy(best_codes, cbuf, 32);
                }
            }
            idx[n * G + gi] = static_cast<uint8_t>(best_id);
            std::memcpy(&code[n * K + gi * 32], best_codes, 32);
        }
    });
}

}  // namespace

// ------------------------------------------------------------- layouts/plans
BlobLayout blob_layout(const bitq_wdesc& d) {
    BlobLayout L{};
    L.Np = round_up(d.N, kRowTile);
    L.Kp = round_up(d.K, kKBlock);
    L.P = d.planes;
    L.Tn = L.Np / kRowTile;
    L.Tb = L.Kp / kKBlock;
    L.off_planes = kHeaderBytes;
    L.planes_bytes = static_cast<size_t>(L.Tn * L.Tb * L.P) * 1024;
    L.off_c0 = align256(L.off_planes + L.planes_bytes);
    switch (d.fmt) {
        case BITQ_SIGN1: L.c0_bytes = 4 * L.Np; L.c1_bytes = 0; break;
        case BITQ_RABIT: L.c0_bytes = 2 * L.P * L.Np; L.c1_bytes = 2 * L.P * L.Kp; break;
        case BITQ_TERNARY: L.c0_bytes = 4; L.c1_bytes = 0; break;
        case BITQ_W2A8:
        case BITQ_WNAM: L.c0_bytes = 4 * L.Np * L.Tb; L.c1_bytes = 0; break;
        case BITQ_BVSR4: L.c0_bytes = L.Np * (L.Kp / 32); L.c1_bytes = 256 * 5 * 4; break;
        case BITQ_HGF: L.c0_bytes = 4; L.c1_bytes = 2 * static_cast<size_t>(d.rank) * L.Kp; break;
        default: L.c0_bytes = L.c1_bytes = 0;
    }
    L.off_c1 = align256(L.off_c0 + L.c0_bytes);
    L.off_c2 = align256(L.off_c1 + L.c1_bytes);
    L.c2_bytes = d.fmt == BITQ_HGF ? 2 * static_cast<size_t>(L.Np) * d.rank : 0;
    L.total = align256(L.off_c2 + L.c2_bytes);
    return L;
}

ActLayout act_layout(int M, int K, int rank) {
    ActLayout A{};
    A.M = M;
    A.K = K;
    A.Kp = round_up(K, kKBlock);
    A.Kw = A.Kp / 32;
    A.off_planes = 0;
    A.off_S = align256(static_cast<size_t>(M * A.Kw) * 32);
    A.off_q = align256(A.off_S + static_cast<size_t>(M * A.Kw) * 4);
    A.off_qm = align256(A.off_q + static_cast<size_t>(M * A.Kp));
    A.off_d = align256(A.off_qm + 16 * static_cast<size_t>((M + 15) / 16) * A.Kp);  // whole token tiles
    A.off_amax = align256(A.off_d + 4 * static_cast<size_t>(M));
    A.off_h = align256(A.off_amax + 4 * static_cast<size_t>(M));
    A.total = align256(A.off_h + 4 * static_cast<size_t>(M) * rank);
    return A;
}

BinActLayout binact_layout(int M, int K) {
    BinActLayout A{};
    A.M = M;
    A.K = K;
    A.Kp = round_up(K, kKBlock);
    A.Kw = A.Kp / 32;
    A.off_beta = align256(4 * static_cast<size_t>(M) * A.Kw);
    A.total = align256(A.off_beta + 4 * static_cast<size_t>(M));
    return A;
}

Plan make_plan(const bitq_wdesc& d, int M, bool fused) {
    Plan p{};
    const bool lut = (d.fmt == BITQ_SIGN1 || d.fmt == BITQ_RABIT);
    const int64_t Np = round_up(d.N, kRowTile);
    const int64_t NB = round_up(d.K, kKBlock) / kKBlock;
    p.M = M;
    if (!lut) {
        // Integer formats: one workgroup of 256 lanes per rows_per_wg rows
        // covers the whole k range (256/rows_per_wg k-groups x
        // blocks_per_split blocks per round); no workspace.
        // Rows per workgroup (16 or 8): 8 rows double the waves of layers
        // with fewer than 16384 rows, which keeps more waves per SIMD to hide
        // the popcount chains (measured faster on every such layer shape).
        // WNAM is built for 8 rows (16 with the fused quantizer) and 1, 2, 4
        // or 8 blocks per lane only.  With the fused activation quantizer
        // every workgroup repeats the quantization, and 16 rows per workgroup
        // halve that work: faster from 4096 rows on (measured 5.9 against
        // 6.5 us at 11008x4096).
        const bool wnam = d.fmt == BITQ_WNAM;
        const int rg = fused ? (d.N >= 4096 ? 16 : 8) : (d.N >= 16384 && !wnam ? 16 : 8);
        const bool wide = rg == 16 && NB > kWideMinBlocks &&
                          (fused || (d.fmt == BITQ_BVSR4 && M == 1 && NB <= 4 * 32));  // BVSR4: one round
        p.waves_per_wg = wide ? 8 : 4;
        const int64_t kgroups = 64 * p.waves_per_wg / rg;
        const int64_t need = (NB + kgroups - 1) / kgroups;
        const int sizes[6] = {1, 2, 3, 4, 6, 8};
        p.blocks_per_split = 8;
        for (int sz : sizes)
            if (sz >= need && !(wnam && (sz == 3 || sz == 6))) {
                p.blocks_per_split = sz;
                break;
            }
        p.rows_per_wg = rg;
        p.row_groups = static_cast<int>((d.N + rg - 1) / rg);
        p.splits = 1;
        p.off_partials = 0;
        p.ws_bytes = 0;
        // the contraction is compute-bound on the VALU from 2 tokens on; from
        // mfma_min_tokens(fmt) tokens the int8 matrix-core kernel is faster
        // and takes over (HGF and BVSR4 stay on the VALU)
        p.mfma = mfma_min_tokens(d.fmt) > 0 && M >= mfma_min_tokens(d.fmt);
        return p;
    }
    p.waves_per_wg = lut ? 4 : 1;
    p.rows_per_wg = kRowTile * p.waves_per_wg;
    p.row_groups = static_cast<int>((Np + p.rows_per_wg - 1) / p.rows_per_wg);
    // Blocks per split are compile-time variants of the kernel (1, 2, 4, 8):
    // the largest of 1, 2, 4 that still gives at least 512 workgroups, and
    // never more than 63 splits (the split-k word counts arrivals in 6 bits).
    const int64_t target = 512;
    int kb = 4;
    while (kb > 1 && p.row_groups * ((NB + kb - 1) / kb) < target && (NB + kb / 2 - 1) / (kb / 2) <= 63) kb >>= 1;
    while ((NB + kb - 1) / kb > 63) kb *= 2;  // K > 32256: 8 blocks per split (K <= 64512, checked)
    p.blocks_per_split = kb;
    p.splits = static_cast<int>((NB + p.blocks_per_split - 1) / p.blocks_per_split);
    p.off_partials = 0;
    p.ws_bytes = p.splits > 1 ? align256(static_cast<size_t>(M) * Np * 8) : 0;  // one split-k word per row
    return p;
}

MfmaShape mfma_shape(const bitq_wdesc& d, int M) {
    // TT token tiles of 16.  One workgroup per CU (at most kWholeRowGrid, at
    // most one per 16-row sub-tile) of KW waves over k: one token tile takes
    // 16 waves (four per SIMD, up to 128 registers each; measured faster
    // than 8 waves: W2A8 11008x4096 M = 16 7.94 -> 7.01 us), more tiles 8
    // (two per SIMD, up to 256 registers each).  Each wave issues the loads
    // of CH blocks together: its NB / KW blocks in as few rounds of at most
    // 2 blocks as possible, evenly filled.
    MfmaShape s{};
    s.TT = std::min(4, (M + 15) / 16);
    // sub-tiles per pass: one when every workgroup owns at most one (up to
    // 4096 rows), so that no surplus slot repeats the products of the last
    s.RS = round_up(d.N, kRowTile) / 16 <= kWholeRowGrid ? 1 : kMfmaSubs;
    const int64_t NB = round_up(d.K, kKBlock) / kKBlock;
    const int64_t nsub = round_up(d.N, kRowTile) / 16;
    s.KW = s.TT == 1 ? 16 : 8;
    const int64_t cmax = 2;
    const int64_t nbw = (NB + s.KW - 1) / s.KW, rounds = (nbw + cmax - 1) / cmax;
    s.CH = static_cast<int>((nbw + rounds - 1) / rounds);
    s.grid = static_cast<int>(std::min<int64_t>(kWholeRowGrid, nsub));
    s.block = 64 * s.KW;
    return s;
}

LaunchShape launch_shape(const bitq_wdesc& d, int M, int x_dtype, uint32_t flags) {
    LaunchShape ls{0, 256};
    const int64_t tiles = round_up(d.N, kRowTile) / kRowTile;
    if (x_dtype == BITQ_DT_BINARY) {  // XNOR kernel: 8 rows per workgroup
        ls.grid = xcd_row_groups(tiles, 8);
        return ls;
    }
    const bool fused = (flags & BITQ_F_FUSE_QUANT) != 0;
    const Plan p = make_plan(d, M, fused);
    if (d.fmt == BITQ_SIGN1 || d.fmt == BITQ_RABIT) {
        ls.grid = p.row_groups * p.splits;
    } else if (p.mfma) {
        const MfmaShape m = mfma_shape(d, M);
        ls.grid = m.grid;
        ls.block = m.block;
    } else {
        ls.grid = xcd_row_groups(tiles, p.rows_per_wg);
        ls.block = 64 * p.waves_per_wg;
    }
    return ls;
}

}  // namespace bitq

using namespace bitq;

// ---------------------------------------------------------------- C ABI
extern "C" {

int32_t bitq_version(void) { return BITQ_VERSION; }

const char* bitq_last_error(void) { return g_error.c_str(); }

bitq_status bitq_packed_size(const bitq_wdesc* desc, size_t* bytes) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (!bytes) return fail(BITQ_E_ARG, "bytes is NULL");
    *bytes = blob_layout(*desc).total;
    return ok();
}

bitq_status bitq_pack_weights(const bitq_wdesc* desc, const bitq_logical* src, void* dst, size_t dst_bytes) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (!src) return fail(BITQ_E_ARG, "src is NULL");
    if (!dst) return fail(BITQ_E_ARG, "dst is NULL");
    size_t need = blob_layout(*desc).total;
    if (dst_bytes < need) return fail(BITQ_E_CAPACITY, "dst has %zu bytes, blob needs %zu", dst_bytes, need);
    if ((s = check_logical(*desc, src))) return s;
    try {
        return pack_impl(*desc, src, dst, dst_bytes, 0);
    } catch (...) {
        return fail(BITQ_E_ARG, "host allocation failed while packing");
    }
}

bitq_status bitq_quantize_weights(const bitq_wdesc* desc, const float* W, void* dst, size_t dst_bytes,
                                  int32_t nthreads) {
    bitq_quant_opts opts{};
    return bitq_quantize_weights_opts(desc, W, &opts, dst, dst_bytes, nthreads);
}

bitq_status bitq_quantize_weights_opts(const bitq_wdesc* desc, const float* W, const bitq_quant_opts* opts,
                                       void* dst, size_t dst_bytes, int32_t nthreads) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (!opts) return fail(BITQ_E_ARG, "opts is NULL");
    for (int i = 0; i < 6; ++i)
        if (opts->reserved[i]) return fail(BITQ_E_ARG, "opts->reserved[%d] must be 0", i);
    if (opts->wnam_bit_balance != 0 && opts->wnam_bit_balance != 1)
        return fail(BITQ_E_ARG, "wnam_bit_balance must be 0 or 1");
    if (opts->wnam_bit_balance && (desc->fmt != BITQ_WNAM || desc->planes != 3))
        return fail(BITQ_E_ARG, "wnam_bit_balance needs the WNAM format with planes = 3 (codes 0..4)");
    if (opts->rabit_svid_sweeps < 0 || opts->rabit_svid_sweeps > 1000)
        return fail(BITQ_E_ARG, "rabit_svid_sweeps=%d out of range [0, 1000]", opts->rabit_svid_sweeps);
    if (opts->rabit_svid_sweeps && desc->fmt != BITQ_RABIT)
        return fail(BITQ_E_ARG, "rabit_svid_sweeps applies to the RABIT format only");
    if (!W) return fail(BITQ_E_ARG, "W is NULL");
    if (!dst) return fail(BITQ_E_ARG, "dst is NULL");
    const bitq_wdesc d = *desc;
    size_t need = blob_layout(d).total;
    if (dst_bytes < need) return fail(BITQ_E_CAPACITY, "dst has %zu bytes, blob needs %zu", dst_bytes, need);
    const int64_t N = d.N, K = d.K;
    for (int64_t i = 0; i < N * K; ++i)
        if (!std::isfinite(W[i])) return fail(BITQ_E_ARG, "W[%lld] is not finite", (long long)i);
    try {
        bitq_logical lg{};
        std::vector<int8_t> i8;
        std::vector<uint8_t> u8, idx;
        std::vector<uint16_t> g, h, delta, zero;
        std::vector<float> alpha, cache;
        switch (d.fmt) {
            case BITQ_SIGN1: {
                i8.resize(N * K);
                alpha.resize(N);
                for (int64_t n = 0; n < N; ++n) {
                    double sabs = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double w = W[n * K + k];
                        i8[n * K + k] = sign_pm1(w);
                        sabs += std::fabs(w);
                    }
                    alpha[n] = static_cast<float>(sabs / static_cast<double>(K));
                }
                lg.sign = i8.data();
                lg.alpha = alpha.data();
                break;
            }
            case BITQ_RABIT:
                quantize_rabit(d, W, i8, g, h, nthreads);
                refine_rabit_svid(d, W, i8, g, h, opts->rabit_svid_sweeps, nthreads);
                lg.sign = i8.data();
                lg.g = g.data();
                lg.h = h.data();
                break;
            case BITQ_TERNARY:
                lg.gamma = quantize_ternary(W, N * K, i8);
                lg.tern = i8.data();
                break;
            case BITQ_W2A8:
            case BITQ_WNAM:
                if (opts->wnam_bit_balance)
                    quantize_bit_balance(d, W, u8, delta, zero, nthreads);
                else
                    quantize_w2a8(d, W, u8, delta, zero, nthreads);
                lg.code = u8.data();
                lg.delta = delta.data();
                lg.zero = zero.data();
                break;
            case BITQ_HGF:
                return fail(BITQ_E_UNSUPPORTED, "HGF layers are packed with bitq_pack_weights (the correction "
                                                "path's A, B and alpha are trained parameters, not derived from W)");
            case BITQ_BVSR4:
                cache.resize(256 * 5);
                bvsr_cache(d, W, cache.data());
                bvsr_search(d, W, cache.data(), u8, idx, nthreads);
                lg.code = u8.data();
                lg.idx = idx.data();
                lg.cache = cache.data();
                break;
        }
        return pack_impl(d, &lg, dst, dst_bytes, nthreads);
    } catch (...) {
        return fail(BITQ_E_ARG, "host allocation failed while quantizing");
    }
}

bitq_status bitq_quantize_weights_hgf(const bitq_wdesc* desc, const float* W, const uint16_t* lora_a,
                                      const uint16_t* lora_b, float lora_alpha, void* dst, size_t dst_bytes,
                                      int32_t nthreads) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (desc->fmt != BITQ_HGF) return fail(BITQ_E_ARG, "bitq_quantize_weights_hgf needs an HGF descriptor");
    if (!W) return fail(BITQ_E_ARG, "W is NULL");
    if (!dst) return fail(BITQ_E_ARG, "dst is NULL");
    const bitq_wdesc d = *desc;
    size_t need = blob_layout(d).total;
    if (dst_bytes < need) return fail(BITQ_E_CAPACITY, "dst has %zu bytes, blob needs %zu", dst_bytes, need);
    const int64_t N = d.N, K = d.K;
    for (int64_t i = 0; i < N * K; ++i)
        if (!std::isfinite(W[i])) return fail(BITQ_E_ARG, "W[%lld] is not finite", (long long)i);
    try {
        std::vector<int8_t> T;
        bitq_logical lg{};
        lg.gamma = quantize_ternary(W, N * K, T);
        lg.tern = T.data();
        lg.lora_a = lora_a;
        lg.lora_b = lora_b;
        lg.lora_alpha = lora_alpha;
        if ((s = check_logical(d, &lg))) return s;
        return pack_impl(d, &lg, dst, dst_bytes, nthreads);
    } catch (...) {
        return fail(BITQ_E_ARG, "host allocation failed while quantizing");
    }
}

bitq_status bitq_act_size(int32_t M, int32_t K, size_t* bytes) {
    if (!bytes) return fail(BITQ_E_ARG, "bytes is NULL");
    if (M < 1 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [1, 64]", M);
    if (K < 32 || K > (1 << 20) || K % 32) return fail(BITQ_E_SHAPE, "K=%d must be a multiple of 32 in [32, 2^20]", K);
    *bytes = act_layout(M, K).total;
    return ok();
}

bitq_status bitq_quantize_act(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K, void* act_dev,
                              size_t act_bytes, void* stream) {
    return bitq_quantize_act_bits(x_dev, x_dtype, M, K, 8, act_dev, act_bytes, stream);
}

bitq_status bitq_quantize_act_bits(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K, int32_t abits,
                                   void* act_dev, size_t act_bytes, void* stream) {
    size_t need = 0;
    bitq_status s = bitq_act_size(M, K, &need);
    if (s) return s;
    if (abits < 2 || abits > 8) return fail(BITQ_E_SHAPE, "abits=%d out of range [2, 8]", abits);
    if (!x_dev || !act_dev) return fail(BITQ_E_ARG, "x_dev/act_dev is NULL");
    if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
        return fail(BITQ_E_ARG, "x_dtype must be BITQ_DT_F32 or BITQ_DT_BF16");
    if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
    if (!aligned(act_dev, 256)) return fail(BITQ_E_ALIGN, "act_dev must be 256-byte aligned");
    if (act_bytes < need) return fail(BITQ_E_CAPACITY, "act buffer has %zu bytes, needs %zu", act_bytes, need);
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    e = launch_quantize_act(x_dev, x_dtype, M, K, abits, act_dev, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_hgf_act_size(const bitq_wdesc* desc, int32_t M, size_t* act_bytes, size_t* ws_bytes) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (desc->fmt != BITQ_HGF) return fail(BITQ_E_ARG, "bitq_hgf_act_size needs an HGF descriptor");
    if (!act_bytes || !ws_bytes) return fail(BITQ_E_ARG, "act_bytes/ws_bytes is NULL");
    if (M < 1 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [1, 64]", M);
    *act_bytes = act_layout(M, desc->K, desc->rank).total;
    *ws_bytes = align256(8 * static_cast<size_t>(M) * desc->rank);
    return ok();
}

bitq_status bitq_quantize_act_hgf(const bitq_wdesc* desc, const void* w_dev, const void* x_dev, int32_t x_dtype,
                                  int32_t M, void* act_dev, size_t act_bytes, void* ws_dev, size_t ws_bytes,
                                  void* stream) {
    size_t need_act = 0, need_ws = 0;
    bitq_status s = bitq_hgf_act_size(desc, M, &need_act, &need_ws);
    if (s) return s;
    if (!w_dev || !x_dev || !act_dev || !ws_dev) return fail(BITQ_E_ARG, "a device pointer is NULL");
    if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
        return fail(BITQ_E_ARG, "x_dtype must be BITQ_DT_F32 or BITQ_DT_BF16");
    if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
    if (!aligned(w_dev, 256) || !aligned(act_dev, 256) || !aligned(ws_dev, 256))
        return fail(BITQ_E_ALIGN, "w_dev, act_dev and ws_dev must be 256-byte aligned");
    if (act_bytes < need_act)
        return fail(BITQ_E_CAPACITY, "act buffer has %zu bytes, needs %zu", act_bytes, need_act);
    if (ws_bytes < need_ws) return fail(BITQ_E_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need_ws);
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    e = launch_quantize_act_hgf(x_dev, x_dtype, M, desc->K, desc->rank, w_dev, blob_layout(*desc), act_dev, ws_dev,
                                stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_quantize_act_hgf_noalloc(const bitq_wdesc* desc, const void* w_dev, const void* x_dev,
                                          int32_t x_dtype, int32_t M, void* act_dev, size_t act_bytes,
                                          void* stream) {
    size_t need_act = 0, need_ws = 0;
    bitq_status s = bitq_hgf_act_size(desc, M, &need_act, &need_ws);
    if (s) return s;
    const size_t words = static_cast<size_t>(M) * static_cast<size_t>(desc->rank);
    if (words > static_cast<size_t>(kNoAllocScratchWords))
        return fail(BITQ_E_CAPACITY, "M * rank = %zu exceeds the library scratch of %d words", words,
                    kNoAllocScratchWords);
    if (!w_dev || !x_dev || !act_dev) return fail(BITQ_E_ARG, "a device pointer is NULL");
    if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
        return fail(BITQ_E_ARG, "x_dtype must be BITQ_DT_F32 or BITQ_DT_BF16");
    if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
    if (!aligned(w_dev, 256) || !aligned(act_dev, 256))
        return fail(BITQ_E_ALIGN, "w_dev and act_dev must be 256-byte aligned");
    if (act_bytes < need_act)
        return fail(BITQ_E_CAPACITY, "act buffer has %zu bytes, needs %zu", act_bytes, need_act);
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    e = launch_quantize_act_hgf_noalloc(x_dev, x_dtype, M, desc->K, desc->rank, w_dev, blob_layout(*desc), act_dev,
                                        stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while setting up the scratch or launching", e);
    return ok();
}

bitq_status bitq_binact_size(int32_t M, int32_t K, size_t* bytes) {
    if (!bytes) return fail(BITQ_E_ARG, "bytes is NULL");
    if (M < 1 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [1, 64]", M);
    if (K < 32 || K > (1 << 20) || K % 32) return fail(BITQ_E_SHAPE, "K=%d must be a multiple of 32 in [32, 2^20]", K);
    *bytes = binact_layout(M, K).total;
    return ok();
}

bitq_status bitq_binarize_act(const void* x_dev, int32_t x_dtype, int32_t M, int32_t K, void* act_dev,
                              size_t act_bytes, void* stream) {
    size_t need = 0;
    bitq_status s = bitq_binact_size(M, K, &need);
    if (s) return s;
    if (!x_dev || !act_dev) return fail(BITQ_E_ARG, "x_dev/act_dev is NULL");
    if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
        return fail(BITQ_E_ARG, "x_dtype must be BITQ_DT_F32 or BITQ_DT_BF16");
    if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
    if (!aligned(act_dev, 256)) return fail(BITQ_E_ALIGN, "act_dev must be 256-byte aligned");
    if (act_bytes < need) return fail(BITQ_E_CAPACITY, "binary activation buffer has %zu bytes, needs %zu", act_bytes, need);
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    e = launch_binarize_act(x_dev, x_dtype, M, K, act_dev, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_workspace_size(const bitq_wdesc* desc, int32_t M, size_t* bytes) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (!bytes) return fail(BITQ_E_ARG, "bytes is NULL");
    if (M < 1 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [1, 64]", M);
    *bytes = make_plan(*desc, M).ws_bytes;
    return ok();
}

static bitq_status gemv_common(const bitq_wdesc* desc, const void* w_dev, const void* x_dev, int32_t x_dtype,
                               int32_t M, float* y_dev, void* ws_dev, size_t ws_bytes, uint32_t flags,
                               void* stream) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    const bitq_wdesc d = *desc;
    if (!w_dev || !x_dev || !y_dev) return fail(BITQ_E_ARG, "a device pointer is NULL");
    if (flags & ~(BITQ_F_ACC_INT32 | BITQ_F_FUSE_QUANT)) return fail(BITQ_E_ARG, "unknown flags 0x%x", flags);
    if (flags & BITQ_F_FUSE_QUANT) {  // raw x, quantized in the GEMV kernel's prologue
        if (d.fmt != BITQ_TERNARY && d.fmt != BITQ_W2A8 && d.fmt != BITQ_BVSR4 && d.fmt != BITQ_WNAM)
            return fail(BITQ_E_UNSUPPORTED, "BITQ_F_FUSE_QUANT supports TERNARY, W2A8, BVSR4 and WNAM");
        if (M != 1) return fail(BITQ_E_UNSUPPORTED, "BITQ_F_FUSE_QUANT is a bitq_gemv (M = 1) option");
        if (flags & BITQ_F_ACC_INT32)
            return fail(BITQ_E_UNSUPPORTED, "BITQ_F_FUSE_QUANT does not combine with BITQ_F_ACC_INT32");
        if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
            return fail(BITQ_E_ARG, "BITQ_F_FUSE_QUANT takes raw activations (BITQ_DT_F32 or BITQ_DT_BF16)");
        if (d.K > kMaxFusedK) return fail(BITQ_E_UNSUPPORTED, "BITQ_F_FUSE_QUANT supports K <= %d", kMaxFusedK);
        if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
        if (!aligned(w_dev, 256)) return fail(BITQ_E_ALIGN, "w_dev must be 256-byte aligned");
        if (!aligned(y_dev, 4)) return fail(BITQ_E_ALIGN, "y_dev must be 4-byte aligned");
        const Plan plan = make_plan(d, 1, true);
        int is950 = 0;
        int e = current_device_is_gfx950(&is950);
        if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
        if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
        e = launch_gemv_fused(d, plan, w_dev, x_dev, x_dtype, y_dev, stream);
        if (e == kLaunchNotBuilt) return fail(BITQ_E_UNSUPPORTED, "no fused kernel for this layer shape");
        if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
        return ok();
    }
    const bool binary = x_dtype == BITQ_DT_BINARY;
    if (binary) {  // fully binary XNOR path: SIGN1 weights x sign activations
        if (d.fmt != BITQ_SIGN1)
            return fail(BITQ_E_UNSUPPORTED, "binary activations (BITQ_DT_BINARY) need the SIGN1 format");
        if (!aligned(x_dev, 256)) return fail(BITQ_E_ALIGN, "binary activation buffer must be 256-byte aligned");
        if (!aligned(w_dev, 256)) return fail(BITQ_E_ALIGN, "w_dev must be 256-byte aligned");
        if (!aligned(y_dev, 4)) return fail(BITQ_E_ALIGN, "y_dev must be 4-byte aligned");
        int is950 = 0;
        int e = current_device_is_gfx950(&is950);
        if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
        if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
        e = launch_gemv_xnor(d, w_dev, x_dev, M, y_dev, flags, stream);
        if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
        return ok();
    }
    const bool float_fmt = (d.fmt == BITQ_SIGN1 || d.fmt == BITQ_RABIT);
    if (float_fmt) {
        if (M != 1) return fail(BITQ_E_UNSUPPORTED, "SIGN1/RABIT support M = 1 only");
        if (x_dtype != BITQ_DT_F32 && x_dtype != BITQ_DT_BF16)
            return fail(BITQ_E_ARG, "SIGN1/RABIT take raw activations (BITQ_DT_F32 or BITQ_DT_BF16)");
        if (flags & BITQ_F_ACC_INT32) return fail(BITQ_E_UNSUPPORTED, "BITQ_F_ACC_INT32 needs an integer format");
        if (!aligned(x_dev, 16)) return fail(BITQ_E_ALIGN, "x_dev must be 16-byte aligned");
    } else {
        if (x_dtype != BITQ_DT_ACT)
            return fail(BITQ_E_ARG, "TERNARY/W2A8/BVSR4/WNAM/HGF take an activation buffer (BITQ_DT_ACT)");
        if (!aligned(x_dev, 256)) return fail(BITQ_E_ALIGN, "activation buffer must be 256-byte aligned");
    }
    if (!aligned(w_dev, 256)) return fail(BITQ_E_ALIGN, "w_dev must be 256-byte aligned");
    if (!aligned(y_dev, 4)) return fail(BITQ_E_ALIGN, "y_dev must be 4-byte aligned");
    Plan plan = make_plan(d, M);
    if (plan.ws_bytes > 0) {
        if (!ws_dev) return fail(BITQ_E_ARG, "workspace is NULL");
        if (!aligned(ws_dev, 256)) return fail(BITQ_E_ALIGN, "workspace must be 256-byte aligned");
        if (ws_bytes < plan.ws_bytes)
            return fail(BITQ_E_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, plan.ws_bytes);
    }
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    if (float_fmt)
        e = launch_gemv_float(d, plan, w_dev, x_dev, x_dtype, y_dev, ws_dev, stream);
    else
        e = launch_gemv_int(d, plan, w_dev, x_dev, M, y_dev, ws_dev, flags, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_gemv(const bitq_wdesc* desc, const void* w_dev, const void* x_dev, int32_t x_dtype, float* y_dev,
                      void* ws_dev, size_t ws_bytes, uint32_t flags, void* stream) {
    return gemv_common(desc, w_dev, x_dev, x_dtype, 1, y_dev, ws_dev, ws_bytes, flags, stream);
}

bitq_status bitq_gemm_smallM(const bitq_wdesc* desc, const void* w_dev, const void* act_dev, int32_t M,
                             float* y_dev, void* ws_dev, size_t ws_bytes, uint32_t flags, void* stream) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (desc->fmt == BITQ_RABIT)
        return fail(BITQ_E_UNSUPPORTED, "bitq_gemm_smallM supports SIGN1 (binary activations), TERNARY, W2A8, "
                                        "BVSR4, WNAM and HGF");
    if (M < 2 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [2, 64]", M);
    const int32_t dt = desc->fmt == BITQ_SIGN1 ? BITQ_DT_BINARY : BITQ_DT_ACT;
    return gemv_common(desc, w_dev, act_dev, dt, M, y_dev, ws_dev, ws_bytes, flags, stream);
}

// ------------------------------------------------- measurement context kernels
bitq_status bitq_ctx_launch_shape(const bitq_wdesc* desc, int32_t M, int32_t x_dtype, uint32_t flags,
                                  int32_t* grid, int32_t* block) {
    bitq_status s = check_desc(desc);
    if (s) return s;
    if (!grid || !block) return fail(BITQ_E_ARG, "grid/block is NULL");
    if (M < 1 || M > 64) return fail(BITQ_E_SHAPE, "M=%d out of range [1, 64]", M);
    if (x_dtype < BITQ_DT_F32 || x_dtype > BITQ_DT_BINARY) return fail(BITQ_E_ARG, "unknown x_dtype %d", x_dtype);
    if (flags & ~(BITQ_F_ACC_INT32 | BITQ_F_FUSE_QUANT)) return fail(BITQ_E_ARG, "unknown flags 0x%x", flags);
    const LaunchShape ls = launch_shape(*desc, M, x_dtype, flags);
    *grid = ls.grid;
    *block = ls.block;
    return ok();
}

static bitq_status ctx_device_ok() {
    int is950 = 0;
    int e = current_device_is_gfx950(&is950);
    if (e) return fail(BITQ_E_DEVICE, "HIP error %d while querying the device", e);
    if (!is950) return fail(BITQ_E_UNSUPPORTED, "current device is not gfx950");
    return BITQ_OK;
}

bitq_status bitq_ctx_empty(int32_t grid, void* stream) {
    if (grid < 1 || grid > (1 << 20)) return fail(BITQ_E_SHAPE, "grid=%d out of range [1, 2^20]", grid);
    bitq_status s = ctx_device_ok();
    if (s) return s;
    int e = launch_ctx_empty(grid, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_ctx_stream(const void* src_dev, size_t bytes, int32_t grid, float* out_dev, int32_t nout,
                            void* stream) {
    if (!src_dev) return fail(BITQ_E_ARG, "src_dev is NULL");
    if (bytes == 0 || bytes % 16) return fail(BITQ_E_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    if (grid < 1 || grid > (1 << 20)) return fail(BITQ_E_SHAPE, "grid=%d out of range [1, 2^20]", grid);
    if (nout < 0 || nout > (1 << 24)) return fail(BITQ_E_SHAPE, "nout=%d out of range [0, 2^24]", nout);
    if (nout > 0 && !out_dev) return fail(BITQ_E_ARG, "out_dev is NULL");
    if (!aligned(src_dev, 16)) return fail(BITQ_E_ALIGN, "src_dev must be 16-byte aligned");
    if (out_dev && !aligned(out_dev, 4)) return fail(BITQ_E_ALIGN, "out_dev must be 4-byte aligned");
    bitq_status s = ctx_device_ok();
    if (s) return s;
    int e = launch_ctx_stream(src_dev, bytes, grid, out_dev, nout, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

bitq_status bitq_ctx_spin(int32_t microseconds, void* stream) {
    if (microseconds < 1 || microseconds > 10000)
        return fail(BITQ_E_SHAPE, "microseconds=%d out of range [1, 10000]", microseconds);
    bitq_status s = ctx_device_ok();
    if (s) return s;
    int e = launch_ctx_spin(microseconds, stream);
    if (e) return fail(BITQ_E_DEVICE, "HIP launch error %d", e);
    return ok();
}

}  // extern "C"
