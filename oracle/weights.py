"""Offline weight quantizers: fp32 W -> logical quantized form (test
infrastructure only).

Each function returns the *logical* form that both the oracle's GEMV and the
library's host packer consume (plain integer codes plus coefficient arrays):

  sign    : B int8 {+-1} [N,K], alpha float32 [N]
  rabit   : B int8 {+-1} [P,N,K], g float16 [P,N], h float16 [P,K]
  ternary : T int8 {-1,0,1} [N,K], gamma float32
  w2a8    : q uint8 {0..3} [N,K], delta float16 [N,K/128], zero float16 [N,K/128]
  bvsr    : code uint8 {0..15} [N,K], idx uint8 [N,K/32], cache float32 [256,5]
"""
from __future__ import annotations

import numpy as np

from .common import sign_pm1, to_f16


# ----------------------------------------------------------------- 1-bit sign
def quantize_sign(W: np.ndarray):
    """[BitNet] §2.1-2.2: w_b = sign(w) and W ~ alpha * sign(W).

    The page uses one alpha per matrix; the workload uses one per output row,
    alpha_n = mean_k |W[n,k]| (the per-matrix form is the special case of
    equal rows).  The mean is of |W| (|sign(W)| is identically 1), taken in
    fp64 and stored as fp32.
    """
    W = np.asarray(W, dtype=np.float32)
    B = sign_pm1(W)
    alpha = np.mean(np.abs(W.astype(np.float64)), axis=1).astype(np.float32)
    return B, alpha


# ------------------------------------------------------- RaBiT residual binary
def rank1_fit(A: np.ndarray, iters: int = 30):
    """Leading singular pair of a non-negative matrix by power iteration (fp64).

    v0 = 1/sqrt(K); repeat: u = A v / ||A v||, v = A^T u / ||A^T u||;
    sigma = u^T A v.  Returns (u, v, sigma); u, v >= 0 for A >= 0.
    A zero matrix gives u = v = 0, sigma = 0.
    """
    A = np.asarray(A, dtype=np.float64)
    N, K = A.shape
    v = np.full(K, 1.0 / np.sqrt(K))
    u = np.zeros(N)
    for _ in range(iters):
        u = A @ v
        nu = np.linalg.norm(u)
        if nu == 0.0:
            return np.zeros(N), np.zeros(K), 0.0
        u = u / nu
        v = A.T @ u
        nv = np.linalg.norm(v)
        if nv == 0.0:
            return np.zeros(N), np.zeros(K), 0.0
        v = v / nv
    sigma = float(u @ (A @ v))
    return u, v, sigma


def rabit_scales(A: np.ndarray, iters: int = 30):
    """Row/column scales (g, h) of the rank-1 fit g h^T ~ A, stored as fp16.

    Minimizing ||R - g.B.h||_F with B = sign(R) equals minimizing
    || |R| - g h^T ||_F, whose optimum is the leading singular pair of |R|;
    sigma is split evenly: g = sqrt(sigma) u, h = sqrt(sigma) v.
    """
    u, v, sigma = rank1_fit(A, iters)
    r = np.sqrt(max(sigma, 0.0))
    return to_f16(r * u), to_f16(r * v)


def quantize_rabit(W: np.ndarray, paths: int = 2, iters: int = 30, svid_sweeps: int = 0):
    """[RaBiT] §2.1 (two-path form W^ = g1.B1.h1 + g2.B2.h2) and §2.2 (the
    residual forward: B1 = sign(W), R1 = W - W^1, B2 = sign(R1)).

    Each path binarizes the current residual and fits its (g, h) to the
    residual's magnitude by a rank-1 fit; the next residual subtracts the path
    using the *stored* fp16 g and h, so that the recursion can be re-checked
    from the stored values alone.  That greedy pass is followed by
    `svid_sweeps` Gauss-Seidel sweeps (refine_rabit_svid; 0 = greedy only).
    """
    R = np.asarray(W, dtype=np.float32).astype(np.float64)
    N, K = R.shape
    B = np.empty((paths, N, K), dtype=np.int8)
    g = np.empty((paths, N), dtype=np.float16)
    h = np.empty((paths, K), dtype=np.float16)
    for p in range(paths):
        B[p] = sign_pm1(R)
        g[p], h[p] = rabit_scales(np.abs(R), iters)
        R = R - (g[p].astype(np.float64)[:, None] * B[p]) * h[p].astype(np.float64)[None, :]
    if svid_sweeps:
        refine_rabit_svid(W, B, g, h, svid_sweeps, iters)
    return B, g, h


def rabit_path(B_p, g_p, h_p):
    """g_p (.) B_p (.) h_p from the stored values, fp64 [N, K]."""
    return (g_p.astype(np.float64)[:, None] * B_p) * h_p.astype(np.float64)[None, :]


def refine_rabit_svid(W, B, g, h, sweeps: int = 20, iters: int = 30):
    """[RaBiT] §2.2, function-aware initialization step 1: iterative residual
    SVID, alternating over the paths Gauss-Seidel style (20 sweeps is the
    page's default).  Path by path, the target is what the other paths leave,

        T_p = W - sum_{q != p} g_q (.) B_q (.) h_q    (stored fp16 scales),
        B_p = sign(T_p),   (g_p, h_p) = rank-1 fit of |T_p|,

    which is the exact minimizer of ||T_p - g (.) B (.) h|| over that path:
    for positive g h the best B is sign(T), and then ||T - g(.)B(.)h|| equals
    || |T| - g h^T ||, minimized by the leading singular pair.  So the
    reconstruction error does not grow except through the fp16 rounding of
    g and h.  Updates B, g, h in place (B [P, N, K] int8, g [P, N], h [P, K]
    fp16) and returns them."""
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    P = B.shape[0]
    for _ in range(sweeps):
        for p in range(P):
            T = W64.copy()
            for q in range(P):          # the other paths, subtracted in path order
                if q != p:
                    T = T - rabit_path(B[q], g[q], h[q])
            B[p] = sign_pm1(T)
            g[p], h[p] = rabit_scales(np.abs(T), iters)
    return B, g, h


# ------------------------------------------------------------------- ternary
def quantize_ternary(W: np.ndarray):
    """[HGF] §1.2 ternary_quantize: gamma = mean|W| (the code computes the
    absolute mean although the prose says absmax; the code is followed),
    T = clamp(round(W / gamma), -1, 1), W ~ gamma * T.

    gamma: fp64 mean stored as fp32; W/gamma in fp32; round half to even.
    """
    W = np.asarray(W, dtype=np.float32)
    gamma = np.float32(np.mean(np.abs(W.astype(np.float64))))
    if gamma == 0:
        return np.zeros(W.shape, dtype=np.int8), np.float32(0.0)
    T = np.clip(np.rint(W / gamma), -1, 1).astype(np.int8)
    return T, gamma


# ---------------------------------------------------------------------- W2A8
def quantize_w2a8(W: np.ndarray, group: int = 128):
    """[ABQ] §3.2 Eq. (3) with the compensation switched off (gamma = 0) and
    the clipping factors of Eq. (1) at 1: plain asymmetric min/max
    round-to-nearest on 2 bits, per group of `group` consecutive inputs:

        lo, hi = min, max of the group
        delta  = fl16((hi - lo) / 3)
        z      = clamp(rint(-lo / delta), 0, 3)          (integer zero point)
        q      = clamp(rint(W / delta) + z, 0, 3)
        W^     = delta * (q - z)

    A group whose step is zero (all weights equal) gets delta = 1, z = 0,
    q = 0.  Arithmetic in fp64 from the fp32 weights and the fp16 step.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % group == 0
    G = K // group
    Wg = W.reshape(N, G, group).astype(np.float64)
    lo = Wg.min(axis=-1)
    hi = Wg.max(axis=-1)
    delta16 = to_f16((hi - lo) / 3.0)
    delta = delta16.astype(np.float64)
    degenerate = delta == 0.0
    safe = np.where(degenerate, 1.0, delta)
    z = np.clip(np.rint(-lo / safe), 0, 3)
    q = np.clip(np.rint(Wg / safe[..., None]) + z[..., None], 0, 3)
    z = np.where(degenerate, 0.0, z)
    q = np.where(degenerate[..., None], 0.0, q)
    delta16 = np.where(degenerate, np.float16(1.0), delta16).astype(np.float16)
    return (q.reshape(N, K).astype(np.uint8), delta16, z.astype(np.float16))


def quantize_wnam(W: np.ndarray, bits: int, group: int = 128):
    """Arbitrary weight bit width n = `bits` (1..4) for the WnAm bit-plane
    GEMV ([ABQ] §1 quantization freedom; §3.2 Eq. (3) with gamma = 0 and the
    clipping factors of Eq. (1) at 1): the same asymmetric min/max
    round-to-nearest as W2A8, on L = 2^n - 1 steps per group:

        delta = fl16((hi - lo) / L)
        z     = clamp(rint(-lo / delta), 0, L)           (integer zero point)
        q     = clamp(rint(W / delta) + z, 0, L)          (n bit-planes)
        W^    = delta * (q - z)

    A group whose step is zero gets delta = 1, z = 0, q = 0.  With n = 2 this
    is quantize_w2a8.
    """
    assert 1 <= bits <= 4
    L = float((1 << bits) - 1)
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % group == 0
    G = K // group
    Wg = W.reshape(N, G, group).astype(np.float64)
    lo = Wg.min(axis=-1)
    hi = Wg.max(axis=-1)
    step16 = to_f16((hi - lo) / L)
    step = step16.astype(np.float64)
    flat = step == 0.0
    div = np.where(flat, 1.0, step)
    zp = np.clip(np.rint(-lo / div), 0, L)
    codes = np.clip(np.rint(Wg / div[..., None]) + zp[..., None], 0, L)
    zp = np.where(flat, 0.0, zp)
    codes = np.where(flat[..., None], 0.0, codes)
    step16 = np.where(flat, np.float16(1.0), step16).astype(np.float16)
    return codes.reshape(N, K).astype(np.uint8), step16, zp.astype(np.float16)


# ---------------------------------------------------------------------- BVSR
BVSR_GROUP = 32
BVSR_NBITS = 4
BVSR_NR = 16          # ratios r_i = 1.6 + 0.8 i / 15
BVSR_NL = 16          # spans L_j = ((j + 1/2)/16)-quantile of group ranges



def quantize_bit_balance(W: np.ndarray, group: int = 128):
    """[ABQ] §3.3 bit balance: the 2-bit integer grid, whose four values
    ({-2,-1,0,1} or {-1,0,1,2}) break the symmetry of the weight
    distribution, is widened to the symmetric five values {-2,-1,0,1,2}.
    Per group of `group` inputs, with a symmetric round-to-nearest step:

        delta = fl16(max |W| / 2)
        t     = clamp(rint(W / delta), -2, 2)
        code  = t + 2                 (0..4, stored on three bit planes)
        z     = 2                     (so W^ = delta * (code - z) = delta * t)

    A group whose step is zero gets delta = 1 and code 2 (W^ = 0).
    Arithmetic in fp64 from the fp32 weights and the fp16 step.  Returns
    (code uint8 [N, K], delta fp16 [N, G], zero fp16 [N, G]) in the WnAm
    logical form with n = 3.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % group == 0
    G = K // group
    Wg = W.reshape(N, G, group).astype(np.float64)
    amax = np.abs(Wg).max(axis=-1)
    step16 = to_f16(amax / 2.0)
    step = step16.astype(np.float64)
    flat = step == 0.0
    div = np.where(flat, 1.0, step)
    t = np.clip(np.rint(Wg / div[..., None]), -2, 2)
    t = np.where(flat[..., None], 0.0, t)
    step16 = np.where(flat, np.float16(1.0), step16).astype(np.float16)
    zero = np.full((N, G), 2.0, dtype=np.float16)
    return (t + 2).reshape(N, K).astype(np.uint8), step16, zero

def quantile_linear(sorted_vals: np.ndarray, qf: float) -> float:
    """Linear-interpolation quantile of sorted data, written out so that the
    arithmetic order is fixed: pos = q (n-1); i = floor(pos);
    L = s[i] + (pos - i) * (s[i+1] - s[i])."""
    s = sorted_vals
    n = s.shape[0]
    pos = qf * (n - 1)
    i = int(np.floor(pos))
    if i >= n - 1:
        return float(s[n - 1])
    frac = pos - i
    return float(s[i] + frac * (s[i + 1] - s[i]))


def bvsr_cache(W: np.ndarray):
    """[BVSR] (introduction): coefficient sets are subset sums of a geometric
    series, scaled and shifted by data-dependent terms; the candidate space
    pairs geometric sets with an auxiliary grid aligned to the data range, and
    the sets are shared across weight vectors through a "coefficient cache".

    Reading taken (the page gives no construction): 256 sets, id = 16 i + j,
        r_i = 1.6 + 0.8 i / 15          (i = 0..15)
        L_j = ((j + 1/2)/16)-quantile of the per-group range (max - min)
              over the whole tensor     (j = 0..15)
        a = L_j / (1 + r + r^2 + r^3),  c_k = a r^k (k = 0..3),  b = -L_j / 2
    so the 16 representable points b + sum_k c_k beta_k span [-L/2, L/2].
    Computed in fp64, stored as fp32: cache[id] = (c0, c1, c2, c3, b).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % BVSR_GROUP == 0
    Wg = W.reshape(-1, BVSR_GROUP).astype(np.float64)
    spans = np.sort(Wg.max(axis=1) - Wg.min(axis=1))
    cache = np.zeros((BVSR_NR * BVSR_NL, 5), dtype=np.float32)
    for i in range(BVSR_NR):
        r = 1.6 + (0.8 * i) / 15.0
        r2 = r * r
        r3 = r2 * r
        denom = 1.0 + r + r2 + r3
        for j in range(BVSR_NL):
            L = quantile_linear(spans, (j + 0.5) / BVSR_NL)
            a = L / denom
            cache[16 * i + j] = (a, a * r, a * r2, a * r3, -L / 2.0)
    return cache


def bvsr_points(cache: np.ndarray) -> np.ndarray:
    """The 16 representable values of each set, fp64 [S, 16]:
    v(code) = (((b + c0 beta0) + c1 beta1) + c2 beta2) + c3 beta3, beta_k =
    bit k of code."""
    c = np.asarray(cache, dtype=np.float32).astype(np.float64)
    codes = np.arange(16)
    v = np.repeat(c[:, 4:5], 16, axis=1)
    for k in range(4):
        bit = ((codes >> k) & 1).astype(bool)
        v = np.where(bit[None, :], v + c[:, k:k + 1], v)
    return v


def bvsr_encode(W: np.ndarray, cache: np.ndarray, idx: np.ndarray):
    """Nearest representable point of the chosen set for every weight.

    [BVSR] (introduction): given a weight vector and a coefficient set, the
    bitvectors are chosen to minimize the MSE, i.e. each element takes the
    nearest of the 16 points (ties -> smaller code).  Returns (code [N,K],
    sse [N, K/32]) with the group SSE summed in element order in fp64.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // BVSR_GROUP
    pts = bvsr_points(cache)                                   # [S,16]
    w = W.reshape(N * G, BVSR_GROUP).astype(np.float64)
    p = pts[np.asarray(idx).reshape(-1).astype(np.int64)]      # [NG,16]
    d = w[:, :, None] - p[:, None, :]
    d2 = d * d
    code = np.argmin(d2, axis=-1)
    dmin = np.take_along_axis(d2, code[..., None], axis=-1)[..., 0]
    sse = np.zeros(N * G)
    for e in range(BVSR_GROUP):
        sse = sse + dmin[:, e]
    return code.reshape(N, K).astype(np.uint8), sse.reshape(N, G)


def bvsr_search(W: np.ndarray, cache: np.ndarray, chunk: int = 2048):
    """Exhaustive search over the cache (the [BVSR] introduction's per-vector
    exhaustive search): for every group of 32 weights and every set, encode
    with nearest points and take the set of least group SSE (ties -> lower id).
    Returns (code uint8 [N,K], idx uint8 [N,K/32], sse float64 [N,K/32])."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // BVSR_GROUP
    pts = bvsr_points(cache)
    S = pts.shape[0]
    w_all = W.reshape(N * G, BVSR_GROUP).astype(np.float64)
    best_sse = np.full(N * G, np.inf)
    best_id = np.zeros(N * G, dtype=np.int64)
    best_code = np.zeros((N * G, BVSR_GROUP), dtype=np.int64)
    for c0 in range(0, N * G, chunk):
        w = w_all[c0:c0 + chunk]
        bs = best_sse[c0:c0 + chunk]
        bi = best_id[c0:c0 + chunk]
        bc = best_code[c0:c0 + chunk]
        for s in range(S):
            d = w[:, :, None] - pts[s][None, None, :]
            d2 = d * d
            code = np.argmin(d2, axis=-1)
            dmin = np.take_along_axis(d2, code[..., None], axis=-1)[..., 0]
            sse = np.zeros(w.shape[0])
            for e in range(BVSR_GROUP):
                sse = sse + dmin[:, e]
            better = sse < bs
            bs[better] = sse[better]
            bi[better] = s
            bc[better] = code[better]
    return (best_code.reshape(N, K).astype(np.uint8),
            best_id.reshape(N, G).astype(np.uint8),
            best_sse.reshape(N, G))
