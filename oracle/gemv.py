"""Reference GEMV y = W^ x^ for every format (test infrastructure only).

The oracle dequantizes explicitly (W^ materialized in fp64, in row chunks)
and takes an fp64 dot product with the activation the kernel multiplies; the
integer paths also get their exact int64 partial sums.  All inputs are the
logical forms of oracle/weights.py.

Shapes: W^ is [N, K]; activations are [M, K]; outputs are [M, N].
"""
from __future__ import annotations

import numpy as np

from . import act as act_mod
from .weights import BVSR_GROUP, bvsr_points

TOL_REL = 2e-3          # |y - y_ref| <= TOL_REL * sum_k |w^_nk x^_mk|
ROW_CHUNK = 1024


def _chunked_matmul(deq, N: int, xhat: np.ndarray):
    """y[m, n] = sum_k W^[n,k] xhat[m,k] and bound[m, n] = sum_k |W^| |xhat|,
    dequantizing rows [n0, n1) at a time with deq(n0, n1) -> fp64 [rows, K]."""
    xhat = np.asarray(xhat, dtype=np.float64)
    M = xhat.shape[0]
    y = np.zeros((M, N))
    bound = np.zeros((M, N))
    ax = np.abs(xhat)
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        Wd = deq(n0, n1)
        y[:, n0:n1] = xhat @ Wd.T
        bound[:, n0:n1] = ax @ np.abs(Wd).T
    return y, TOL_REL * bound


# ------------------------------------------------------------------- dequant
def deq_sign(B, alpha, n0=0, n1=None):
    """[BitNet] §2.2: W^ = alpha * sign(W) (alpha per row here)."""
    n1 = B.shape[0] if n1 is None else n1
    return alpha[n0:n1].astype(np.float64)[:, None] * B[n0:n1].astype(np.float64)


def deq_rabit(B, g, h, n0=0, n1=None):
    """[RaBiT] §2.1: W^ = sum_p g_p (.) B_p (.) h_p (row scale g, column h)."""
    n1 = B.shape[1] if n1 is None else n1
    out = np.zeros((n1 - n0, B.shape[2]))
    for p in range(B.shape[0]):
        out += (g[p, n0:n1].astype(np.float64)[:, None] * B[p, n0:n1].astype(np.float64)) \
            * h[p].astype(np.float64)[None, :]
    return out


def deq_ternary(T, gamma, n0=0, n1=None):
    """[HGF] §1.2: W^ = gamma * T."""
    n1 = T.shape[0] if n1 is None else n1
    return np.float64(gamma) * T[n0:n1].astype(np.float64)


def deq_w2a8(q, delta, zero, n0=0, n1=None, group: int = 128):
    """[ABQ] §3.2 Eq. (3): W^ = delta * (q - z) per group."""
    n1 = q.shape[0] if n1 is None else n1
    R = n1 - n0
    K = q.shape[1]
    qq = q[n0:n1].astype(np.float64).reshape(R, K // group, group)
    dd = delta[n0:n1].astype(np.float64)[..., None]
    zz = zero[n0:n1].astype(np.float64)[..., None]
    return (dd * (qq - zz)).reshape(R, K)


def deq_bvsr(code, idx, cache, n0=0, n1=None):
    """[BVSR]: each weight is the point b + sum_k c_k beta_k of its group's set."""
    n1 = code.shape[0] if n1 is None else n1
    pts = bvsr_points(cache)
    R = n1 - n0
    K = code.shape[1]
    ids = np.repeat(idx[n0:n1].astype(np.int64), BVSR_GROUP, axis=1)      # [R, K]
    return pts[ids.reshape(-1), code[n0:n1].reshape(-1).astype(np.int64)].reshape(R, K)


# ------------------------------------------------------------ float outputs
def gemv_sign(B, alpha, x):
    """y = alpha (.) (B x); returns (y, tol).  x: [M, K] float32."""
    return _chunked_matmul(lambda a, b: deq_sign(B, alpha, a, b), B.shape[0], x)


def gemv_rabit(B, g, h, x):
    """y = (sum_p g_p.B_p.h_p) x; returns (y, tol).  x: [M, K] (bf16 values)."""
    return _chunked_matmul(lambda a, b: deq_rabit(B, g, h, a, b), B.shape[1], x)


def gemv_xnor(B, alpha, xb, beta):
    """Fully binary product ([BitNet] §2.3): y = alpha (.) beta (B x_b) with
    x_b in {-1,+1}; returns (y, tol).  The dequantized operands are alpha B and
    beta x_b."""
    xhat = np.asarray(xb, dtype=np.float64) * np.asarray(beta, dtype=np.float64)[:, None]
    return _chunked_matmul(lambda a, b: deq_sign(B, alpha, a, b), B.shape[0], xhat)


def xnor_int(B, xb):
    """Y[m, n] = sum_k B[n,k] x_b[m,k] (int64, exact)."""
    return np.asarray(xb, dtype=np.int64) @ np.asarray(B, dtype=np.int64).T


def act_hat(q, d):
    """x^ = q * d, the activation the integer paths multiply."""
    return q.astype(np.float64) * np.asarray(d, dtype=np.float64)[:, None]


def gemv_ternary(T, gamma, q, d):
    return _chunked_matmul(lambda a, b: deq_ternary(T, gamma, a, b), T.shape[0], act_hat(q, d))


def gemv_w2a8(qw, delta, zero, q, d, group: int = 128):
    return _chunked_matmul(lambda a, b: deq_w2a8(qw, delta, zero, a, b, group),
                           qw.shape[0], act_hat(q, d))


def gemv_bvsr(code, idx, cache, q, d):
    return _chunked_matmul(lambda a, b: deq_bvsr(code, idx, cache, a, b),
                           code.shape[0], act_hat(q, d))


# ------------------------------------------- HGF gated low-rank correction
SILU_SLOPE_MAX = 1.1    # >= max_z |d silu / dz| (about 1.0998)


def silu(z):
    """SiLU, z * sigmoid(z) = z / (1 + exp(-z)), in fp64: the activation of
    [HGF] §2.1's correction path.  Large negative z gives exp(-z) = inf and
    the quotient -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def lora_down(x, A):
    """h = silu(x A) ([HGF] §2.1): x [M, K] is the layer input before
    activation quantization, A [K, r] the down matrix; fp64 [M, r]."""
    return silu(np.asarray(x, dtype=np.float64) @ np.asarray(A, dtype=np.float64))


def lora_gate(alpha):
    """The gate tanh(alpha), which [HGF] §2.1 uses to keep it in (-1, 1)."""
    return np.tanh(np.float64(alpha))


def lora_correction(x, A, B, alpha):
    """[HGF] §2.1: tanh(alpha) * (silu(x A) B) with B [r, N]; returns the
    fp64 [M, N] correction and its tolerance.

    The bound covers what an fp32 evaluation can lose: |gate| sum_j |B_jn|
    (|h_j| + SILU_SLOPE_MAX sum_k |x_k A_kj|), times the float tolerance."""
    x = np.asarray(x, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    h = lora_down(x, A)
    g = lora_gate(alpha)
    out = g * (h @ B)
    zabs = np.abs(x) @ np.abs(A)
    bound = abs(g) * ((np.abs(h) + SILU_SLOPE_MAX * zabs) @ np.abs(B))
    return out, TOL_REL * bound


def gemv_hgf(T, gamma, q, d, x, A, B, alpha):
    """[HGF] §2.1 and §4.1: the ternary product of the quantized activations
    plus the gated low-rank correction of the unquantized input x; returns
    (y, tol) with the two paths' tolerances added."""
    yt, tt = gemv_ternary(T, gamma, q, d)
    yl, tl = lora_correction(x, A, B, alpha)
    return yt + yl, tt + tl


# ------------------------------------------------- exact integer partial sums
def ternary_int(T, q):
    """[HGF] §1.2 Y_int = int8_matmul(X_quant, W_quant^T): [M, N] int64."""
    return q.astype(np.int64) @ T.astype(np.int64).T


def w2a8_int(qw, q, group: int = 128):
    """A[m, n, g] = sum_{k in g} qw[n,k] q[m,k]  (int64 [M, N, K/group])."""
    N, K = qw.shape
    M = q.shape[0]
    G = K // group
    a = qw.astype(np.int64).reshape(N, G, group)
    b = q.astype(np.int64).reshape(M, G, group)
    return np.einsum("ngk,mgk->mng", a, b)


def bvsr_int(code, q):
    """P[m, n, g, b] = sum_{k in g} beta_b[n,k] q[m,k] (int64 [M,N,K/32,4])."""
    N, K = code.shape
    M = q.shape[0]
    G = K // BVSR_GROUP
    c = code.astype(np.int64).reshape(N, G, BVSR_GROUP)
    qq = q.astype(np.int64).reshape(M, G, BVSR_GROUP)
    out = np.empty((M, N, G, 4), dtype=np.int64)
    for b in range(4):
        out[..., b] = np.einsum("ngk,mgk->mng", (c >> b) & 1, qq)
    return out


# ------------------------- outputs rebuilt from the partial sums (epilogues)
def ternary_from_int(Y, gamma, d):
    """[HGF] §1.2 dequantization Y = Y_int * (gamma_x (x) gamma_W / 127); with
    d = amax/127 the per-token factor is gamma * d."""
    return Y.astype(np.float64) * np.float64(gamma) * np.asarray(d, np.float64)[:, None]


def w2a8_from_int(A, S, delta, zero, d):
    """y = d * sum_g delta[n,g] (A[m,n,g] - z[n,g] S[m,g])."""
    dl = delta.astype(np.float64)[None]
    zz = zero.astype(np.float64)[None]
    t = dl * (A.astype(np.float64) - zz * S.astype(np.float64)[:, None, :])
    return np.asarray(d, np.float64)[:, None] * t.sum(axis=-1)


def bvsr_from_int(P, S, idx, cache, d):
    """y = d * sum_g (b_id S[g] + sum_k c_{id,k} P[g,k])."""
    c = np.asarray(cache, dtype=np.float32).astype(np.float64)[idx.astype(np.int64)]  # [N,G,5]
    t = c[None, :, :, 4] * S.astype(np.float64)[:, None, :]
    t = t + (c[None, :, :, :4] * P.astype(np.float64)).sum(axis=-1)
    return np.asarray(d, np.float64)[:, None] * t.sum(axis=-1)


def group_sums(q, group):
    return act_mod.group_sums(q, group)
