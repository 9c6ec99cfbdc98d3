"""Independent reader of the packed weight blob (test infrastructure only).

Written from the blob specification (the "Packed blob layout" section of the
library's public header), not from the packer's code.  It turns a blob back
into the logical quantized form so that the packer can be checked by a round
trip and the GEMV parity can start from what the device actually reads.

Specification (all little-endian):
  header, 256 bytes: u32 magic 0x51544942, u32 version 1, u32 format,
      u32 N, u32 K, u32 P (planes), u32 group, u32 Np, u32 Kp, u32 reserved,
      u64 off_planes, u64 off_c0, u64 off_c1, u64 total_bytes; then at byte
      72 f32 hbound[3] (SIGN1: 1; RABIT: max over k of |h_p[k]|); HGF only,
      at byte 88: u64 off_c2, u32 rank, f32 alpha, f32 gate (tanh(alpha)
      rounded to fp32), f32 amax_a (max |A|).
  Np = N rounded up to 64 (row tile), Kp = K rounded up to 128 (k block).
  planes section: 1024-byte tiles ordered [row tile t][k block b][plane p];
      inside a tile, row r (= n - 64 t) owns 16 bytes = 4 uint32 words,
      word w covering k = 128 b + 32 w .. +31 with bit i <-> k = 128b+32w+i.
      Rows >= N and k >= K are zero bits.
  coefficient sections by format:
      1 sign    c0 = alpha  f32 [Np]
      2 rabit   c0 = g      f16 [P][Np],  c1 = h f16 [P][Kp]
      3 ternary c0 = gamma  f32 [1]          (plane 0: T=+1, plane 1: T=-1)
      4 w2a8    c0 = dz     u32 [Np/64][Kp/128][64], low half = delta (f16),
                high half = zero point (f16)  (plane i = bit i of q)
      5 bvsr    c0 = idx    u8  [Np/64][Kp/128][64][4] (byte j = group 4b+j),
                c1 = cache  f32 [256][5], entry (c_0, c_1/2, c_2/4, c_3/8, b);
                plane s of a 32-input word holds its inputs 8s .. 8s+7, one per
                nibble: bits 4e .. 4e+3 belong to input 8s + (e >> 1) + 4 (e & 1),
                bit 4e + j = beta_j of that input
      6 wnam    as w2a8 with P = n planes      (plane i = bit i of q)
      7 hgf     as ternary, plus c1 = A^T f16 [r][Kp] (row j = column j of
                A) and c2 = B^T f16 [Np][r] (row n = column n of B)
  Every section starts at a multiple of 256 bytes.
"""
from __future__ import annotations

import numpy as np

from . import bitserial

MAGIC = 0x51544942
HEADER_BYTES = 256
ROW_TILE = 64
K_BLOCK = 128
FORMATS = {1: "sign", 2: "rabit", 3: "ternary", 4: "w2a8", 5: "bvsr", 6: "wnam", 7: "hgf"}


def parse_header(blob: np.ndarray) -> dict:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    u32 = b[:40].view(np.uint32)
    u64 = b[40:72].view(np.uint64)
    h = dict(magic=int(u32[0]), version=int(u32[1]), fmt=int(u32[2]), N=int(u32[3]),
             K=int(u32[4]), P=int(u32[5]), group=int(u32[6]), Np=int(u32[7]),
             Kp=int(u32[8]), off_planes=int(u64[0]), off_c0=int(u64[1]),
             off_c1=int(u64[2]), total=int(u64[3]),
             hbound=b[72:84].view(np.float32).astype(np.float64))
    if h["magic"] != MAGIC:
        raise ValueError("bad magic")
    if h["fmt"] == 7:
        h["off_c2"] = int(b[88:96].view(np.uint64)[0])
        h["rank"] = int(b[96:100].view(np.uint32)[0])
        f = b[100:112].view(np.float32)
        h["alpha"], h["gate"], h["amax_a"] = np.float32(f[0]), np.float32(f[1]), np.float32(f[2])
    return h


def _section(b, off, nbytes, dtype):
    return b[off:off + nbytes].view(dtype)


def plane_bits(blob: np.ndarray, h: dict) -> np.ndarray:
    """All plane bits as uint8 [P, Np, Kp]."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    P, Np, Kp = h["P"], h["Np"], h["Kp"]
    Tn, Tb = Np // ROW_TILE, Kp // K_BLOCK
    words = _section(b, h["off_planes"], Tn * Tb * P * 1024, np.uint32)
    words = words.reshape(Tn, Tb, P, ROW_TILE, 4)
    words = words.transpose(2, 0, 3, 1, 4).reshape(P, Np, Kp // 32)
    return bitserial.unpack_bits(words)


def unpack(blob: np.ndarray) -> dict:
    """Blob -> logical form (plus 'pad_ok': padded rows/columns are zero)."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    h = parse_header(b)
    fmt, N, K, P, Np, Kp = h["fmt"], h["N"], h["K"], h["P"], h["Np"], h["Kp"]
    bits = plane_bits(b, h)
    pad_ok = bool(bits[:, N:, :].sum() == 0 and bits[:, :, K:].sum() == 0)
    bits = bits[:, :N, :K]
    Tn, Tb = Np // ROW_TILE, Kp // K_BLOCK
    out = dict(header=h, format=FORMATS[fmt])
    if fmt == 1:
        out["B"] = (2 * bits[0].astype(np.int8) - 1)
        alpha = _section(b, h["off_c0"], 4 * Np, np.float32)
        out["alpha"] = alpha[:N].copy()
        pad_ok &= bool(np.all(alpha[N:] == 0))
    elif fmt == 2:
        out["B"] = (2 * bits.astype(np.int8) - 1)
        g = _section(b, h["off_c0"], 2 * P * Np, np.float16).reshape(P, Np)
        hh = _section(b, h["off_c1"], 2 * P * Kp, np.float16).reshape(P, Kp)
        out["g"], out["h"] = g[:, :N].copy(), hh[:, :K].copy()
        pad_ok &= bool(np.all(g[:, N:] == 0) and np.all(hh[:, K:] == 0))
    elif fmt in (3, 7):
        plus, minus = bits[0].astype(np.int8), bits[1].astype(np.int8)
        out["both_set"] = bool(np.any(plus & minus))
        out["T"] = plus - minus
        out["gamma"] = np.float32(_section(b, h["off_c0"], 4, np.float32)[0])
        if fmt == 7:
            r = h["rank"]
            At = _section(b, h["off_c1"], 2 * r * Kp, np.float16).reshape(r, Kp)
            Bt = _section(b, h["off_c2"], 2 * Np * r, np.float16).reshape(Np, r)
            out["A"] = At[:, :K].T.copy()          # [K, r]
            out["B"] = Bt[:N].T.copy()             # [r, N]
            out["alpha"], out["gate"], out["amax_a"] = h["alpha"], h["gate"], h["amax_a"]
            pad_ok &= bool(np.all(At[:, K:] == 0) and np.all(Bt[N:] == 0))
    elif fmt in (4, 6):   # w2a8 (2 planes), wnam (P planes): code = sum_p 2^p plane_p
        out["q"] = sum((bits[p].astype(np.int64) << p) for p in range(P)).astype(np.uint8)
        dz = _section(b, h["off_c0"], 4 * Np * (Kp // K_BLOCK), np.uint32)
        dz = dz.reshape(Tn, Tb, ROW_TILE).transpose(0, 2, 1).reshape(Np, Tb)
        delta = (dz & 0xFFFF).astype(np.uint16).view(np.float16)
        zero = (dz >> 16).astype(np.uint16).view(np.float16)
        G = K // h["group"]
        out["delta"], out["zero"] = delta[:N, :G].copy(), zero[:N, :G].copy()
        pad_ok &= bool(np.all(dz[N:] == 0))
    elif fmt == 5:
        # natural bit position 32 g + 4 e + j of plane s -> bit j of the code
        # of input 32 g + 8 s + (e >> 1) + 4 (e & 1)
        G = K // 32
        nib = bits.reshape(P, N, G, 8, 4).astype(np.uint8)
        vals = sum(nib[..., j] << j for j in range(4))          # [s, n, g, e]
        pos = np.array([(e >> 1) + 4 * (e & 1) for e in range(8)])
        code = np.zeros((N, G, 32), dtype=np.uint8)
        for sp in range(P):
            code[:, :, 8 * sp + pos] = vals[sp]
        out["code"] = code.reshape(N, K)
        idx = _section(b, h["off_c0"], Np * (Kp // 32), np.uint8)
        idx = idx.reshape(Tn, Tb, ROW_TILE, 4).transpose(0, 2, 1, 3).reshape(Np, Kp // 32)
        out["idx"] = idx[:N, :K // 32].copy()
        stored = _section(b, h["off_c1"], 256 * 5 * 4, np.float32).reshape(256, 5)
        out["cache"] = np.ldexp(stored, np.array([0, 1, 2, 3, 0], dtype=np.int32)).astype(np.float32)
        pad_ok &= bool(np.all(idx[N:] == 0) and np.all(idx[:, K // 32:] == 0))
    else:
        raise ValueError(f"unknown format {fmt}")
    out["pad_ok"] = pad_ok
    return out
