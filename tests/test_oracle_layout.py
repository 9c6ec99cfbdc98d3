"""Pins of the oracle's blob reader (oracle/layout.py) on blobs assembled by
hand, byte by byte, from the layout specification."""
import struct

import numpy as np

from oracle import layout


def _header(fmt, N, K, P, group, off_c0, off_c1, total):
    Np = (N + 63) // 64 * 64
    Kp = (K + 127) // 128 * 128
    h = struct.pack("<10I4Q", 0x51544942, 1, fmt, N, K, P, group, Np, Kp, 0,
                    256, off_c0, off_c1, total)
    return bytearray(h + bytes(256 - len(h))), Np, Kp


def _set_bit(blob, Np, Kp, P, p, n, k):
    Tb = Kp // 128
    t, r = divmod(n, 64)
    b, kk = divmod(k, 128)
    w, i = divmod(kk, 32)
    off = 256 + ((t * Tb + b) * P + p) * 1024 + r * 16 + w * 4
    word = struct.unpack_from("<I", blob, off)[0] | (1 << i)
    struct.pack_into("<I", blob, off, word)


def _set_bvsr_bit(blob, Np, Kp, n, k, j):
    """beta_j of weight (n, k) in the BVSR4 plane layout: plane s = (k % 32) // 8
    of the 32-input word, nibble e with (e >> 1) + 4 (e & 1) = k % 8, bit j of it."""
    pos = k % 8
    e = 2 * pos if pos < 4 else 2 * (pos - 4) + 1
    _set_bit(blob, Np, Kp, 4, (k % 32) // 8, n, (k // 32) * 32 + 4 * e + j)


def test_hand_blob_sign():
    N, K = 70, 200                  # 2 row tiles, 2 k blocks, ragged both ways
    hdr, Np, Kp = _header(1, N, K, 1, 0, 0, 0, 0)
    planes = 2 * 2 * 1 * 1024
    off_c0 = 256 + planes
    total = off_c0 + ((4 * Np + 255) // 256) * 256
    hdr, Np, Kp = _header(1, N, K, 1, 0, off_c0, off_c0 + 4 * Np, total)
    blob = hdr + bytearray(total - 256)
    ones = [(0, 0), (0, 31), (1, 32), (63, 127), (64, 128), (69, 199), (65, 130)]
    for n, k in ones:
        _set_bit(blob, Np, Kp, 1, 0, n, k)
    alpha = np.arange(Np, dtype=np.float32) * (np.arange(Np) < N)
    blob[off_c0:off_c0 + 4 * Np] = alpha.tobytes()
    out = layout.unpack(np.frombuffer(bytes(blob), np.uint8))
    B = out["B"]
    assert B.shape == (N, K)
    expect = -np.ones((N, K), np.int8)
    for n, k in ones:
        expect[n, k] = 1
    assert np.array_equal(B, expect)
    assert np.array_equal(out["alpha"], alpha[:N]) and out["pad_ok"]
    # a bit set in a padded column is reported
    _set_bit(blob, Np, Kp, 1, 0, 3, 250)
    assert not layout.unpack(np.frombuffer(bytes(blob), np.uint8))["pad_ok"]


def test_hand_blob_w2a8_and_bvsr_coefficients():
    N, K = 64, 256
    # W2A8: q = bit0 + 2 bit1; dz word per (row tile, block, row)
    planes = 1 * 2 * 2 * 1024
    off_c0 = 256 + planes
    total = off_c0 + 4 * 64 * 2
    hdr, Np, Kp = _header(4, N, K, 2, 128, off_c0, total, total)
    blob = hdr + bytearray(total - 256)
    _set_bit(blob, Np, Kp, 2, 0, 5, 7)          # q[5,7] = 1
    _set_bit(blob, Np, Kp, 2, 1, 5, 8)          # q[5,8] = 2
    _set_bit(blob, Np, Kp, 2, 0, 9, 130)
    _set_bit(blob, Np, Kp, 2, 1, 9, 130)        # q[9,130] = 3
    dz_off = off_c0 + (0 * 2 + 1) * 256 + 9 * 4  # tile 0, block 1, row 9
    struct.pack_into("<HH", blob, dz_off, int(np.float16(0.25).view(np.uint16)),
                     int(np.float16(2.0).view(np.uint16)))
    out = layout.unpack(np.frombuffer(bytes(blob), np.uint8))
    q = out["q"]
    assert q[5, 7] == 1 and q[5, 8] == 2 and q[9, 130] == 3 and q.sum() == 6
    assert float(out["delta"][9, 1]) == 0.25 and float(out["zero"][9, 1]) == 2.0
    assert float(out["delta"][9, 0]) == 0.0

    # BVSR: code = sum_k 2^k beta_k; idx byte j of the (tile, block, row) dword
    N, K = 64, 128
    planes = 1 * 1 * 4 * 1024
    off_c0 = 256 + planes
    off_c1 = off_c0 + 256
    total = off_c1 + ((256 * 5 * 4 + 255) // 256) * 256
    hdr, Np, Kp = _header(5, N, K, 4, 32, off_c0, off_c1, total)
    blob = hdr + bytearray(total - 256)
    _set_bvsr_bit(blob, Np, Kp, 2, 40, 0)
    _set_bvsr_bit(blob, Np, Kp, 2, 40, 3)        # code[2,40] = 9
    _set_bvsr_bit(blob, Np, Kp, 63, 127, 2)      # code[63,127] = 4
    _set_bvsr_bit(blob, Np, Kp, 7, 5, 1)         # code[7,5] = 2
    blob[off_c0 + 2 * 4 + 1] = 200               # idx[2, group 1]
    blob[off_c0 + 63 * 4 + 3] = 7                # idx[63, group 3]
    cache = np.arange(1280, dtype=np.float32).reshape(256, 5)
    stored = cache * np.array([1, 0.5, 0.25, 0.125, 1], np.float32)   # c_j 2^-j, then b
    blob[off_c1:off_c1 + 5120] = stored.tobytes()
    out = layout.unpack(np.frombuffer(bytes(blob), np.uint8))
    assert out["code"][2, 40] == 9 and out["code"][63, 127] == 4 and out["code"][7, 5] == 2
    assert out["code"].sum() == 15
    assert out["idx"][2, 1] == 200 and out["idx"][63, 3] == 7 and out["idx"].sum() == 207
    assert np.array_equal(out["cache"], cache)


def test_hand_blob_rabit_and_ternary():
    N, K = 64, 128
    P = 2
    planes = 1 * 1 * P * 1024
    off_c0 = 256 + planes
    off_c1 = off_c0 + 256                 # g: 2*64*2 = 256 bytes
    total = off_c1 + 512                  # h: 2*128*2 = 512 bytes
    hdr, Np, Kp = _header(2, N, K, P, 0, off_c0, off_c1, total)
    blob = hdr + bytearray(total - 256)
    _set_bit(blob, Np, Kp, P, 1, 10, 100)
    g = np.zeros((2, 64), np.float16)
    g[1, 10] = 0.5
    h = np.zeros((2, 128), np.float16)
    h[0, 3] = 1.5
    blob[off_c0:off_c0 + 256] = g.tobytes()
    blob[off_c1:off_c1 + 512] = h.tobytes()
    out = layout.unpack(np.frombuffer(bytes(blob), np.uint8))
    assert out["B"][1, 10, 100] == 1 and (out["B"] == 1).sum() == 1
    assert float(out["g"][1, 10]) == 0.5 and float(out["h"][0, 3]) == 1.5

    # ternary: plane 0 = +1, plane 1 = -1
    off_c0 = 256 + planes
    total = off_c0 + 256
    hdr, Np, Kp = _header(3, N, K, 2, 0, off_c0, total, total)
    blob = hdr + bytearray(total - 256)
    _set_bit(blob, Np, Kp, 2, 0, 1, 1)
    _set_bit(blob, Np, Kp, 2, 1, 2, 2)
    struct.pack_into("<f", blob, off_c0, 0.125)
    out = layout.unpack(np.frombuffer(bytes(blob), np.uint8))
    assert out["T"][1, 1] == 1 and out["T"][2, 2] == -1 and np.abs(out["T"]).sum() == 2
    assert out["gamma"] == np.float32(0.125) and not out["both_set"]
