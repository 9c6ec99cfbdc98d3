"""Python binding of libbitq (argument marshalling only).

Every function here forwards to the C ABI of the same name in
bit_plane_gemv_amd/libbitq.so (declared in include/bitq.h); all computation
happens in that library.  Device buffers are passed as torch tensors (their
data_ptr()) or raw integer addresses; PyTorch is used only to own device
memory and to name the current HIP stream.

Importing this package fails loudly if libbitq.so has not been built
(python bit_plane_gemv_amd/build.py); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# BITQ_LIBRARY selects another build of the same library (the sanitizer
# build of build.py --sanitize); by default the in-tree libbitq.so
LIB_PATH = os.environ.get("BITQ_LIBRARY") or os.path.join(_HERE, "libbitq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libbitq.so not found at {LIB_PATH}; build it with "
                      "`python bit_plane_gemv_amd/build.py`")

# One HIP runtime per process: torch wheels bundle their own libamdhip64, and
# loading libbitq.so first would bind it to the system runtime while torch
# later loads a second one (device pointers and streams are then not shared).
# Importing torch first makes libbitq.so bind to the runtime torch uses.
try:
    import torch as _torch  # noqa: F401
except ImportError:
    _torch = None
_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes() -> list:
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process: " + ", ".join(_hip_runtimes()))

# ------------------------------------------------------------------ enums
OK, E_ARG, E_SHAPE, E_ALIGN, E_UNSUPPORTED, E_CAPACITY, E_DEVICE = 0, -1, -2, -3, -4, -5, -6
SIGN1, RABIT, TERNARY, W2A8, BVSR4, WNAM, HGF = 1, 2, 3, 4, 5, 6, 7
DT_F32, DT_BF16, DT_ACT, DT_BINARY = 0, 1, 2, 3
F_ACC_INT32 = 1
F_FUSE_QUANT = 2   # bitq_gemv: raw x, the activation quantizer runs in the GEMV kernel

FORMAT_NAMES = {SIGN1: "sign", RABIT: "rabit", TERNARY: "ternary", W2A8: "w2a8", BVSR4: "bvsr",
                WNAM: "wnam", HGF: "hgf"}
FORMATS = {v: k for k, v in FORMAT_NAMES.items()}
DEFAULT_PLANES = {SIGN1: 1, RABIT: 2, TERNARY: 2, W2A8: 2, BVSR4: 4, WNAM: 4, HGF: 2}
DEFAULT_GROUP = {SIGN1: 0, RABIT: 0, TERNARY: 0, W2A8: 128, BVSR4: 32, WNAM: 128, HGF: 0}
DEFAULT_ABITS = {SIGN1: 0, RABIT: 0, TERNARY: 8, W2A8: 8, BVSR4: 8, WNAM: 4, HGF: 8}
DEFAULT_RANK = {HGF: 32}


class BitqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"bitq status {status}: {message}")
        self.status = status


class WDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("planes", ctypes.c_int32), ("group", ctypes.c_int32), ("abits", ctypes.c_int32),
                ("rank", ctypes.c_int32)]


class QuantOpts(ctypes.Structure):
    _fields_ = [("rabit_svid_sweeps", ctypes.c_int32), ("wnam_bit_balance", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 6)]


class Logical(ctypes.Structure):
    _fields_ = [("sign", ctypes.c_void_p), ("tern", ctypes.c_void_p), ("code", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("g", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("gamma", ctypes.c_float), ("delta", ctypes.c_void_p), ("zero", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("cache", ctypes.c_void_p), ("lora_a", ctypes.c_void_p),
                ("lora_b", ctypes.c_void_p), ("lora_alpha", ctypes.c_float)]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_sigs = {
    "bitq_version": ([], _I32),
    "bitq_last_error": ([], ctypes.c_char_p),
    "bitq_packed_size": ([ctypes.POINTER(WDesc), ctypes.POINTER(_SZ)], _I32),
    "bitq_pack_weights": ([ctypes.POINTER(WDesc), ctypes.POINTER(Logical), _P, _SZ], _I32),
    "bitq_quantize_weights": ([ctypes.POINTER(WDesc), _P, _P, _SZ, _I32], _I32),
    "bitq_quantize_weights_opts": ([ctypes.POINTER(WDesc), _P, ctypes.POINTER(QuantOpts), _P, _SZ, _I32],
                                   _I32),
    "bitq_quantize_weights_hgf": ([ctypes.POINTER(WDesc), _P, _P, _P, ctypes.c_float, _P, _SZ, _I32], _I32),
    "bitq_act_size": ([_I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "bitq_quantize_act": ([_P, _I32, _I32, _I32, _P, _SZ, _P], _I32),
    "bitq_quantize_act_bits": ([_P, _I32, _I32, _I32, _I32, _P, _SZ, _P], _I32),
    "bitq_hgf_act_size": ([ctypes.POINTER(WDesc), _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)], _I32),
    "bitq_quantize_act_hgf": ([ctypes.POINTER(WDesc), _P, _P, _I32, _I32, _P, _SZ, _P, _SZ, _P], _I32),
    "bitq_quantize_act_hgf_noalloc": ([ctypes.POINTER(WDesc), _P, _P, _I32, _I32, _P, _SZ, _P], _I32),
    "bitq_binact_size": ([_I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "bitq_binarize_act": ([_P, _I32, _I32, _I32, _P, _SZ, _P], _I32),
    "bitq_workspace_size": ([ctypes.POINTER(WDesc), _I32, ctypes.POINTER(_SZ)], _I32),
    "bitq_gemv": ([ctypes.POINTER(WDesc), _P, _P, _I32, _P, _P, _SZ, _U32, _P], _I32),
    "bitq_gemm_smallM": ([ctypes.POINTER(WDesc), _P, _P, _I32, _P, _P, _SZ, _U32, _P], _I32),
    # measurement context kernels (include/bitq_ctx.h)
    "bitq_ctx_empty": ([_I32, _P], _I32),
    "bitq_ctx_stream": ([_P, _SZ, _I32, _P, _I32, _P], _I32),
    "bitq_ctx_spin": ([_I32, _P], _I32),
    "bitq_ctx_launch_shape": ([ctypes.POINTER(WDesc), _I32, _I32, _U32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)],
                              _I32),
}
for _name, (_args, _ret) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTED = tuple(_sigs)


def _check(status: int):
    if status != OK:
        raise BitqError(status, _lib.bitq_last_error().decode())


def _ptr(x) -> int | None:
    """Device/host address of a tensor, numpy array or raw int (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def wdesc(fmt, N: int, K: int, planes: int | None = None, group: int | None = None,
          abits: int | None = None, rank: int | None = None) -> WDesc:
    if isinstance(fmt, str):
        fmt = FORMATS[fmt]
    return WDesc(fmt, N, K, DEFAULT_PLANES[fmt] if planes is None else planes,
                 DEFAULT_GROUP[fmt] if group is None else group,
                 DEFAULT_ABITS[fmt] if abits is None else abits,
                 DEFAULT_RANK.get(fmt, 0) if rank is None else rank)


# -------------------------------------------------------------- host calls
def version() -> int:
    return _lib.bitq_version()


def last_error() -> str:
    return _lib.bitq_last_error().decode()


def packed_size(desc: WDesc) -> int:
    n = _SZ(0)
    _check(_lib.bitq_packed_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _logical_shapes(desc: WDesc) -> dict:
    """Shape of each array field of bitq_logical that the descriptor's format
    reads (include/bitq.h, "Logical (unpacked) quantized form")."""
    N, K, P = desc.N, desc.K, desc.planes
    if desc.fmt == SIGN1:
        return {"sign": (N, K), "alpha": (N,)}
    if desc.fmt == RABIT:
        return {"sign": (P, N, K), "g": (P, N), "h": (P, K)}
    if desc.fmt == TERNARY:
        return {"tern": (N, K)}
    if desc.fmt in (W2A8, WNAM):
        return {"code": (N, K), "delta": (N, K // 128), "zero": (N, K // 128)}
    if desc.fmt == BVSR4:
        return {"code": (N, K), "idx": (N, K // 32), "cache": (256, 5)}
    if desc.fmt == HGF:
        return {"tern": (N, K), "lora_a": (K, desc.rank), "lora_b": (desc.rank, N)}
    return {}


def pack_weights(desc: WDesc, **fields) -> np.ndarray:
    """Pack a logical form (numpy arrays named as in bitq_logical) into a blob.
    Every array the format reads must be given, with the shape the header
    documents (ValueError otherwise): the C packer takes no lengths."""
    need = _logical_shapes(desc)
    for name, shape in need.items():
        if name not in fields or fields[name] is None:
            raise ValueError(f"{FORMAT_NAMES.get(desc.fmt, desc.fmt)} needs the field {name!r}")
        got = np.shape(fields[name])
        if tuple(got) != tuple(shape):
            raise ValueError(f"field {name!r} has shape {tuple(got)}, the descriptor needs {tuple(shape)}")
    keep = []
    lg = Logical()
    conv = {"sign": np.int8, "tern": np.int8, "code": np.uint8, "alpha": np.float32,
            "g": np.uint16, "h": np.uint16, "delta": np.uint16, "zero": np.uint16,
            "idx": np.uint8, "cache": np.float32, "lora_a": np.uint16, "lora_b": np.uint16}
    for name, val in fields.items():
        if name in ("gamma", "lora_alpha"):
            setattr(lg, name, float(val))
            continue
        arr = np.asarray(val)
        if arr.dtype == np.float16:
            arr = arr.view(np.uint16)
        arr = np.ascontiguousarray(arr, dtype=conv[name])
        keep.append(arr)
        setattr(lg, name, arr.ctypes.data)
    blob = np.zeros(packed_size(desc), dtype=np.uint8)
    _check(_lib.bitq_pack_weights(ctypes.byref(desc), ctypes.byref(lg), blob.ctypes.data, blob.nbytes))
    return blob


def quantize_weights(desc: WDesc, W: np.ndarray, nthreads: int = 0, svid_sweeps: int = 0,
                     bit_balance: bool = False) -> np.ndarray:
    """fp32 W [N, K] -> packed blob with the library's own offline quantizer
    (RABIT: svid_sweeps Gauss-Seidel refinement sweeps after the greedy pass;
    WNAM with 3 planes: bit_balance selects the symmetric five-level grid)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.shape != (desc.N, desc.K):
        raise ValueError(f"W has shape {W.shape}, descriptor says {(desc.N, desc.K)}")
    blob = np.zeros(packed_size(desc), dtype=np.uint8)
    if svid_sweeps or bit_balance:
        opts = QuantOpts(svid_sweeps, int(bit_balance))
        _check(_lib.bitq_quantize_weights_opts(ctypes.byref(desc), W.ctypes.data, ctypes.byref(opts),
                                               blob.ctypes.data, blob.nbytes, nthreads))
    else:
        _check(_lib.bitq_quantize_weights(ctypes.byref(desc), W.ctypes.data, blob.ctypes.data,
                                          blob.nbytes, nthreads))
    return blob


def quantize_weights_hgf(desc: WDesc, W: np.ndarray, lora_a, lora_b, lora_alpha: float,
                         nthreads: int = 0) -> np.ndarray:
    """fp32 W [N, K] -> HGF blob: the library's ternary quantizer for W plus
    the correction parameters A [K, r], B [r, N] (fp16 arrays or their bits)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.shape != (desc.N, desc.K):
        raise ValueError(f"W has shape {W.shape}, descriptor says {(desc.N, desc.K)}")
    a = np.ascontiguousarray(np.asarray(lora_a).view(np.uint16) if np.asarray(lora_a).dtype == np.float16
                             else lora_a, dtype=np.uint16)
    b = np.ascontiguousarray(np.asarray(lora_b).view(np.uint16) if np.asarray(lora_b).dtype == np.float16
                             else lora_b, dtype=np.uint16)
    if desc.fmt == HGF and (a.shape != (desc.K, desc.rank) or b.shape != (desc.rank, desc.N)):
        raise ValueError("lora_a must be [K, rank] and lora_b [rank, N]")
    blob = np.zeros(packed_size(desc), dtype=np.uint8)
    _check(_lib.bitq_quantize_weights_hgf(ctypes.byref(desc), W.ctypes.data, a.ctypes.data, b.ctypes.data,
                                          float(lora_alpha), blob.ctypes.data, blob.nbytes, nthreads))
    return blob


def act_size(M: int, K: int) -> int:
    n = _SZ(0)
    _check(_lib.bitq_act_size(M, K, ctypes.byref(n)))
    return n.value


def hgf_act_size(desc: WDesc, M: int) -> tuple:
    """(activation buffer bytes, workspace bytes) of an HGF layer's activation step."""
    a, w = _SZ(0), _SZ(0)
    _check(_lib.bitq_hgf_act_size(ctypes.byref(desc), M, ctypes.byref(a), ctypes.byref(w)))
    return a.value, w.value


def binact_size(M: int, K: int) -> int:
    n = _SZ(0)
    _check(_lib.bitq_binact_size(M, K, ctypes.byref(n)))
    return n.value


def binact_layout(M: int, K: int) -> dict:
    """Section offsets of a binary activation buffer (as include/bitq.h)."""
    Kp = (K + 127) // 128 * 128
    Kw = Kp // 32
    a = lambda v: (v + 255) // 256 * 256
    off_beta = a(4 * M * Kw)
    return dict(Kp=Kp, Kw=Kw, off_bits=0, off_beta=off_beta, total=a(off_beta + 4 * M))


def workspace_size(desc: WDesc, M: int = 1) -> int:
    n = _SZ(0)
    _check(_lib.bitq_workspace_size(ctypes.byref(desc), M, ctypes.byref(n)))
    return n.value


# ------------------------------------------------------------ device calls
def binarize_act(x, x_dtype: int, M: int, K: int, act, act_bytes: int | None = None, stream=None):
    nbytes = act.numel() * act.element_size() if act_bytes is None else act_bytes
    _check(_lib.bitq_binarize_act(_ptr(x), x_dtype, M, K, _ptr(act), nbytes, _stream(stream)))


def quantize_act(x, x_dtype: int, M: int, K: int, act, act_bytes: int | None = None, stream=None,
                 abits: int = 8):
    nbytes = act.numel() * act.element_size() if act_bytes is None else act_bytes
    if abits == 8:
        _check(_lib.bitq_quantize_act(_ptr(x), x_dtype, M, K, _ptr(act), nbytes, _stream(stream)))
    else:
        _check(_lib.bitq_quantize_act_bits(_ptr(x), x_dtype, M, K, abits, _ptr(act), nbytes,
                                           _stream(stream)))


def quantize_act_hgf(desc: WDesc, w, x, x_dtype: int, M: int, act, ws, act_bytes: int | None = None,
                     ws_bytes: int | None = None, stream=None):
    abytes = act.numel() * act.element_size() if act_bytes is None else act_bytes
    wbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.bitq_quantize_act_hgf(ctypes.byref(desc), _ptr(w), _ptr(x), x_dtype, M, _ptr(act), abytes,
                                      _ptr(ws), wbytes, _stream(stream)))


def quantize_act_hgf_noalloc(desc: WDesc, w, x, x_dtype: int, M: int, act, act_bytes: int | None = None,
                             stream=None):
    """bitq_quantize_act_hgf without a workspace (the library's static device
    scratch holds the down projection's words; nothing is allocated)."""
    abytes = act.numel() * act.element_size() if act_bytes is None else act_bytes
    _check(_lib.bitq_quantize_act_hgf_noalloc(ctypes.byref(desc), _ptr(w), _ptr(x), x_dtype, M, _ptr(act), abytes,
                                              _stream(stream)))


def _nbytes(buf) -> int:
    """Size of a device buffer (0 for None: calls that need no workspace)."""
    return 0 if buf is None else buf.numel() * buf.element_size()


def gemv(desc: WDesc, w, x, x_dtype: int, y, ws, ws_bytes: int | None = None, flags: int = 0,
         stream=None):
    nbytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.bitq_gemv(ctypes.byref(desc), _ptr(w), _ptr(x), x_dtype, _ptr(y), _ptr(ws),
                          nbytes, flags, _stream(stream)))


def gemm_smallM(desc: WDesc, w, act, M: int, y, ws, ws_bytes: int | None = None, flags: int = 0,
                stream=None):
    nbytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.bitq_gemm_smallM(ctypes.byref(desc), _ptr(w), _ptr(act), M, _ptr(y), _ptr(ws),
                                 nbytes, flags, _stream(stream)))


# ------------------------------------------- measurement context kernels
def ctx_empty(grid: int, stream=None):
    """A launch of `grid` workgroups that does nothing (bitq_ctx_empty)."""
    _check(_lib.bitq_ctx_empty(grid, _stream(stream)))


def ctx_stream(src, nbytes: int, grid: int, out, nout: int, stream=None):
    """Read nbytes of src once with `grid` workgroups and write nout floats
    (bitq_ctx_stream): the streaming floor of a GEMV over those bytes."""
    _check(_lib.bitq_ctx_stream(_ptr(src), nbytes, grid, _ptr(out), nout, _stream(stream)))


def ctx_launch_shape(desc: WDesc, M: int, x_dtype: int, flags: int = 0) -> tuple:
    """(workgroups, lanes per workgroup) of the kernel bitq_gemv (M = 1) or
    bitq_gemm_smallM launches for these arguments."""
    g, b = _I32(0), _I32(0)
    _check(_lib.bitq_ctx_launch_shape(ctypes.byref(desc), M, x_dtype, flags, ctypes.byref(g), ctypes.byref(b)))
    return g.value, b.value


def ctx_spin(microseconds: int, stream=None):
    """One wave that waits the given wall-clock time (bitq_ctx_spin)."""
    _check(_lib.bitq_ctx_spin(microseconds, _stream(stream)))


def act_layout(M: int, K: int, rank: int = 0) -> dict:
    """Section offsets of an activation buffer (mirrors bitq_act_size; rank > 0:
    the HGF buffer of bitq_hgf_act_size with its h section)."""
    Kp = (K + 127) // 128 * 128
    Kw = Kp // 32

    def a256(v):
        return (v + 255) // 256 * 256
    off_S = a256(M * Kw * 32)
    off_q = a256(off_S + M * Kw * 4)
    off_qm = a256(off_q + M * Kp)
    off_d = a256(off_qm + 16 * ((M + 15) // 16) * Kp)   # qm: whole tiles of 16 tokens
    off_amax = a256(off_d + 4 * M)
    off_h = a256(off_amax + 4 * M)
    return dict(Kp=Kp, Kw=Kw, off_planes=0, off_S=off_S, off_q=off_q, off_qm=off_qm, off_d=off_d,
                off_amax=off_amax, off_h=off_h, total=a256(off_h + 4 * M * rank))
