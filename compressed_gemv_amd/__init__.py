"""Python binding of libqgemv (the MI355X compressed-weight product).

Thin marshalling over the C ABI in include/qgemv.h: every function here has
the name of the C entry point it calls, takes torch tensors that already
live on the GPU, allocates outputs with torch when none are given, passes
raw device pointers and torch's current HIP stream, and raises QError on a
non-zero status.  All arithmetic runs in the HIP kernels; there is no CPU
fallback, and any call fails loudly when the shared library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "QError", "load", "lib_path", "q_abi_version", "q_format_version", "q_status_str",
    "qgroup_sizes", "qpack_group", "qunpack_group", "qgemv_group",
    "qgroup_outlier_ws", "qpack_group_outlier", "qgemv_group_outlier", "qgemv_group_multi",
    "qcodebook_default", "qpack_group_cb", "qgemv_group_cb",
    "qtq_centroids", "qtq_rotation", "qtq_quant_keys", "qtq_project", "qtq_logits", "qtq_quant_values", "qtq_attend",
    "qbinlr_sizes", "qpack_binlr", "qunpack_binlr", "qgemv_binlr", "qgemv_binlr_noalloc",
    "qstream_read", "qgemm_prefill_ws", "qgemm_prefill", "Q_F32", "Q_BF16", "Q_FMT_GROUP", "Q_FMT_BINLR",
]

Q_OK, Q_EINVAL, Q_EALIGN, Q_EUNSUPPORTED, Q_ERANGE, Q_EWORKSPACE, Q_EHIP = 0, -1, -2, -3, -4, -5, -6
Q_F32, Q_BF16, Q_F16 = 0, 1, 2
Q_FMT_GROUP, Q_FMT_BINLR = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


def lib_path() -> str:
    return os.path.join(_HERE, "libqgemv.so")


class QError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({q_status_str(status)})")


class qweight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("bits", ctypes.c_int), ("group", ctypes.c_int),
        ("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
        ("r", ctypes.c_int64), ("ubits", ctypes.c_void_p), ("vtbits", ctypes.c_void_p),
        ("s1", ctypes.c_void_p), ("s2", ctypes.c_void_p),
        ("side", ctypes.c_void_p), ("oidx", ctypes.c_void_p), ("n_out", ctypes.c_int64),
        ("book_ids", ctypes.c_void_p), ("books", ctypes.c_void_p), ("n_books", ctypes.c_int),
    ]


class qgroup_mat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("y", ctypes.c_void_p)]


def load() -> ctypes.CDLL:
    """Load libqgemv.so from the package directory (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libqgemv.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    I64, I32, P, SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "q_abi_version": (I32, []),
        "q_format_version": (I32, []),
        "q_status_str": (ctypes.c_char_p, [I32]),
        "qgroup_sizes": (I32, [I64, I64, I32, I32, SZ, SZ]),
        "qpack_group": (I32, [P, I64, I64, I32, I32, P, P, P]),
        "qunpack_group": (I32, [P, P, I64, I64, I32, I32, P, P, P]),
        "qgemv_group": (I32, [P, P, I64, I64, I32, I32, P, I32, I64, P, I32, P]),
        "qgroup_outlier_ws": (I32, [I64, I64, SZ]),
        "qgemv_group_multi": (I32, [ctypes.POINTER(qgroup_mat), I32, I64, I32, I32, P, I32, I64, I32, P]),
        "qpack_group_outlier": (I32, [P, I64, I64, I32, I32, I64, P, P, P, P, P, ctypes.c_size_t, P]),
        "qgemv_group_outlier": (I32, [P, P, P, P, I64, I64, I64, I32, I32, P, I32, I64, P, I32, P]),
        "qcodebook_default": (I32, [I32, P, ctypes.POINTER(ctypes.c_int)]),
        "qpack_group_cb": (I32, [P, I64, I64, I32, I32, P, I32, P, P, P, P]),
        "qgemv_group_cb": (I32, [P, P, P, P, I32, I64, I64, I32, I32, P, I32, I64, P, I32, P]),
        "qtq_centroids": (I32, [I32, I32, ctypes.POINTER(ctypes.c_float), P]),
        "qtq_rotation": (I32, [I32, P, P]),
        "qtq_sizes": (I32, [I64, I32, SZ, SZ, SZ]),
        "qtq_quant_keys": (I32, [P, I64, I32, P, P, ctypes.c_float, P, P, P, P, P]),
        "qtq_logits_ws": (I32, [I64, I64, SZ]),
        "qtq_project": (I32, [P, P, P, P]),
        "qtq_logits": (I32, [P, P, P, I64, I64, I32, ctypes.c_float, P, P, P, P, I64, P, P, ctypes.c_size_t, P]),
        "qtq_quant_values": (I32, [P, I64, I32, P, ctypes.c_float, P, P, P, P]),
        "qtq_attend_ws": (I32, [I64, I64, I64, SZ]),
        "qtq_attend": (I32, [P, P, I64, I64, I32, ctypes.c_float, P, P, P, I64, P, P, ctypes.c_size_t, P]),
        "qbinlr_sizes": (I32, [I64, I64, I64, I64, SZ, SZ, SZ]),
        "qpack_binlr": (I32, [P, P, I64, I64, I64, P, P, P]),
        "qunpack_binlr": (I32, [P, P, I64, I64, I64, P, P, P]),
        "qgemv_binlr": (I32, [P, P, P, P, I64, I64, I64, P, I32, I64, P, I32, P, ctypes.c_size_t, P]),
        "qgemv_binlr_noalloc": (I32, [P, P, P, P, I64, I64, I64, P, I32, I64, P, I32, P]),
        "qstream_read": (I32, [P, ctypes.c_size_t, P, P]),
        "qgemm_prefill_ws": (I32, [ctypes.POINTER(qweight), I64, SZ]),
        "qgemm_prefill": (I32, [ctypes.POINTER(qweight), P, I32, I64, P, I32, P, ctypes.c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int, what: str):
    if status != Q_OK:
        raise QError(status, what)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return Q_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return Q_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_bytes(t: Optional[torch.Tensor], nbytes: int, what: str):
    """A buffer the kernels read or write nbytes of: it must hold them (the C
    ABI receives bare pointers and cannot check).  Every wrapper checks all
    sizes first and then, with _need_cuda, that every tensor is on the
    device."""
    if t is None:
        raise ValueError(f"{what}: missing")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what}: {_nbytes(t)} bytes, needs {nbytes}")


def _need_numel(t: Optional[torch.Tensor], numel: int, what: str, dtypes=None, exact=True):
    """An array argument with numel elements (at least numel when not exact:
    a longer table of which the kernels read the first numel entries) and one
    of dtypes."""
    if t is None:
        raise ValueError(f"{what}: missing")
    if t.numel() != numel if exact else t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, expected {'' if exact else 'at least '}{numel}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {dtypes}")


_ACT = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)   # activations (bf16 as 16-bit bits)
_OUT = (torch.float32, torch.bfloat16)
_H16 = (torch.int16, torch.uint16, torch.float16)                    # fp16 bit patterns


def _batch(x: torch.Tensor, K: int, what: str = "x") -> int:
    """Rows of an activation tensor [B][K] (or [K] for one row)."""
    if x.dtype not in _ACT:
        raise ValueError(f"{what}: dtype {x.dtype} is not fp32 or bf16")
    if x.dim() == 1:
        B = 1
    elif x.dim() == 2:
        B = x.shape[0]
    else:
        raise ValueError(f"{what}: expected [B][K] or [K], got shape {tuple(x.shape)}")
    if x.numel() != B * K:
        raise ValueError(f"{what}: shape {tuple(x.shape)} does not match K = {K}")
    return B


def q_abi_version() -> int:
    return load().q_abi_version()


def q_format_version() -> int:
    return load().q_format_version()


def q_status_str(status: int) -> str:
    return load().q_status_str(status).decode()


# ------------------------------------------------------------------ group RTN
def qgroup_sizes(N: int, K: int, bits: int, group: int):
    c, m = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qgroup_sizes(N, K, bits, group, ctypes.byref(c), ctypes.byref(m)), "qgroup_sizes")
    return c.value, m.value


def qpack_group(W: torch.Tensor, bits: int, group: int, codes=None, meta=None, stream=None):
    """Quantize + pack fp32 W[N][K] -> (codes uint8[N*K*b/8], meta int32[N*K/g])."""
    _need_cuda(W)
    if W.dim() != 2 or W.dtype != torch.float32:
        raise ValueError("W must be fp32 [N][K]")
    N, K = W.shape
    cb, mb = qgroup_sizes(N, K, bits, group)
    if codes is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=W.device)
    if meta is None:
        meta = torch.empty(mb // 4, dtype=torch.int32, device=W.device)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    _need_cuda(codes, meta)
    _check(load().qpack_group(_ptr(W), N, K, bits, group, _ptr(codes), _ptr(meta), _stream(stream)),
           "qpack_group")
    return codes, meta


def qunpack_group(codes, meta, N: int, K: int, bits: int, group: int, want_w: bool = False, stream=None):
    cb, mb = qgroup_sizes(N, K, bits, group)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    q = torch.empty((N, K), dtype=torch.uint8, device=codes.device)
    w = torch.empty((N, K), dtype=torch.float32, device=codes.device) if want_w else None
    _need_cuda(codes, meta)
    _check(load().qunpack_group(_ptr(codes), _ptr(meta), N, K, bits, group, _ptr(q), _ptr(w),
                                _stream(stream)), "qunpack_group")
    return (q, w) if want_w else q


def qgemv_group(codes, meta, N: int, K: int, bits: int, group: int, x: torch.Tensor,
                y: Optional[torch.Tensor] = None, y_dtype=torch.float32, stream=None):
    """y[B][N] = x[B][K] W_hat^T; x is bf16 (or int16/uint16 bf16 bits) or fp32."""
    cb, mb = qgroup_sizes(N, K, bits, group)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    B = _batch(x, K)
    if y is None:
        y = torch.empty((B, N), dtype=y_dtype, device=x.device)
    _need_numel(y, B * N, "y", _OUT)
    _need_cuda(codes, meta, x, y)
    _check(load().qgemv_group(_ptr(codes), _ptr(meta), N, K, bits, group, _ptr(x), _dtype_code(x), B,
                              _ptr(y), _dtype_code(y), _stream(stream)), "qgemv_group")
    return y


def qgemv_group_multi(mats, K: int, bits: int, group: int, x: torch.Tensor, ys=None,
                      y_dtype=torch.float32, stream=None):
    """[y_i] for mats = [(codes_i, meta_i, N_i)] sharing x, K, bits, group, in
    one launch."""
    B = _batch(x, K)
    if ys is None:
        ys = [torch.empty((B, n), dtype=y_dtype, device=x.device) for (_, _, n) in mats]
    if len(ys) != len(mats):
        raise ValueError("one output per matrix")
    for (c, m, n), y in zip(mats, ys):
        cb, mb = qgroup_sizes(n, K, bits, group)
        _need_bytes(c, cb, "codes")
        _need_bytes(m, mb, "meta")
        _need_numel(y, B * n, "y", _OUT)
        if y.dtype != ys[0].dtype:
            raise ValueError("all outputs of a grouped call share one dtype")
    arr = (qgroup_mat * len(mats))(*[qgroup_mat(c.data_ptr(), m.data_ptr(), n, y.data_ptr())
                                     for (c, m, n), y in zip(mats, ys)])
    _need_cuda(x, *[t for (c, m, _), y in zip(mats, ys) for t in (c, m, y)])
    _check(load().qgemv_group_multi(arr, len(mats), K, bits, group, _ptr(x), _dtype_code(x), B,
                                    _dtype_code(ys[0]), _stream(stream)), "qgemv_group_multi")
    return ys


# ------------------------------------------------ group RTN + outlier columns
def qgroup_outlier_ws(K: int, n_out: int) -> int:
    n = ctypes.c_size_t()
    _check(load().qgroup_outlier_ws(K, n_out, ctypes.byref(n)), "qgroup_outlier_ws")
    return n.value


def qpack_group_outlier(W: torch.Tensor, bits: int, group: int, n_out: int, stream=None):
    """(codes, meta, side uint16[N][n_out] fp16 bits, idx int32[n_out]) for fp32 W[N][K]."""
    _need_cuda(W)
    if W.dim() != 2 or W.dtype != torch.float32:
        raise ValueError("W must be fp32 [N][K]")
    N, K = W.shape
    cb, mb = qgroup_sizes(N, K, bits, group)
    codes = torch.empty(cb, dtype=torch.uint8, device=W.device)
    meta = torch.empty(mb // 4, dtype=torch.int32, device=W.device)
    side = torch.empty((N, n_out), dtype=torch.int16, device=W.device)
    idx = torch.empty(n_out, dtype=torch.int32, device=W.device)
    ws = torch.empty(qgroup_outlier_ws(K, n_out), dtype=torch.uint8, device=W.device)
    _check(load().qpack_group_outlier(_ptr(W), N, K, bits, group, n_out, _ptr(codes), _ptr(meta),
                                      _ptr(side), _ptr(idx), _ptr(ws), ws.numel(), _stream(stream)),
           "qpack_group_outlier")
    return codes, meta, side, idx


def qgemv_group_outlier(codes, meta, side, idx, N: int, K: int, bits: int, group: int, x: torch.Tensor,
                        y: Optional[torch.Tensor] = None, y_dtype=torch.float32, stream=None):
    """y[B][N] = x W_rest_hat^T + x[:, idx] side^T."""
    cb, mb = qgroup_sizes(N, K, bits, group)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    n_out = idx.numel()
    _need_numel(idx, n_out, "idx", (torch.int32,))
    _need_numel(side, N * n_out, "side", _H16, exact=False)
    B = _batch(x, K)
    if y is None:
        y = torch.empty((B, N), dtype=y_dtype, device=x.device)
    _need_numel(y, B * N, "y", _OUT)
    _need_cuda(codes, meta, side, idx, x, y)
    _check(load().qgemv_group_outlier(_ptr(codes), _ptr(meta), _ptr(side), _ptr(idx), idx.numel(), N, K, bits,
                                      group, _ptr(x), _dtype_code(x), B, _ptr(y), _dtype_code(y),
                                      _stream(stream)), "qgemv_group_outlier")
    return y


# ------------------------------------------------- group codes with codebooks
def qcodebook_default(bits: int) -> torch.Tensor:
    """The library's default dictionary for b-bit codes: uint8 [8][2^b] (host)."""
    L = 1 << bits
    out = torch.zeros((8, L), dtype=torch.uint8)
    n = ctypes.c_int()
    _check(load().qcodebook_default(bits, ctypes.c_void_p(out.data_ptr()), ctypes.byref(n)), "qcodebook_default")
    return out[: n.value]


def qpack_group_cb(W: torch.Tensor, bits: int, group: int, books: torch.Tensor, stream=None):
    """(codes, meta, book_ids uint8[N][K/g]) for fp32 W[N][K] with the
    dictionary books (uint8 [D][2^b], on the device)."""
    if W.dim() != 2 or W.dtype != torch.float32:
        raise ValueError("W must be fp32 [N][K]")
    _need_numel(books, books.shape[0] << bits, "books", (torch.uint8,), exact=False)
    _need_cuda(W, books)
    N, K = W.shape
    cb, mb = qgroup_sizes(N, K, bits, group)
    codes = torch.empty(cb, dtype=torch.uint8, device=W.device)
    meta = torch.empty(mb // 4, dtype=torch.int32, device=W.device)
    ids = torch.empty((N, K // group), dtype=torch.uint8, device=W.device)
    _check(load().qpack_group_cb(_ptr(W), N, K, bits, group, _ptr(books), books.shape[0], _ptr(codes),
                                 _ptr(meta), _ptr(ids), _stream(stream)), "qpack_group_cb")
    return codes, meta, ids


def qgemv_group_cb(codes, meta, book_ids, books, N: int, K: int, bits: int, group: int, x: torch.Tensor,
                   y: Optional[torch.Tensor] = None, y_dtype=torch.float32, stream=None):
    """y[B][N] = x W_hat^T with w_hat = s * books[id][q] / 2^(7-b) + o."""
    cb, mb = qgroup_sizes(N, K, bits, group)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    _need_numel(book_ids, N * (K // group), "book_ids", (torch.uint8,), exact=False)
    _need_numel(books, books.shape[0] << bits, "books", (torch.uint8,), exact=False)
    B = _batch(x, K)
    if y is None:
        y = torch.empty((B, N), dtype=y_dtype, device=x.device)
    _need_numel(y, B * N, "y", _OUT)
    _need_cuda(codes, meta, book_ids, books, x, y)
    _check(load().qgemv_group_cb(_ptr(codes), _ptr(meta), _ptr(book_ids), _ptr(books), books.shape[0], N, K,
                                 bits, group, _ptr(x), _dtype_code(x), B, _ptr(y), _dtype_code(y),
                                 _stream(stream)), "qgemv_group_cb")
    return y


# ------------------------------------------------- key-cache quantization
def qtq_centroids(d: int, mbits: int):
    """(delta, table uint8 numpy [2^mbits]) on the 7-bit centroid grid."""
    import numpy as np
    t = np.zeros(1 << mbits, dtype=np.uint8)
    dl = ctypes.c_float()
    _check(load().qtq_centroids(d, mbits, ctypes.byref(dl), t.ctypes.data_as(ctypes.c_void_p)), "qtq_centroids")
    return dl.value, t


def qtq_rotation(G):
    """Q of G = QR, diag(R) > 0, for a host fp64 array G [d][d]."""
    import numpy as np
    G = np.ascontiguousarray(G, dtype=np.float64)
    out = np.empty_like(G)
    _check(load().qtq_rotation(G.shape[0], G.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p)),
           "qtq_rotation")
    return out


def qtq_quant_keys(K: torch.Tensor, bits: int, Pi: torch.Tensor, S: torch.Tensor, delta: float, table,
                   stream=None):
    """(codes int32[n*4*(bits-1)], signs int32[n][4], norms int32[n]) for fp32 keys K[n][128]."""
    import numpy as np
    if K.dim() != 2 or K.shape[1] != 128 or K.dtype != torch.float32:
        raise ValueError("keys must be fp32 [n][128]")
    _need_numel(Pi, 128 * 128, "Pi", (torch.float64,))
    _need_numel(S, 128 * 128, "S", (torch.float64,))
    _need_cuda(K, Pi, S)
    n = K.shape[0]
    cb, sb, nb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qtq_sizes(n, bits, ctypes.byref(cb), ctypes.byref(sb), ctypes.byref(nb)), "qtq_sizes")
    codes = torch.empty(cb.value // 4, dtype=torch.int32, device=K.device)
    signs = torch.empty((n, 4), dtype=torch.int32, device=K.device)
    norms = torch.empty(n, dtype=torch.int32, device=K.device)
    t = np.ascontiguousarray(table, dtype=np.uint8)
    _check(load().qtq_quant_keys(_ptr(K), n, bits, _ptr(Pi), _ptr(S), float(delta), t.ctypes.data_as(ctypes.c_void_p),
                                 _ptr(codes), _ptr(signs), _ptr(norms), _stream(stream)), "qtq_quant_keys")
    return codes, signs, norms


def qtq_project(S: torch.Tensor, Pi: torch.Tensor, stream=None) -> torch.Tensor:
    """S Pi (fp64, device), the second matrix qtq_logits takes."""
    _need_numel(S, 128 * 128, "S", (torch.float64,))
    _need_numel(Pi, 128 * 128, "Pi", (torch.float64,))
    _need_cuda(S, Pi)
    out = torch.empty((128, 128), dtype=torch.float64, device=S.device)
    _check(load().qtq_project(_ptr(S), _ptr(Pi), _ptr(out), _stream(stream)), "qtq_project")
    return out


def qtq_logits(codes, signs, norms, n: int, heads: int, bits: int, delta: float, table, Pi, SPi, Qv: torch.Tensor,
               out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """out[heads][nq][n] fp32 logits for queries Qv[heads][nq][128] (fp32);
    SPi = qtq_project(S, Pi)."""
    import numpy as np
    if Qv.dim() != 3 or Qv.shape[0] != heads or Qv.shape[2] != 128 or Qv.dtype != torch.float32:
        raise ValueError(f"queries must be fp32 [{heads}][nq][128]")
    nq = Qv.shape[1]
    cb, sb, nb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qtq_sizes(n * heads, bits, ctypes.byref(cb), ctypes.byref(sb), ctypes.byref(nb)), "qtq_sizes")
    _need_bytes(codes, cb.value, "codes")
    _need_bytes(signs, sb.value, "signs")
    _need_bytes(norms, nb.value, "norms")
    _need_numel(Pi, 128 * 128, "Pi", (torch.float64,))
    _need_numel(SPi, 128 * 128, "SPi", (torch.float64,))
    if out is None:
        out = torch.empty((heads, nq, n), dtype=torch.float32, device=Qv.device)
    _need_numel(out, heads * nq * n, "out", (torch.float32,))
    need = ctypes.c_size_t()
    _check(load().qtq_logits_ws(heads, nq, ctypes.byref(need)), "qtq_logits_ws")
    if ws is None:
        ws = torch.empty(need.value, dtype=torch.uint8, device=Qv.device)
    _need_bytes(ws, need.value, "ws")
    t = np.ascontiguousarray(table, dtype=np.uint8)
    _need_cuda(codes, signs, norms, Pi, SPi, Qv, out, ws)
    _check(load().qtq_logits(_ptr(codes), _ptr(signs), _ptr(norms), n, heads, bits, float(delta),
                             t.ctypes.data_as(ctypes.c_void_p), _ptr(Pi), _ptr(SPi), _ptr(Qv), nq, _ptr(out), _ptr(ws),
                             ws.numel(), _stream(stream)), "qtq_logits")
    return out


def qtq_quant_values(V: torch.Tensor, bits: int, Pi: torch.Tensor, delta: float, table, stream=None):
    """(codes int32[n*4*bits], norms int32[n]) for fp32 values V[n][128]."""
    import numpy as np
    if V.dim() != 2 or V.shape[1] != 128 or V.dtype != torch.float32:
        raise ValueError("values must be fp32 [n][128]")
    _need_numel(Pi, 128 * 128, "Pi", (torch.float64,))
    _need_cuda(V, Pi)
    n = V.shape[0]
    codes = torch.empty(n * 4 * bits, dtype=torch.int32, device=V.device)
    norms = torch.empty(n, dtype=torch.int32, device=V.device)
    t = np.ascontiguousarray(table, dtype=np.uint8)
    _check(load().qtq_quant_values(_ptr(V), n, bits, _ptr(Pi), float(delta), t.ctypes.data_as(ctypes.c_void_p),
                                   _ptr(codes), _ptr(norms), _stream(stream)), "qtq_quant_values")
    return codes, norms


def qtq_attend_ws(n: int, heads: int, nq: int) -> int:
    need = ctypes.c_size_t()
    _check(load().qtq_attend_ws(n, heads, nq, ctypes.byref(need)), "qtq_attend_ws")
    return need.value


def qtq_attend(codes, norms, n: int, heads: int, bits: int, delta: float, table, Pi, P: torch.Tensor,
               out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """out[heads][nq][128] = P[heads][nq][n] times the dequantized values."""
    import numpy as np
    if P.dim() != 3 or P.shape[0] != heads or P.shape[2] != n or P.dtype != torch.float32:
        raise ValueError(f"weights must be fp32 [{heads}][nq][{n}]")
    nq = P.shape[1]
    _need_bytes(codes, n * heads * 16 * bits, "codes")
    _need_bytes(norms, n * heads * 4, "norms")
    _need_numel(Pi, 128 * 128, "Pi", (torch.float64,))
    if out is None:
        out = torch.empty((heads, nq, 128), dtype=torch.float32, device=P.device)
    _need_numel(out, heads * nq * 128, "out", (torch.float32,))
    need = qtq_attend_ws(n, heads, nq)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=P.device)
    _need_bytes(ws, need, "ws")
    t = np.ascontiguousarray(table, dtype=np.uint8)
    _need_cuda(codes, norms, Pi, P, out, ws)
    _check(load().qtq_attend(_ptr(codes), _ptr(norms), n, heads, bits, float(delta), t.ctypes.data_as(ctypes.c_void_p),
                             _ptr(Pi), _ptr(P), nq, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "qtq_attend")
    return out


# ---------------------------------------------------------------- binary LR
def qbinlr_sizes(N: int, K: int, r: int, B: int = 1):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qbinlr_sizes(N, K, r, B, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "qbinlr_sizes")
    return a.value, b.value, c.value


def qpack_binlr(U: torch.Tensor, V: torch.Tensor, ubits=None, vtbits=None, stream=None):
    if U.dim() != 2 or V.dim() != 2 or U.dtype != torch.int8 or V.dtype != torch.int8 or U.shape[1] != V.shape[1]:
        raise ValueError("U [N][r] and V [K][r] must be int8 with the same r")
    N, r = U.shape
    K = V.shape[0]
    ub, vb, _ = qbinlr_sizes(N, K, r)
    if ubits is None:
        ubits = torch.empty(ub // 4, dtype=torch.int32, device=U.device)
    if vtbits is None:
        vtbits = torch.empty(vb // 4, dtype=torch.int32, device=U.device)
    _need_bytes(ubits, ub, "ubits")
    _need_bytes(vtbits, vb, "vtbits")
    _need_cuda(U, V, ubits, vtbits)
    _check(load().qpack_binlr(_ptr(U), _ptr(V), N, K, r, _ptr(ubits), _ptr(vtbits), _stream(stream)),
           "qpack_binlr")
    return ubits, vtbits


def qunpack_binlr(ubits, vtbits, N: int, K: int, r: int, stream=None):
    ub, vb, _ = qbinlr_sizes(N, K, r)
    _need_bytes(ubits, ub, "ubits")
    _need_bytes(vtbits, vb, "vtbits")
    U = torch.empty((N, r), dtype=torch.int8, device=ubits.device)
    V = torch.empty((K, r), dtype=torch.int8, device=ubits.device)
    _need_cuda(ubits, vtbits)
    _check(load().qunpack_binlr(_ptr(ubits), _ptr(vtbits), N, K, r, _ptr(U), _ptr(V), _stream(stream)),
           "qunpack_binlr")
    return U, V


def qgemv_binlr(ubits, vtbits, s1, s2, N: int, K: int, r: int, x: torch.Tensor,
                y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                y_dtype=torch.float32, stream=None):
    B = _batch(x, K)
    ub, vb, wsb = qbinlr_sizes(N, K, r, B)
    _need_bytes(ubits, ub, "ubits")
    _need_bytes(vtbits, vb, "vtbits")
    _need_numel(s1, N, "s1", _H16, exact=False)
    _need_numel(s2, K, "s2", _H16, exact=False)
    if ws is None:
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _need_bytes(ws, wsb, "ws")
    if y is None:
        y = torch.empty((B, N), dtype=y_dtype, device=x.device)
    _need_numel(y, B * N, "y", _OUT)
    _need_cuda(ubits, vtbits, s1, s2, x, y, ws)
    _check(load().qgemv_binlr(_ptr(ubits), _ptr(vtbits), _ptr(s1), _ptr(s2), N, K, r, _ptr(x),
                              _dtype_code(x), B, _ptr(y), _dtype_code(y), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "qgemv_binlr")
    return y


def qgemv_binlr_noalloc(ubits, vtbits, s1, s2, N: int, K: int, r: int, x: torch.Tensor,
                        y: Optional[torch.Tensor] = None, y_dtype=torch.float32, stream=None):
    """qgemv_binlr with the library's per-device scratch array as workspace
    (no workspace argument; the C call allocates nothing).  Pass y to keep
    the whole call free of allocations."""
    B = _batch(x, K)
    ub, vb, _ = qbinlr_sizes(N, K, r, B)
    _need_bytes(ubits, ub, "ubits")
    _need_bytes(vtbits, vb, "vtbits")
    _need_numel(s1, N, "s1", _H16, exact=False)
    _need_numel(s2, K, "s2", _H16, exact=False)
    if y is None:
        y = torch.empty((B, N), dtype=y_dtype, device=x.device)
    _need_numel(y, B * N, "y", _OUT)
    _need_cuda(ubits, vtbits, s1, s2, x, y)
    _check(load().qgemv_binlr_noalloc(_ptr(ubits), _ptr(vtbits), _ptr(s1), _ptr(s2), N, K, r, _ptr(x),
                                      _dtype_code(x), B, _ptr(y), _dtype_code(y), _stream(stream)),
           "qgemv_binlr_noalloc")
    return y


# -------------------------------------------------------------- measurement
def qstream_read(buf: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Read buf once as a plain 16-byte nontemporal stream (bandwidth
    reference); out is a device int32 scratch word."""
    nbytes = _nbytes(buf)
    if nbytes % 16:
        raise ValueError("buf: size not a multiple of 16 bytes")
    _need_bytes(out, 4, "out")
    _need_cuda(buf, out)
    _check(load().qstream_read(_ptr(buf), nbytes, _ptr(out), _stream(stream)), "qstream_read")


# ------------------------------------------------------------------ prefill
def make_qweight_group(codes, meta, N, K, bits, group, side=None, idx=None, book_ids=None,
                       books=None) -> qweight:
    """A qweight descriptor (optionally with outlier side columns, or with
    per-group books of a dictionary); it keeps references to the tensors it
    points into."""
    n_out = 0 if idx is None else idx.numel()
    cb, mb = qgroup_sizes(N, K, bits, group)
    _need_bytes(codes, cb, "codes")
    _need_bytes(meta, mb, "meta")
    if n_out:
        _need_numel(idx, n_out, "idx", (torch.int32,))
        _need_numel(side, N * n_out, "side", _H16, exact=False)
    if books is not None:
        _need_numel(books, books.shape[0] << bits, "books", (torch.uint8,), exact=False)
        _need_numel(book_ids, N * (K // group), "book_ids", (torch.uint8,), exact=False)
    _need_cuda(codes, meta, side, idx, book_ids, books)
    w = qweight(Q_FMT_GROUP, N, K, bits, group, codes.data_ptr(), meta.data_ptr(), 0, None, None, None, None,
                side.data_ptr() if n_out else None, idx.data_ptr() if n_out else None, n_out,
                None if book_ids is None else book_ids.data_ptr(), None if books is None else books.data_ptr(),
                0 if books is None else books.shape[0])
    w._tensors = (codes, meta, side, idx, book_ids, books)
    return w


def make_qweight_binlr(ubits, vtbits, s1, s2, N, K, r) -> qweight:
    """A qweight descriptor; it keeps references to the tensors it points into."""
    ub, vb, _ = qbinlr_sizes(N, K, r)
    _need_bytes(ubits, ub, "ubits")
    _need_bytes(vtbits, vb, "vtbits")
    _need_numel(s1, N, "s1", _H16, exact=False)
    _need_numel(s2, K, "s2", _H16, exact=False)
    _need_cuda(ubits, vtbits, s1, s2)
    w = qweight(Q_FMT_BINLR, N, K, 0, 0, None, None, r, ubits.data_ptr(), vtbits.data_ptr(),
                s1.data_ptr(), s2.data_ptr())
    w._tensors = (ubits, vtbits, s1, s2)
    return w


def qgemm_prefill_ws(w: qweight, M: int) -> int:
    n = ctypes.c_size_t()
    _check(load().qgemm_prefill_ws(ctypes.byref(w), M, ctypes.byref(n)), "qgemm_prefill_ws")
    return n.value


def qgemm_prefill(w: qweight, X: torch.Tensor, Y: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, y_dtype=torch.float32, stream=None):
    if X.dim() != 2 or X.shape[1] != w.K:
        raise ValueError(f"X must be [M][{w.K}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    need = qgemm_prefill_ws(w, M)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=X.device)
    if need:
        _need_bytes(ws, need, "ws")
    if Y is None:
        Y = torch.empty((M, w.N), dtype=y_dtype, device=X.device)
    _need_numel(Y, M * w.N, "Y", _OUT)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _need_cuda(X, Y, ws, *w._tensors)
    _check(load().qgemm_prefill(ctypes.byref(w), _ptr(X), _dtype_code(X), M, _ptr(Y), _dtype_code(Y),
                                _ptr(ws), nbytes, _stream(stream)), "qgemm_prefill")
    return Y
