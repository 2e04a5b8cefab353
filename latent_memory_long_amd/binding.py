"""Python binding of libmsa.so: the C entry points of include/msa.h, same names.

Only argument marshalling happens here: torch tensors provide device memory, pinned host
memory and the current stream; shapes and pointers are passed to the library, and every
step of the path runs in its HIP kernels.  If the library is missing the import fails:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MSA_LIBRARY names another build of the same library (the host-sanitizer build of the
# tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP, MSA_ERR_IO = range(6)
MSA_F32, MSA_BF16 = 0, 1
MSA_ROPE_K, MSA_ROPE_V, MSA_ROPE_KR = 1, 2, 4


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"msa status {status}: {message}")
        self.status = status
        self.message = message


class BankInfo(ctypes.Structure):
    """msa_bank_info of include/msa.h."""
    _fields_ = [("dtype", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_docs", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("h_r", ctypes.c_int32), ("d", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("rope_mask", ctypes.c_uint32), ("rope_base", ctypes.c_float),
                ("reserved", ctypes.c_int32), ("n_tokens", ctypes.c_int64), ("n_chunks", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python latent_memory_long_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ, U32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t, ctypes.c_uint32)
    sig = {
        "msa_version": (I32, []),
        "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "msa_last_error": (ctypes.c_char_p, []),
        "msa_chunk_offsets": (I64, [P, I32, I32, P]),
        "msa_krbar_elems": (I64, [ctypes.c_int, I64, I32, I32]),
        "msa_krbar_pack": (ctypes.c_int, [ctypes.c_int, I64, I32, I32, P, P, P]),
        "msa_krbar_unpack": (ctypes.c_int, [ctypes.c_int, I64, I32, I32, P, P, P]),
        "msa_pool": (ctypes.c_int, [ctypes.c_int, I32, I64, I64, P, P, I32, I32, I32, I32, F, U32,
                                    P, P, P, P, P, P, P]),
        "msa_route_scan": (ctypes.c_int, [ctypes.c_int, I32, I64, P, I32, P, I32, I32, I32, I64, P,
                                          P, P, P, P, P]),
        "msa_topk_workspace": (SZ, [I32, I32, I32]),
        "msa_topk": (ctypes.c_int, [I32, I32, P, I32, P, P, P, SZ, P]),
        "msa_route_topk_workspace": (SZ, [I32, I32, I32]),
        "msa_route_topk_noalloc": (ctypes.c_int, [ctypes.c_int, I32, I64, P, I32, P, I32, I32, I32, I64, P,
                                                  P, I32, P, P, P, P]),
        "msa_route_topk": (ctypes.c_int, [ctypes.c_int, I32, I64, P, I32, P, I32, I32, I32, I64, P,
                                          P, I32, P, P, P, P, SZ, P]),
        "msa_sparse_attn_workspace": (SZ, [ctypes.c_int, I32, I64, I64, I32, I32, I32, I32]),
        "msa_sparse_attn": (ctypes.c_int, [ctypes.c_int, I32, I64, I64, P, P, I32, P, P, P, I32, I32,
                                           I32, F, F, I32, P, I32, I64, P, P, P, I32, P, P, P, SZ, P]),
        "msa_sparse_attn_backward_workspace": (SZ, [I64, I64, I32, I32, I32]),
        "msa_sparse_attn_backward": (ctypes.c_int, [ctypes.c_int, I32, I64, I64, P, P, I32, P, P, P, I32,
                                                    I32, I32, F, F, I32, P, I32, I64, P, P, P, I32, P, P,
                                                    P, P, P, P, P, P, P, SZ, P]),
        "msa_route_aux_loss": (ctypes.c_int, [I32, I32, I32, P, P, F, P, P, P]),
        "msa_bank_save": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(BankInfo), P, P, P, P, P]),
        "msa_bank_read_info": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(BankInfo)]),
        "msa_bank_load": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(BankInfo), P, P, P, P, P]),
        "msa_route_backward_workspace": (SZ, [I32, I32, I64, I32]),
        "msa_route_backward": (ctypes.c_int, [ctypes.c_int, I32, I64, P, I32, P, I32, I32, I32, I64, P,
                                              P, P, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int):
    if status != MSA_OK:
        raise MsaError(status, lib.msa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    raise MsaError(MSA_ERR_UNSUPPORTED, f"dtype {t.dtype} (need float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MsaError(MSA_ERR_INVALID_ARG, "tensor must be contiguous")
    return t.data_ptr()


_FLOAT = (torch.float32, torch.bfloat16)


def _need(t, name: str, dtype=None, shape=None):
    """Refuse a tensor argument whose dtype, shape or layout does not match what the C entry
    point will read through its pointer (a wrong integer width there would be read as
    garbage offsets).  ``dtype`` is one dtype or a tuple of allowed ones; ``shape`` a tuple
    whose None entries match any size."""
    if not isinstance(t, torch.Tensor):
        raise MsaError(MSA_ERR_INVALID_ARG, f"{name} must be a torch tensor (got {type(t).__name__})")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if dtype is not None and t.dtype not in allowed:
        raise MsaError(MSA_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, need {' or '.join(map(str, allowed))}")
    if shape is not None:
        bad = t.dim() != len(shape) or any(w is not None and int(n) != int(w) for n, w in zip(t.shape, shape))
        if bad:
            want = "(" + ", ".join("*" if w is None else str(int(w)) for w in shape) + ")"
            raise MsaError(MSA_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, need {want}")
    if not t.is_contiguous():
        raise MsaError(MSA_ERR_INVALID_ARG, f"{name} must be contiguous")
    return t


def _same_device(*named, pinned_ok=()):
    """Every named tensor on one GPU; those listed in ``pinned_ok`` may instead be in
    page-locked host memory.  None entries are skipped."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.is_cuda:
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise MsaError(MSA_ERR_INVALID_ARG, f"{name} is on {t.device}, other arguments on {dev}")
        elif name in pinned_ok and t.is_pinned():
            continue
        else:
            where = "a device tensor or pinned host memory" if name in pinned_ok else "a device tensor"
            raise MsaError(MSA_ERR_INVALID_ARG, f"{name} must be {where}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        _need(ws, "workspace")
        _same_device(("workspace", ws))
        if ws.numel() * ws.element_size() >= nbytes:
            return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- routing keys

class RouteKeys:
    """The routing keys Kr-bar of a bank (n_chunks rows of h_r heads of dim d), in the
    library's bank layout (include/msa.h, "Routing-key bank layout"): bf16 keys in tiles of
    16 rows laid out as matrix-core operands, float32 keys row-major.  ``data`` is a flat
    tensor of msa_krbar_elems() elements; it is not indexable by row -- ``rows()`` returns
    the keys as a row-major [n_chunks, h_r, d] tensor, ``from_rows()`` builds the layout
    from one."""

    __slots__ = ("data", "n_chunks", "h_r", "d")

    def __init__(self, data: torch.Tensor, n_chunks: int, h_r: int, d: int):
        n_chunks, h_r, d = int(n_chunks), int(h_r), int(d)
        _need(data, "RouteKeys data", _FLOAT)
        _need(data, "RouteKeys data", _FLOAT, (msa_krbar_elems(_dtype_code(data), n_chunks, h_r, d),))
        self.data, self.n_chunks, self.h_r, self.d = data, n_chunks, h_r, d

    @property
    def dtype(self):
        return self.data.dtype

    @property
    def device(self):
        return self.data.device

    @property
    def is_cuda(self):
        return self.data.is_cuda

    @property
    def shape(self):
        """The logical shape (n_chunks, h_r, d)."""
        return (self.n_chunks, self.h_r, self.d)

    @staticmethod
    def empty(n_chunks: int, h_r: int, d: int, dtype=torch.bfloat16, device="cuda", pin_memory: bool = False,
              zero: bool = False):
        """Storage for n_chunks rows; ``zero`` fills it with zeros (padding rows included, so
        banks pooled into it compare equal bit for bit)."""
        n = msa_krbar_elems(_dtype_code_of(dtype), n_chunks, h_r, d)
        make = torch.zeros if zero else torch.empty
        if pin_memory:
            return RouteKeys(make(n, dtype=dtype, pin_memory=True), n_chunks, h_r, d)
        return RouteKeys(make(n, dtype=dtype, device=device), n_chunks, h_r, d)

    @staticmethod
    def from_rows(rows: torch.Tensor, stream=None) -> "RouteKeys":
        """Routing keys from a row-major [n_chunks, h_r, d] device tensor (msa_krbar_pack)."""
        _need(rows, "rows", _FLOAT, (None, None, None))
        _same_device(("rows", rows))
        C, h_r, d = rows.shape
        keys = RouteKeys.empty(C, h_r, d, rows.dtype, rows.device)
        msa_krbar_pack(rows, keys, stream)
        return keys

    def rows(self, stream=None) -> torch.Tensor:
        """The keys as a new row-major [n_chunks, h_r, d] tensor on the same device
        (msa_krbar_unpack)."""
        out = torch.empty(self.shape, dtype=self.dtype, device=self.device)
        msa_krbar_unpack(self, out, stream)
        return out

    def to(self, device, non_blocking: bool = False) -> "RouteKeys":
        return RouteKeys(self.data.to(device, non_blocking=non_blocking), self.n_chunks, self.h_r, self.d)

    def cpu(self) -> "RouteKeys":
        return self.to("cpu")

    def clone(self) -> "RouteKeys":
        return RouteKeys(self.data.clone(), self.n_chunks, self.h_r, self.d)

    def grown(self, n_chunks: int) -> "RouteKeys":
        """A copy with room for n_chunks >= self.n_chunks rows: the existing rows keep their
        place, so msa_pool can write new documents after them (offsets starting at the old
        row count)."""
        if n_chunks < self.n_chunks:
            raise MsaError(MSA_ERR_INVALID_ARG, f"cannot shrink routing keys from {self.n_chunks} to {n_chunks} rows")
        out = RouteKeys.empty(n_chunks, self.h_r, self.d, self.dtype, self.device, zero=True)
        out.data[: self.data.numel()].copy_(self.data)
        return out

    def equal(self, other: "RouteKeys") -> bool:
        return (isinstance(other, RouteKeys) and self.shape == other.shape and self.dtype == other.dtype
                and torch.equal(self.data, other.data))

    def __repr__(self):
        return f"RouteKeys(n_chunks={self.n_chunks}, h_r={self.h_r}, d={self.d}, dtype={self.dtype}, device={self.device})"


def _dtype_code_of(dtype) -> int:
    if dtype == torch.float32:
        return MSA_F32
    if dtype == torch.bfloat16:
        return MSA_BF16
    raise MsaError(MSA_ERR_UNSUPPORTED, f"dtype {dtype} (need float32 or bfloat16)")


def _keys(K, name: str = "Krbar") -> RouteKeys:
    """Routing keys as a RouteKeys: float32 keys may also be a row-major [C, h_r, d] tensor."""
    if isinstance(K, RouteKeys):
        return K
    if isinstance(K, torch.Tensor) and K.dtype == torch.float32 and K.dim() == 3 and K.is_contiguous():
        return RouteKeys(K.view(-1), K.shape[0], K.shape[1], K.shape[2])
    raise MsaError(MSA_ERR_INVALID_ARG, f"{name} must be a RouteKeys (bf16 keys are stored in the tiled bank "
                                        f"layout; RouteKeys.from_rows packs row-major keys), or for float32 a "
                                        f"[C, h_r, d] tensor")


def msa_krbar_elems(dtype: int, n_chunks: int, h_r: int, d: int) -> int:
    """Elements of routing-key storage for a bank of n_chunks rows."""
    n = int(lib.msa_krbar_elems(dtype, n_chunks, h_r, d))
    if n < 0:
        raise MsaError(MSA_ERR_INVALID_ARG, msa_last_error())
    return n


def msa_krbar_pack(rows: torch.Tensor, keys: RouteKeys, stream=None):
    """Row-major [n_chunks, h_r, d] -> the bank layout (padding rows written as zero)."""
    _need(rows, "rows", keys.dtype, keys.shape)
    _same_device(("rows", rows), ("keys", keys.data))
    _check(lib.msa_krbar_pack(_dtype_code(rows), keys.n_chunks, keys.h_r, keys.d, _ptr(rows), _ptr(keys.data),
                              _stream(stream)))


def msa_krbar_unpack(keys: RouteKeys, rows: torch.Tensor, stream=None):
    """The bank layout -> row-major [n_chunks, h_r, d]."""
    _need(rows, "rows", keys.dtype, keys.shape)
    _same_device(("rows", rows), ("keys", keys.data))
    _check(lib.msa_krbar_unpack(_dtype_code(rows), keys.n_chunks, keys.h_r, keys.d, _ptr(keys.data), _ptr(rows),
                                _stream(stream)))


# ----------------------------------------------------------------------------- entry points

def msa_version() -> int:
    return int(lib.msa_version())


def msa_status_string(status: int) -> str:
    return lib.msa_status_string(status).decode()


def msa_last_error() -> str:
    return lib.msa_last_error().decode()


def msa_chunk_offsets(doc_tok_off, chunk: int = 64) -> np.ndarray:
    """Host-side bank layout: chunk_off[N+1] (int64) from token offsets."""
    off = np.ascontiguousarray(np.asarray(doc_tok_off, dtype=np.int64))
    n = len(off) - 1
    out = np.zeros(max(n + 1, 1), dtype=np.int64)
    c = lib.msa_chunk_offsets(off.ctypes.data, n, chunk, out.ctypes.data)
    if c < 0:
        raise MsaError(MSA_ERR_INVALID_ARG, msa_last_error())
    return out


def msa_pool(K: torch.Tensor, V: torch.Tensor, Kr: torch.Tensor, doc_tok_off: torch.Tensor,
             chunk_off: torch.Tensor, n_chunks: int, chunk: int = 64, rope_base: float = 1e6,
             rope_mask: int = MSA_ROPE_K, out=None, stream=None):
    """Step A.  K, V [T, h_kv, d]; Kr [T, h_r, d]; offsets int64 on the device; n_chunks the
    rows written.  Returns (Kbar, Vbar [rows, h_kv, d], Krbar RouteKeys).  chunk_off gives
    each document's first bank row: to grow a bank, pass it as ``out`` (its K-bar / V-bar
    and RouteKeys sized for the grown bank, e.g. RouteKeys.grown) with offsets that start
    at the rows it already holds."""
    _need(K, "K", _FLOAT, (None, None, None))
    T, h_kv, d = K.shape
    _need(V, "V", K.dtype, (T, h_kv, d))
    _need(Kr, "Kr", K.dtype, (T, None, d))
    h_r = Kr.shape[1]
    _need(doc_tok_off, "doc_tok_off", torch.int64, (None,))
    _need(chunk_off, "chunk_off", torch.int64, (doc_tok_off.numel(),))
    if out is None:
        out = (torch.empty((n_chunks, h_kv, d), dtype=K.dtype, device=K.device),
               torch.empty((n_chunks, h_kv, d), dtype=K.dtype, device=K.device),
               RouteKeys.empty(n_chunks, h_r, d, K.dtype, K.device, zero=True))
    Kb, Vb, Krb = out
    Krb = _keys(Krb)
    _need(Kb, "Kbar", K.dtype, (None, h_kv, d))
    _need(Vb, "Vbar", K.dtype, (Kb.shape[0], h_kv, d))
    if Krb.dtype != K.dtype or Krb.h_r != h_r or Krb.d != d or Krb.n_chunks != Kb.shape[0] or Kb.shape[0] < n_chunks:
        raise MsaError(MSA_ERR_INVALID_ARG, f"bank buffers hold {Kb.shape[0]} K-bar rows and {Krb} for {n_chunks} "
                                            f"rows of h_r={h_r}, d={d}, {K.dtype}")
    _same_device(("K", K), ("V", V), ("Kr", Kr), ("doc_tok_off", doc_tok_off), ("chunk_off", chunk_off),
                 ("Kbar", Kb), ("Vbar", Vb), ("Krbar", Krb.data))
    _check(lib.msa_pool(_dtype_code(K), doc_tok_off.numel() - 1, T, n_chunks, _ptr(doc_tok_off),
                        _ptr(chunk_off), h_kv, h_r, d, chunk, rope_base, rope_mask, _ptr(K), _ptr(V),
                        _ptr(Kr), _ptr(Kb), _ptr(Vb), _ptr(Krb.data), _stream(stream)))
    return Kb, Vb, Krb


def msa_route_scan(Qr: torch.Tensor, q_off: torch.Tensor, max_q_len: int, Krbar: torch.Tensor,
                   chunk_off: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
                   rows: Optional[tuple] = None):
    """Step B.  Returns every document's score, float32 [B, N].  For training pass `rows` =
    (float32 [B, C], int32 [B, C]) device tensors to also get each bank row's best token
    score and the first token reaching it, which msa_route_backward can reuse."""
    Krbar = _keys(Krbar)
    B, N = _route_inputs(Qr, q_off, Krbar, chunk_off)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=Krbar.device)
    _need(out, "doc_scores", torch.float32, (B, N))
    _route_devices(Qr, q_off, Krbar, chunk_off, ("doc_scores", out))
    _check(lib.msa_route_scan(_dtype_code(Krbar.data), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr),
                              Krbar.h_r, Krbar.d, N, Krbar.n_chunks, _ptr(chunk_off),
                              _ptr(Krbar.data), _ptr(out), *_rows(rows, B, Krbar.n_chunks), _stream(stream)))
    return out


def _route_inputs(Qr, q_off, Krbar: RouteKeys, chunk_off):
    """Checks of the router's inputs; returns (queries, documents)."""
    _need(Qr, "Qr", Krbar.dtype, (None, Krbar.h_r, Krbar.d))
    _need(q_off, "q_off", torch.int32, (None,))
    _need(chunk_off, "chunk_off", torch.int64, (None,))
    return q_off.numel() - 1, chunk_off.numel() - 1


def _route_devices(Qr, q_off, Krbar: RouteKeys, chunk_off, *outputs):
    _same_device(("Krbar", Krbar.data), ("Qr", Qr), ("q_off", q_off), ("chunk_off", chunk_off), *outputs)


def _rows(rows: Optional[tuple], B: int, C: int):
    """Pointers of a (row scores, row args) pair, checked, or two nulls."""
    if rows is None:
        return None, None
    rs, ra = rows
    if (rs.dtype != torch.float32 or ra.dtype != torch.int32 or tuple(rs.shape) != (B, C)
            or tuple(ra.shape) != (B, C) or not (rs.is_cuda and ra.is_cuda)):
        raise MsaError(MSA_ERR_INVALID_ARG, f"rows must be float32 and int32 device tensors of shape ({B}, {C})")
    return _ptr(rs), _ptr(ra)


def msa_topk_workspace(n_queries: int, n_docs: int, k: int) -> int:
    return int(lib.msa_topk_workspace(n_queries, n_docs, k))


def msa_topk(doc_scores: torch.Tensor, k: int, out=None, workspace: Optional[torch.Tensor] = None,
             stream=None):
    """Step C.  doc_scores float32 [B, N] -> (ids int32 [B, k], scores float32 [B, k])."""
    _need(doc_scores, "doc_scores", torch.float32, (None, None))
    B, N = doc_scores.shape
    if out is None:
        out = (torch.empty((B, k), dtype=torch.int32, device=doc_scores.device),
               torch.empty((B, k), dtype=torch.float32, device=doc_scores.device))
    ids, sc = out
    _need(ids, "topk_ids", torch.int32, (B, k))
    _need(sc, "topk_scores", torch.float32, (B, k))
    _same_device(("doc_scores", doc_scores), ("topk_ids", ids), ("topk_scores", sc))
    need = msa_topk_workspace(B, N, k)
    ws = _workspace(need, doc_scores.device, workspace) if need else None
    _check(lib.msa_topk(B, N, _ptr(doc_scores), k, _ptr(ids), _ptr(sc), _ptr(ws),
                        need and ws.numel() * ws.element_size(), _stream(stream)))
    return ids, sc


def msa_route_topk_workspace(n_queries: int, n_docs: int, k: int) -> int:
    return int(lib.msa_route_topk_workspace(n_queries, n_docs, k))


def msa_route_topk(Qr: torch.Tensor, q_off: torch.Tensor, max_q_len: int, Krbar: torch.Tensor,
                   chunk_off: torch.Tensor, k: int, want_doc_scores: bool = False, out=None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Steps B + C.  Qr [total_q, h_r, d]; q_off int32 [B+1]; Krbar the bank's RouteKeys.
    Returns (topk_ids int32 [B,k], topk_scores f32 [B,k], doc_scores f32 [B,N] or None)."""
    Krbar = _keys(Krbar)
    B, N = _route_inputs(Qr, q_off, Krbar, chunk_off)
    dev = Krbar.device
    if out is None:
        out = (torch.empty((B, k), dtype=torch.int32, device=dev),
               torch.empty((B, k), dtype=torch.float32, device=dev),
               torch.empty((B, N), dtype=torch.float32, device=dev) if want_doc_scores else None)
    ids, sc, ds = out
    _need(ids, "topk_ids", torch.int32, (B, k))
    _need(sc, "topk_scores", torch.float32, (B, k))
    if ds is not None:
        _need(ds, "doc_scores", torch.float32, (B, N))
    _route_devices(Qr, q_off, Krbar, chunk_off, ("topk_ids", ids), ("topk_scores", sc), ("doc_scores", ds))
    ws, wsb = None, 0
    need = msa_route_topk_workspace(B, N, k) if ds is None else msa_topk_workspace(B, N, k)
    if need:
        ws = _workspace(need, dev, workspace)
        wsb = ws.numel() * ws.element_size()
    _check(lib.msa_route_topk(_dtype_code(Krbar.data), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr),
                              Krbar.h_r, Krbar.d, N, Krbar.n_chunks, _ptr(chunk_off),
                              _ptr(Krbar.data), k, _ptr(ids), _ptr(sc), _ptr(ds), _ptr(ws), wsb,
                              _stream(stream)))
    return ids, sc, ds


MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20


def msa_route_topk_noalloc(Qr: torch.Tensor, q_off: torch.Tensor, max_q_len: int, Krbar, chunk_off: torch.Tensor,
                           k: int, want_doc_scores: bool = False, out=None, stream=None):
    """msa_route_topk without a workspace: the library's per-device scratch array serves
    instead (MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES; larger inputs raise MSA_ERR_WORKSPACE).
    Pass `out` = (topk_ids, topk_scores, doc_scores or None) to allocate nothing here either."""
    Krbar = _keys(Krbar)
    B, N = _route_inputs(Qr, q_off, Krbar, chunk_off)
    dev = Krbar.device
    if out is None:
        out = (torch.empty((B, k), dtype=torch.int32, device=dev),
               torch.empty((B, k), dtype=torch.float32, device=dev),
               torch.empty((B, N), dtype=torch.float32, device=dev) if want_doc_scores else None)
    ids, sc, ds = out
    _need(ids, "topk_ids", torch.int32, (B, k))
    _need(sc, "topk_scores", torch.float32, (B, k))
    if ds is not None:
        _need(ds, "doc_scores", torch.float32, (B, N))
    _route_devices(Qr, q_off, Krbar, chunk_off, ("topk_ids", ids), ("topk_scores", sc), ("doc_scores", ds))
    _check(lib.msa_route_topk_noalloc(_dtype_code(Krbar.data), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr),
                                      Krbar.h_r, Krbar.d, N, Krbar.n_chunks, _ptr(chunk_off), _ptr(Krbar.data), k,
                                      _ptr(ids), _ptr(sc), _ptr(ds), _stream(stream)))
    return ids, sc, ds


def msa_sparse_attn_workspace(dtype: int, n_queries: int, total_q: int, total_kv: int,
                              max_q_len: int, hq: int, h_kv: int, d: int) -> int:
    return int(lib.msa_sparse_attn_workspace(dtype, n_queries, total_q, total_kv, max_q_len, hq,
                                             h_kv, d))


def msa_sparse_attn(Q: torch.Tensor, Kloc: torch.Tensor, Vloc: torch.Tensor, q_off: torch.Tensor,
                    kv_off: torch.Tensor, max_q_len: int, topk_ids: torch.Tensor,
                    chunk_off: torch.Tensor, Kbar: torch.Tensor, Vbar: torch.Tensor,
                    rope_base: float = 1e6, scale: float = 0.0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    lse: Optional[torch.Tensor] = None):
    """Step D.  Q [total_q, hq, d]; Kloc/Vloc [total_kv, h_kv, d]; Kbar/Vbar [C, h_kv, d] on the
    device, or in pinned host memory (then read over the host link).  Returns O.  Pass a
    float32 [total_q, hq] device tensor as `lse` to also get each row's log-sum-exp (natural
    log), which msa_sparse_attn_backward can reuse."""
    B, N, k, kv_source = _attn_inputs(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar)
    total_q, hq, d = Q.shape
    total_kv, h_kv, _ = Kloc.shape
    dev = Q.device
    if out is None:
        out = torch.empty_like(Q)
    _need(out, "O", Q.dtype, tuple(Q.shape))
    if lse is not None:
        _need(lse, "lse", torch.float32, (total_q, hq))
    _attn_devices(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar, ("O", out), ("lse", lse))
    code = _dtype_code(Q)
    _check_lse(lse, total_q, hq)
    need = msa_sparse_attn_workspace(code, B, total_q, total_kv, max_q_len, hq, h_kv, d)
    ws = _workspace(need, dev, workspace)
    _check(lib.msa_sparse_attn(code, B, total_q, total_kv, _ptr(q_off), _ptr(kv_off), max_q_len,
                               _ptr(Q), _ptr(Kloc), _ptr(Vloc), hq, h_kv, d, rope_base, scale, k,
                               _ptr(topk_ids), N, Kbar.shape[0], _ptr(chunk_off), _ptr(Kbar),
                               _ptr(Vbar), kv_source, _ptr(out), _ptr(lse), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))
    return out


def _attn_inputs(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar):
    """Checks of the attention's inputs; returns (queries, documents, k, kv_source)."""
    _need(Q, "Q", _FLOAT, (None, None, None))
    total_q, hq, d = Q.shape
    _need(Kloc, "Kloc", Q.dtype, (None, None, d))
    _need(Vloc, "Vloc", Q.dtype, tuple(Kloc.shape))
    h_kv = Kloc.shape[1]
    _need(q_off, "q_off", torch.int32, (None,))
    B = q_off.numel() - 1
    _need(kv_off, "kv_off", torch.int32, (B + 1,))
    _need(topk_ids, "topk_ids", torch.int32, (B, None))
    _need(chunk_off, "chunk_off", torch.int64, (None,))
    _need(Kbar, "Kbar", Q.dtype, (None, h_kv, d))
    _need(Vbar, "Vbar", Q.dtype, tuple(Kbar.shape))
    kv_source = 0 if Kbar.is_cuda else 1
    return B, chunk_off.numel() - 1, topk_ids.shape[1], kv_source


def _attn_devices(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar, *outputs):
    """Every tensor on one GPU, the bank's content rows there too or both in pinned host memory."""
    if Kbar.is_cuda != Vbar.is_cuda:
        raise MsaError(MSA_ERR_INVALID_ARG, "Kbar and Vbar must both be on the device or both in pinned host memory")
    _same_device(("Q", Q), ("Kloc", Kloc), ("Vloc", Vloc), ("q_off", q_off), ("kv_off", kv_off),
                 ("topk_ids", topk_ids), ("chunk_off", chunk_off), ("Kbar", Kbar), ("Vbar", Vbar), *outputs,
                 pinned_ok=("Kbar", "Vbar"))


def _check_lse(lse: Optional[torch.Tensor], total_q: int, hq: int):
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (total_q, hq) or not lse.is_cuda):
        raise MsaError(MSA_ERR_INVALID_ARG, f"lse must be a float32 device tensor of shape ({total_q}, {hq})")


def msa_sparse_attn_backward_workspace(total_q: int, total_kv: int, hq: int, h_kv: int, d: int) -> int:
    return int(lib.msa_sparse_attn_backward_workspace(total_q, total_kv, hq, h_kv, d))


def msa_sparse_attn_backward(Q: torch.Tensor, Kloc: torch.Tensor, Vloc: torch.Tensor, q_off: torch.Tensor,
                             kv_off: torch.Tensor, max_q_len: int, topk_ids: torch.Tensor,
                             chunk_off: torch.Tensor, Kbar: torch.Tensor, Vbar: torch.Tensor,
                             O: torch.Tensor, dO: torch.Tensor, rope_base: float = 1e6, scale: float = 0.0,
                             dbank: Optional[tuple] = None, out: Optional[tuple] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None,
                             lse: Optional[torch.Tensor] = None):
    """Backward of step D.  Returns (dQ, dKloc, dVloc, dKbar, dVbar), float32.  dKbar / dVbar
    ([n_chunks, h_kv, d] on the device) are added to: pass `dbank` to accumulate into your
    own arrays, else zero-filled ones are made.  `lse`: the forward's log-sum-exp output for
    the same inputs, which saves recomputing it."""
    B, N, k, kv_source = _attn_inputs(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar)
    total_q, hq, d = Q.shape
    total_kv, h_kv, _ = Kloc.shape
    C = Kbar.shape[0]
    _need(O, "O", Q.dtype, tuple(Q.shape))
    _need(dO, "dO", Q.dtype, tuple(Q.shape))
    dev = Q.device
    f32 = torch.float32
    if out is None:
        out = (torch.empty((total_q, hq, d), dtype=f32, device=dev),
               torch.empty((total_kv, h_kv, d), dtype=f32, device=dev),
               torch.empty((total_kv, h_kv, d), dtype=f32, device=dev))
    if dbank is None:
        dbank = (torch.zeros((C, h_kv, d), dtype=f32, device=dev), torch.zeros((C, h_kv, d), dtype=f32, device=dev))
    dQ, dKl, dVl = out
    dKb, dVb = dbank
    f32 = torch.float32
    _need(dQ, "dQ", f32, (total_q, hq, d))
    _need(dKl, "dKloc", f32, (total_kv, h_kv, d))
    _need(dVl, "dVloc", f32, (total_kv, h_kv, d))
    _need(dKb, "dKbar", f32, (C, h_kv, d))
    _need(dVb, "dVbar", f32, (C, h_kv, d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (total_q, hq))
    _attn_devices(Q, Kloc, Vloc, q_off, kv_off, topk_ids, chunk_off, Kbar, Vbar, ("O", O), ("dO", dO),
                  ("dQ", dQ), ("dKloc", dKl), ("dVloc", dVl), ("dKbar", dKb), ("dVbar", dVb), ("lse", lse))
    _check_lse(lse, total_q, hq)
    need = msa_sparse_attn_backward_workspace(total_q, total_kv, hq, h_kv, d)
    ws = _workspace(need, dev, workspace)
    _check(lib.msa_sparse_attn_backward(_dtype_code(Q), B, total_q, total_kv, _ptr(q_off), _ptr(kv_off),
                                        max_q_len, _ptr(Q), _ptr(Kloc), _ptr(Vloc), hq, h_kv, d, rope_base,
                                        scale, k, _ptr(topk_ids), N, C, _ptr(chunk_off), _ptr(Kbar),
                                        _ptr(Vbar), kv_source, _ptr(O), _ptr(lse), _ptr(dO), _ptr(dQ),
                                        _ptr(dKl),
                                        _ptr(dVl), _ptr(dKb), _ptr(dVb), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))
    return dQ, dKl, dVl, dKb, dVb


def msa_route_backward_workspace(n_queries: int, n_docs: int, n_chunks: int, h_r: int) -> int:
    return int(lib.msa_route_backward_workspace(n_queries, n_docs, n_chunks, h_r))


def msa_route_backward(Qr: torch.Tensor, q_off: torch.Tensor, max_q_len: int, Krbar: torch.Tensor,
                       chunk_off: torch.Tensor, dD: torch.Tensor, dKrbar: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None, rows: Optional[tuple] = None):
    """Backward of step B for a loss on the document scores.  dD float32 [B, N] on the
    device.  Returns (dQr, dKrbar), float32; dKrbar is added to (pass your own array to
    accumulate, else a zero-filled one is made).  `rows`: msa_route_scan's row outputs for
    the same inputs, which saves scanning the bank again."""
    Krbar = _keys(Krbar)
    B, N = _route_inputs(Qr, q_off, Krbar, chunk_off)
    C, h_r, d = Krbar.shape
    dev = Krbar.device
    if out is None:
        out = torch.empty((Qr.shape[0], h_r, d), dtype=torch.float32, device=dev)
    if dKrbar is None:
        dKrbar = torch.zeros((C, h_r, d), dtype=torch.float32, device=dev)
    _need(dD, "dD", torch.float32, (B, N))
    _need(out, "dQr", torch.float32, (Qr.shape[0], h_r, d))
    _need(dKrbar, "dKrbar", torch.float32, (C, h_r, d))
    _route_devices(Qr, q_off, Krbar, chunk_off, ("dD", dD), ("dQr", out), ("dKrbar", dKrbar))
    need = msa_route_backward_workspace(B, N, C, h_r)
    ws = _workspace(need, dev, workspace)
    _check(lib.msa_route_backward(_dtype_code(Krbar.data), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr), h_r,
                                  d, N, C, _ptr(chunk_off), _ptr(Krbar.data), _ptr(dD), *_rows(rows, B, C),
                                  _ptr(out), _ptr(dKrbar),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, dKrbar


MSA_AUX_BCE = 0
MSA_AUX_INFONCE = 1


def msa_route_aux_loss(doc_scores: torch.Tensor, labels: torch.Tensor, kind: int = MSA_AUX_BCE,
                       temperature: float = 1.0, out: Optional[tuple] = None, stream=None):
    """Routing auxiliary loss on float32 [B, N] document scores and labels (device).
    Returns (per-query loss [B], dL/dS [B, N]) for L = the mean of the per-query losses."""
    _need(doc_scores, "doc_scores", torch.float32, (None, None))
    B, N = doc_scores.shape
    _need(labels, "labels", torch.float32, (B, N))
    if out is None:
        out = (torch.empty(B, dtype=torch.float32, device=doc_scores.device),
               torch.empty((B, N), dtype=torch.float32, device=doc_scores.device))
    loss, dD = out
    _need(loss, "loss", torch.float32, (B,))
    _need(dD, "dD", torch.float32, (B, N))
    _same_device(("doc_scores", doc_scores), ("labels", labels), ("loss", loss), ("dD", dD))
    _check(lib.msa_route_aux_loss(kind, B, N, _ptr(doc_scores), _ptr(labels), temperature, _ptr(loss),
                                  _ptr(dD), _stream(stream)))
    return loss, dD


def _info_dict(info: BankInfo) -> dict:
    return {f: getattr(info, f) for f, _ in BankInfo._fields_ if f != "reserved"}


def msa_bank_save(path: str, doc_tok_off, chunk_off, layers, chunk: int = 64, rope_base: float = 1e6,
                  rope_mask: int = 1):
    """Writes a bank file.  layers: [(Krbar, Kbar, Vbar), ...] one tuple per routed layer,
    Krbar a RouteKeys (or a float32 [C, h_r, d] tensor), on any device (copied to host
    memory for the write)."""
    dto = np.ascontiguousarray(doc_tok_off, dtype=np.int64)
    cho = np.ascontiguousarray(chunk_off, dtype=np.int64)
    host = []
    for l, (Kr, K, V) in enumerate(layers):
        Kr = _keys(Kr, f"layer {l} Krbar")
        if Kr.n_chunks != int(cho[-1]) or K.shape[0] != int(cho[-1]) or V.shape != K.shape:
            raise MsaError(MSA_ERR_INVALID_ARG, f"layer {l}: {Kr}, K-bar {tuple(K.shape)}, V-bar {tuple(V.shape)} "
                                                f"for {int(cho[-1])} bank rows")
        host.append((Kr.data.detach().cpu(), K.detach().contiguous().cpu(), V.detach().contiguous().cpu()))
    Kr0, K0 = _keys(layers[0][0]), layers[0][1]
    info = BankInfo(_dtype_code(Kr0.data), len(layers), len(dto) - 1, K0.shape[1], Kr0.h_r, Kr0.d, chunk,
                    rope_mask, rope_base, 0, int(dto[-1]), int(cho[-1]))
    arr = lambda i: (ctypes.c_void_p * len(host))(*[h[i].data_ptr() for h in host])
    _check(lib.msa_bank_save(os.fsencode(path), ctypes.byref(info), dto.ctypes.data, cho.ctypes.data, arr(0), arr(1),
                             arr(2)))


def msa_bank_read_info(path: str) -> dict:
    info = BankInfo()
    _check(lib.msa_bank_read_info(os.fsencode(path), ctypes.byref(info)))
    return _info_dict(info)


def msa_bank_load(path: str, device=None, kv_device=None):
    """Reads a bank file.  Returns (doc_tok_off, chunk_off, layers, info): offsets as NumPy
    int64 arrays, layers as [(Krbar RouteKeys, Kbar, Vbar), ...].  Kr-bar goes to ``device`` and K-bar /
    V-bar to ``kv_device`` (default: ``device``; "cpu-pinned" for page-locked host memory);
    None keeps a tensor in host memory."""
    info = BankInfo()
    _check(lib.msa_bank_read_info(os.fsencode(path), ctypes.byref(info)))
    dt = torch.float32 if info.dtype == MSA_F32 else torch.bfloat16
    C, L = info.n_chunks, info.n_layers
    kvdev = device if kv_device is None else kv_device
    # host buffers are page-locked when they feed a device copy or are asked for as such
    kr = [RouteKeys.empty(C, info.h_r, info.d, dt, "cpu", pin_memory=device is not None) for _ in range(L)]
    kv = [tuple(torch.empty((C, info.h_kv, info.d), dtype=dt, pin_memory=kvdev is not None) for _ in range(2))
          for _ in range(L)]
    dto = np.empty(info.n_docs + 1, dtype=np.int64)
    cho = np.empty(info.n_docs + 1, dtype=np.int64)
    arr = lambda ts: (ctypes.c_void_p * L)(*[t.data_ptr() for t in ts])
    _check(lib.msa_bank_load(os.fsencode(path), ctypes.byref(info), dto.ctypes.data, cho.ctypes.data,
                             arr([k.data for k in kr]),
                             arr([k for k, _ in kv]), arr([v for _, v in kv])))
    layers = []
    for l in range(L):
        Kr = kr[l].to(device, non_blocking=True) if device is not None else kr[l]
        if kvdev is None or kvdev == "cpu-pinned":
            K, V = kv[l]
        else:
            K, V = kv[l][0].to(kvdev, non_blocking=True), kv[l][1].to(kvdev, non_blocking=True)
        layers.append((Kr, K, V))
    if device is not None or (kvdev is not None and kvdev != "cpu-pinned"):
        torch.cuda.synchronize()
    return dto, cho, layers, _info_dict(info)
