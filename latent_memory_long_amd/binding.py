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
LIB_PATH = os.path.join(_HERE, "libmsa.so")

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
        "msa_pool": (ctypes.c_int, [ctypes.c_int, I32, I64, I64, P, P, I32, I32, I32, I32, F, U32,
                                    P, P, P, P, P, P, P]),
        "msa_route_scan": (ctypes.c_int, [ctypes.c_int, I32, I64, P, I32, P, I32, I32, I32, I64, P,
                                          P, P, P, P, P]),
        "msa_topk_workspace": (SZ, [I32, I32, I32]),
        "msa_topk": (ctypes.c_int, [I32, I32, P, I32, P, P, P, SZ, P]),
        "msa_route_topk_workspace": (SZ, [I32, I32, I32]),
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


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


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
    """Step A.  K, V [T, h_kv, d]; Kr [T, h_r, d]; offsets int64 on the device.
    Returns (Kbar, Vbar, Krbar) [n_chunks, h, d]."""
    T, h_kv, d = K.shape
    h_r = Kr.shape[1]
    if out is None:
        out = (torch.empty((n_chunks, h_kv, d), dtype=K.dtype, device=K.device),
               torch.empty((n_chunks, h_kv, d), dtype=K.dtype, device=K.device),
               torch.empty((n_chunks, h_r, d), dtype=K.dtype, device=K.device))
    Kb, Vb, Krb = out
    _check(lib.msa_pool(_dtype_code(K), doc_tok_off.numel() - 1, T, n_chunks, _ptr(doc_tok_off),
                        _ptr(chunk_off), h_kv, h_r, d, chunk, rope_base, rope_mask, _ptr(K), _ptr(V),
                        _ptr(Kr), _ptr(Kb), _ptr(Vb), _ptr(Krb), _stream(stream)))
    return Kb, Vb, Krb


def msa_route_scan(Qr: torch.Tensor, q_off: torch.Tensor, max_q_len: int, Krbar: torch.Tensor,
                   chunk_off: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
                   rows: Optional[tuple] = None):
    """Step B.  Returns every document's score, float32 [B, N].  For training pass `rows` =
    (float32 [B, C], int32 [B, C]) device tensors to also get each bank row's best token
    score and the first token reaching it, which msa_route_backward can reuse."""
    B = q_off.numel() - 1
    N = chunk_off.numel() - 1
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=Krbar.device)
    _check(lib.msa_route_scan(_dtype_code(Krbar), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr),
                              Krbar.shape[1], Krbar.shape[2], N, Krbar.shape[0], _ptr(chunk_off),
                              _ptr(Krbar), _ptr(out), *_rows(rows, B, Krbar.shape[0]), _stream(stream)))
    return out


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
    B, N = doc_scores.shape
    if out is None:
        out = (torch.empty((B, k), dtype=torch.int32, device=doc_scores.device),
               torch.empty((B, k), dtype=torch.float32, device=doc_scores.device))
    ids, sc = out
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
    """Steps B + C.  Qr [total_q, h_r, d]; q_off int32 [B+1]; Krbar [C, h_r, d].
    Returns (topk_ids int32 [B,k], topk_scores f32 [B,k], doc_scores f32 [B,N] or None)."""
    B = q_off.numel() - 1
    N = chunk_off.numel() - 1
    dev = Krbar.device
    if out is None:
        out = (torch.empty((B, k), dtype=torch.int32, device=dev),
               torch.empty((B, k), dtype=torch.float32, device=dev),
               torch.empty((B, N), dtype=torch.float32, device=dev) if want_doc_scores else None)
    ids, sc, ds = out
    ws, wsb = None, 0
    need = msa_route_topk_workspace(B, N, k) if ds is None else msa_topk_workspace(B, N, k)
    if need:
        ws = _workspace(need, dev, workspace)
        wsb = ws.numel() * ws.element_size()
    _check(lib.msa_route_topk(_dtype_code(Krbar), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr),
                              Krbar.shape[1], Krbar.shape[2], N, Krbar.shape[0], _ptr(chunk_off),
                              _ptr(Krbar), k, _ptr(ids), _ptr(sc), _ptr(ds), _ptr(ws), wsb,
                              _stream(stream)))
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
    B = q_off.numel() - 1
    total_q, hq, d = Q.shape
    total_kv, h_kv, _ = Kloc.shape
    k = topk_ids.shape[1]
    N = chunk_off.numel() - 1
    kv_source = 0 if Kbar.is_cuda else 1
    if kv_source == 1 and not (Kbar.is_pinned() and Vbar.is_pinned()):
        raise MsaError(MSA_ERR_INVALID_ARG, "host-resident Kbar/Vbar must be pinned")
    dev = Q.device
    if out is None:
        out = torch.empty_like(Q)
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
    B = q_off.numel() - 1
    total_q, hq, d = Q.shape
    total_kv, h_kv, _ = Kloc.shape
    k = topk_ids.shape[1]
    N = chunk_off.numel() - 1
    C = Kbar.shape[0]
    kv_source = 0 if Kbar.is_cuda else 1
    if kv_source == 1 and not (Kbar.is_pinned() and Vbar.is_pinned()):
        raise MsaError(MSA_ERR_INVALID_ARG, "host-resident Kbar/Vbar must be pinned")
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
    B = q_off.numel() - 1
    N = chunk_off.numel() - 1
    C, h_r, d = Krbar.shape
    dev = Krbar.device
    if out is None:
        out = torch.empty((Qr.shape[0], h_r, d), dtype=torch.float32, device=dev)
    if dKrbar is None:
        dKrbar = torch.zeros((C, h_r, d), dtype=torch.float32, device=dev)
    need = msa_route_backward_workspace(B, N, C, h_r)
    ws = _workspace(need, dev, workspace)
    _check(lib.msa_route_backward(_dtype_code(Krbar), B, Qr.shape[0], _ptr(q_off), max_q_len, _ptr(Qr), h_r,
                                  d, N, C, _ptr(chunk_off), _ptr(Krbar), _ptr(dD), *_rows(rows, B, C),
                                  _ptr(out), _ptr(dKrbar),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, dKrbar


MSA_AUX_BCE = 0
MSA_AUX_INFONCE = 1


def msa_route_aux_loss(doc_scores: torch.Tensor, labels: torch.Tensor, kind: int = MSA_AUX_BCE,
                       temperature: float = 1.0, out: Optional[tuple] = None, stream=None):
    """Routing auxiliary loss on float32 [B, N] document scores and labels (device).
    Returns (per-query loss [B], dL/dS [B, N]) for L = the mean of the per-query losses."""
    B, N = doc_scores.shape
    if out is None:
        out = (torch.empty(B, dtype=torch.float32, device=doc_scores.device),
               torch.empty((B, N), dtype=torch.float32, device=doc_scores.device))
    loss, dD = out
    _check(lib.msa_route_aux_loss(kind, B, N, _ptr(doc_scores), _ptr(labels), temperature, _ptr(loss),
                                  _ptr(dD), _stream(stream)))
    return loss, dD


def _info_dict(info: BankInfo) -> dict:
    return {f: getattr(info, f) for f, _ in BankInfo._fields_ if f != "reserved"}


def msa_bank_save(path: str, doc_tok_off, chunk_off, layers, chunk: int = 64, rope_base: float = 1e6,
                  rope_mask: int = 1):
    """Writes a bank file.  layers: [(Krbar, Kbar, Vbar), ...] one tuple per routed layer,
    tensors on any device (copied to host memory for the write)."""
    dto = np.ascontiguousarray(doc_tok_off, dtype=np.int64)
    cho = np.ascontiguousarray(chunk_off, dtype=np.int64)
    Kr0, K0, _ = layers[0]
    host = [tuple(t.detach().contiguous().cpu() for t in trio) for trio in layers]
    info = BankInfo(_dtype_code(Kr0), len(layers), len(dto) - 1, K0.shape[1], Kr0.shape[1], Kr0.shape[2], chunk,
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
    int64 arrays, layers as [(Krbar, Kbar, Vbar), ...].  Kr-bar goes to ``device`` and K-bar /
    V-bar to ``kv_device`` (default: ``device``; "cpu-pinned" for page-locked host memory);
    None keeps a tensor in host memory."""
    info = BankInfo()
    _check(lib.msa_bank_read_info(os.fsencode(path), ctypes.byref(info)))
    dt = torch.float32 if info.dtype == MSA_F32 else torch.bfloat16
    C, L = info.n_chunks, info.n_layers
    kvdev = device if kv_device is None else kv_device
    # host buffers are page-locked when they feed a device copy or are asked for as such
    kr = [torch.empty((C, info.h_r, info.d), dtype=dt, pin_memory=device is not None) for _ in range(L)]
    kv = [tuple(torch.empty((C, info.h_kv, info.d), dtype=dt, pin_memory=kvdev is not None) for _ in range(2))
          for _ in range(L)]
    dto = np.empty(info.n_docs + 1, dtype=np.int64)
    cho = np.empty(info.n_docs + 1, dtype=np.int64)
    arr = lambda ts: (ctypes.c_void_p * L)(*[t.data_ptr() for t in ts])
    _check(lib.msa_bank_load(os.fsencode(path), ctypes.byref(info), dto.ctypes.data, cho.ctypes.data, arr(kr),
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
