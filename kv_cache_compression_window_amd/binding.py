"""Thin Python binding of libkvc (ctypes).  Argument marshalling only.

Every function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU.  torch supplies device memory (outputs and
workspaces allocated here when the caller passes none) and the stream (the
current torch stream unless one is given).  No computation happens in Python,
and there is no fallback: when ``libkvc.so`` is missing, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvc.so")

KVC_F32, KVC_BF16 = 0, 1
KVC_REDUCE_GROUP, KVC_REDUCE_ALL_HEADS = 0, 1
KVC_ERR_WORKSPACE = 5
KVC_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/kvc.h

STATUS_NAMES = {0: "KVC_OK", 1: "KVC_ERR_NULL", 2: "KVC_ERR_SHAPE", 3: "KVC_ERR_DTYPE", 4: "KVC_ERR_ALIGN",
                5: "KVC_ERR_WORKSPACE", 6: "KVC_ERR_UNSUPPORTED", 7: "KVC_ERR_HIP"}

# every symbol include/kvc.h declares
EXPORTS = ["kvc_window_scores", "kvc_window_scores_ex", "kvc_scissor_update", "kvc_channel_scores", "kvc_topk_select",
           "kvc_gather_compact", "kvc_gather_compress", "kvc_channel_expand", "kvc_query_channels",
           "kvc_scissor_refill", "kvc_scissor_insert", "kvc_window_scores_noalloc", "kvc_status_string",
           "kvc_abi_version"]


class KvcShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("S", ctypes.c_int32),
                ("D", ctypes.c_int32), ("w", ctypes.c_int32)]


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m kv_cache_compression_window_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)
    SH = ctypes.POINTER(KvcShape)
    sig = {
        "kvc_window_scores": [SH, I32, P, P, P, P, I32, I32, I32, P, P, SZP, P],
        "kvc_window_scores_ex": [SH, I32, P, P, P, P, I32, I32, I32, I32, P, P, SZP, P],
        "kvc_window_scores_noalloc": [SH, I32, P, P, P, P, I32, I32, I32, P, P],
        "kvc_scissor_update": [I32, I32, I32, I32, I64, P, P, P, P, P, P, P, I32, P],
        "kvc_channel_scores": [SH, I32, P, P, P, P, SZP, P],
        "kvc_topk_select": [P, I32, I32, I32, I32, P, P, SZP, P],
        "kvc_gather_compact": [SH, I32, P, P, P, I32, P, I32, P, P, P],
        "kvc_gather_compress": [SH, I32, P, P, P, I32, P, I32, P, P, P],
        "kvc_channel_expand": [I32, I32, I32, I32, I32, P, P, I32, P, P],
        "kvc_query_channels": [I32, I32, I32, I32, I32, I32, P, P, I32, P, P],
        "kvc_scissor_refill": [I32, I32, I32, I32, I64, P, P, P, I32, I32, P, P, SZP, P],
        "kvc_scissor_insert": [I32, I32, I32, I32, I32, I32, P, I32, I32, I32, I64, P, P, P, P, P, P, P, P, P],
        "kvc_status_string": [I32],
        "kvc_abi_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_char_p if name == "kvc_status_string" else ctypes.c_int32
    return lib


LIB = _load()


def abi_version() -> int:
    return LIB.kvc_abi_version()


def _check(fn: str, status: int):
    if status != 0:
        raise KvcError(fn, status, LIB.kvc_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dim: int):
    if t.dim() != dim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dim}-d CUDA tensor, got {tuple(t.shape)}")


def _shape(q: torch.Tensor, k: torch.Tensor) -> KvcShape:
    B, H, w, D = q.shape
    _, Hkv, S, _ = k.shape
    return KvcShape(B, H, Hkv, S, D, w)


def _workspace(nbytes: int, device, ws):
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _ws_call(cu_budget, sh, dt, q, k, valid, chan, d_keep, reduce, causal, scores, ws, n, stream):
    """kvc_window_scores, or kvc_window_scores_ex when a compute-unit budget is given."""
    if cu_budget in (None, 0):
        return "kvc_window_scores", (sh, dt, q, k, valid, chan, d_keep, reduce, causal, scores, ws, n, stream)
    return "kvc_window_scores_ex", (sh, dt, q, k, valid, chan, d_keep, reduce, causal, int(cu_budget),
                                    scores, ws, n, stream)


def window_scores_ws_bytes(B, H, Hkv, S, D, w, dtype=None, cu_budget=None) -> int:
    sh = KvcShape(B, H, Hkv, S, D, w)
    n = ctypes.c_size_t(0)
    dt = KVC_BF16 if dtype is None else dtype
    name, args = _ws_call(cu_budget, ctypes.byref(sh), dt, None, None, None, None, 0, 0, 0, None, None,
                          ctypes.byref(n), None)
    _check(name, getattr(LIB, name)(*args))
    return n.value


def kvc_window_scores(q, k, valid=None, chan_idx=None, reduce=KVC_REDUCE_GROUP, causal=True, scores=None, ws=None,
                      stream=None, cu_budget=None):
    """scores [B,Hkv,S] float32 of the window rows q [B,H,w,D] against k [B,Hkv,S,D]
    (kvc_window_scores_ex when cu_budget is given and not 0)."""
    _need(q, "q_win", 4)
    _need(k, "k", 4)
    sh = _shape(q, k)
    if valid is not None:
        _need(valid, "valid", 3)
        assert valid.dtype == torch.uint8
    d_keep = 0
    if chan_idx is not None:
        _need(chan_idx, "chan_idx", 3)
        assert chan_idx.dtype == torch.int32
        d_keep = chan_idx.shape[2]
    if scores is None:
        scores = torch.empty((sh.B, sh.Hkv, sh.S), dtype=torch.float32, device=k.device)
    n = ctypes.c_size_t(0)
    name, args = _ws_call(cu_budget, ctypes.byref(sh), _dtype_code(k), None, None, None, None, d_keep, reduce,
                          int(causal), None, None, ctypes.byref(n), None)
    _check(name, getattr(LIB, name)(*args))
    ws = _workspace(n.value, k.device, ws)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    name, args = _ws_call(cu_budget, ctypes.byref(sh), _dtype_code(k), _ptr(q), _ptr(k), _ptr(valid),
                          _ptr(chan_idx), d_keep, reduce, int(causal), _ptr(scores), _ptr(ws), ctypes.byref(n),
                          _stream(stream))
    _check(name, getattr(LIB, name)(*args))
    return scores


def kvc_window_scores_noalloc(q, k, scores, valid=None, chan_idx=None, reduce=KVC_REDUCE_GROUP, causal=True,
                              stream=None):
    """kvc_window_scores into the caller's scores [B,Hkv,S] float32, with the
    library's fixed per-GPU scratch instead of a workspace (nothing allocated)."""
    _need(q, "q_win", 4)
    _need(k, "k", 4)
    _need(scores, "scores", 3)
    sh = _shape(q, k)
    d_keep = 0
    if chan_idx is not None:
        _need(chan_idx, "chan_idx", 3)
        d_keep = chan_idx.shape[2]
    _check("kvc_window_scores_noalloc",
           LIB.kvc_window_scores_noalloc(ctypes.byref(sh), _dtype_code(k), _ptr(q), _ptr(k), _ptr(valid),
                                         _ptr(chan_idx), d_keep, reduce, int(causal), _ptr(scores), _stream(stream)))
    return scores


def kvc_scissor_update(step, valid, hist, counts, probs=None, frac_out=None, evict_idx=None, since=None,
                       stream=None):
    """Record recording number `step` (probs given), write the fraction (frac_out
    given) and/or evict (evict_idx given).  valid [B,Hkv,C] uint8, hist
    [hist_len, B*Hkv, ceil(C/32)] int32 bit-planes, counts [B,Hkv,C] int16 (read as
    uint16), since [B,Hkv,C] int64 or None (every slot observed from the start)."""
    _need(valid, "valid", 3)
    B, Hkv, C = valid.shape
    hist_len = hist.shape[0]
    n_evict = 0 if evict_idx is None else evict_idx.shape[2]
    _check("kvc_scissor_update", LIB.kvc_scissor_update(B, Hkv, C, hist_len, int(step), _ptr(probs), _ptr(valid),
                                                        _ptr(hist), _ptr(counts), _ptr(since), _ptr(frac_out),
                                                        _ptr(evict_idx), n_evict, _stream(stream)))


def scissor_refill_ws_bytes(B, Hkv, C) -> int:
    n = ctypes.c_size_t(0)
    _check("kvc_scissor_refill", LIB.kvc_scissor_refill(B, Hkv, C, 1, 0, None, None, None, 0, 1, None, None,
                                                        ctypes.byref(n), None))
    return n.value


def kvc_scissor_refill(step, valid, counts, hist_len, n_protect, m, queue=None, ws=None, since=None, stream=None):
    """queue [B,Hkv,m] int32: the m slots of the largest low-attention fraction
    (counts over each slot's own observations, min(step+1-since, hist_len)), never a
    hole or one of the first n_protect."""
    _need(valid, "valid", 3)
    B, Hkv, C = valid.shape
    if queue is None:
        queue = torch.empty((B, Hkv, m), dtype=torch.int32, device=valid.device)
    ws = _workspace(scissor_refill_ws_bytes(B, Hkv, C), valid.device, ws)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("kvc_scissor_refill", LIB.kvc_scissor_refill(B, Hkv, C, hist_len, int(step), _ptr(valid), _ptr(counts),
                                                        _ptr(since), n_protect, m, _ptr(queue), _ptr(ws),
                                                        ctypes.byref(n), _stream(stream)))
    return queue


def kvc_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, rec, queue=None, j=0,
                       fill_pos=0, stream=None):
    """The new token k_new/v_new [B,Hkv,D] into slot queue[:,:,j] (or fill_pos) of
    k_cache/v_cache [B,Hkv,C,D]; the slot becomes valid with no observation
    (since [B,Hkv,C] int64 <- rec, the recordings made before it)."""
    _need(k_cache, "k_cache", 4)
    B, Hkv, C, D = k_cache.shape
    m = 0 if queue is None else queue.shape[2]
    _check("kvc_scissor_insert", LIB.kvc_scissor_insert(B, Hkv, C, D, hist.shape[0], _dtype_code(k_cache),
                                                        _ptr(queue), m, j, fill_pos, int(rec), _ptr(k_new),
                                                        _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(valid),
                                                        _ptr(hist), _ptr(counts), _ptr(since), _stream(stream)))


def channel_scores_ws_bytes(B, H, Hkv, S, D, w) -> int:
    sh = KvcShape(B, H, Hkv, S, D, w)
    n = ctypes.c_size_t(0)
    _check("kvc_channel_scores", LIB.kvc_channel_scores(ctypes.byref(sh), KVC_BF16, None, None, None, None,
                                                        ctypes.byref(n), None))
    return n.value


def kvc_channel_scores(q, k, out=None, ws=None, stream=None):
    """ThinK channel scores [B,Hkv,D] float32."""
    _need(q, "q_win", 4)
    _need(k, "k", 4)
    sh = _shape(q, k)
    if out is None:
        out = torch.empty((sh.B, sh.Hkv, sh.D), dtype=torch.float32, device=k.device)
    n = ctypes.c_size_t(0)
    _check("kvc_channel_scores", LIB.kvc_channel_scores(ctypes.byref(sh), _dtype_code(k), None, None, None, None,
                                                        ctypes.byref(n), None))
    ws = _workspace(n.value, k.device, ws)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("kvc_channel_scores", LIB.kvc_channel_scores(ctypes.byref(sh), _dtype_code(k), _ptr(q), _ptr(k), _ptr(out),
                                                        _ptr(ws), ctypes.byref(n), _stream(stream)))
    return out


def topk_ws_bytes(rows, n) -> int:
    """Workspace bytes kvc_topk_select needs for rows of n scores."""
    nb = ctypes.c_size_t(0)
    _check("kvc_topk_select", LIB.kvc_topk_select(None, rows, n, 0, 0, None, None, ctypes.byref(nb), None))
    return nb.value


def kvc_topk_select(scores, k, n_tail=0, idx=None, ws=None, stream=None):
    """idx [..., k] int32 (ascending) of each row of scores [..., n]."""
    if not scores.is_contiguous() or scores.dtype != torch.float32 or not scores.is_cuda:
        raise ValueError("scores must be a contiguous float32 CUDA tensor")
    n = scores.shape[-1]
    rows = scores.numel() // n
    if idx is None:
        idx = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    nb = ctypes.c_size_t(0)
    _check("kvc_topk_select", LIB.kvc_topk_select(None, rows, n, k, n_tail, None, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, scores.device, ws)
    nb = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("kvc_topk_select", LIB.kvc_topk_select(_ptr(scores), rows, n, k, n_tail, _ptr(idx), _ptr(ws),
                                                  ctypes.byref(nb), _stream(stream)))
    return idx


def kvc_gather_compact(k, v, idx, chan_idx=None, k_out=None, v_out=None, stream=None):
    """Compacted (k_out, v_out) [B,Hkv,n_keep,D] of the rows idx [B,Hkv,n_keep]."""
    _need(k, "k", 4)
    B, Hkv, S, D = k.shape
    n_keep = idx.shape[2]
    sh = KvcShape(B, Hkv, Hkv, S, D, 1)
    d_keep = 0 if chan_idx is None else chan_idx.shape[2]
    if k_out is None:
        k_out = torch.empty((B, Hkv, n_keep, D), dtype=k.dtype, device=k.device)
    if v is not None and v_out is None:
        v_out = torch.empty((B, Hkv, n_keep, D), dtype=v.dtype, device=v.device)
    _check("kvc_gather_compact", LIB.kvc_gather_compact(ctypes.byref(sh), _dtype_code(k), _ptr(k), _ptr(v), _ptr(idx),
                                                        n_keep, _ptr(chan_idx), d_keep, _ptr(k_out), _ptr(v_out),
                                                        _stream(stream)))
    return k_out, v_out


def kvc_gather_compress(k, v, idx, chan_idx, k_out=None, v_out=None, stream=None):
    """k_out [B,Hkv,n_keep,d_keep] (kept rows, kept key channels) and v_out
    [B,Hkv,n_keep,D] (kept rows) of the rows idx [B,Hkv,n_keep]."""
    _need(k, "k", 4)
    _need(chan_idx, "chan_idx", 3)
    B, Hkv, S, D = k.shape
    n_keep, d_keep = idx.shape[2], chan_idx.shape[2]
    sh = KvcShape(B, Hkv, Hkv, S, D, 1)
    if k_out is None:
        k_out = torch.empty((B, Hkv, n_keep, d_keep), dtype=k.dtype, device=k.device)
    if v is not None and v_out is None:
        v_out = torch.empty((B, Hkv, n_keep, D), dtype=v.dtype, device=v.device)
    _check("kvc_gather_compress", LIB.kvc_gather_compress(ctypes.byref(sh), _dtype_code(k), _ptr(k), _ptr(v),
                                                          _ptr(idx), n_keep, _ptr(chan_idx), d_keep, _ptr(k_out),
                                                          _ptr(v_out), _stream(stream)))
    return k_out, v_out


def kvc_channel_expand(k_c, chan_idx, D, k_full=None, stream=None):
    """k_full [B,Hkv,n,D]: the compressed keys k_c [B,Hkv,n,d_keep] with zeros added back."""
    _need(k_c, "k_c", 4)
    _need(chan_idx, "chan_idx", 3)
    B, Hkv, n, d_keep = k_c.shape
    if k_full is None:
        k_full = torch.empty((B, Hkv, n, D), dtype=k_c.dtype, device=k_c.device)
    _check("kvc_channel_expand", LIB.kvc_channel_expand(B, Hkv, n, D, _dtype_code(k_c), _ptr(k_c), _ptr(chan_idx),
                                                        d_keep, _ptr(k_full), _stream(stream)))
    return k_full


def kvc_query_channels(q, chan_idx, q_c=None, stream=None):
    """q_c [B,H,n,d_keep]: each query head's rows q [B,H,n,D] cut to its KV head's kept channels."""
    _need(q, "q", 4)
    _need(chan_idx, "chan_idx", 3)
    B, H, n, D = q.shape
    Hkv, d_keep = chan_idx.shape[1], chan_idx.shape[2]
    if q_c is None:
        q_c = torch.empty((B, H, n, d_keep), dtype=q.dtype, device=q.device)
    _check("kvc_query_channels", LIB.kvc_query_channels(B, H, Hkv, n, D, _dtype_code(q), _ptr(q), _ptr(chan_idx),
                                                        d_keep, _ptr(q_c), _stream(stream)))
    return q_c


# ----------------------------------------------------------------------------
# Pre-bound calls: marshal the arguments once and return a function that makes
# the C call with them (one foreign call per use).  For loops that launch the
# same call on the same buffers many times.
# ----------------------------------------------------------------------------

def _bound(fn_name, args):
    f = getattr(LIB, fn_name)

    def call():
        st = f(*args)
        if st != 0:
            _check(fn_name, st)

    return call


def bind_window_scores(q, k, scores, ws, stream, valid=None, chan_idx=None, reduce=KVC_REDUCE_GROUP, causal=True,
                       cu_budget=None):
    _need(q, "q_win", 4)
    _need(k, "k", 4)
    sh = _shape(q, k)
    d_keep = 0 if chan_idx is None else chan_idx.shape[2]
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    name, args = _ws_call(cu_budget, ctypes.byref(sh), _dtype_code(k), _ptr(q), _ptr(k), _ptr(valid),
                          _ptr(chan_idx), d_keep, reduce, int(causal), _ptr(scores), _ptr(ws), ctypes.byref(n),
                          ctypes.c_void_p(stream.cuda_stream))
    call = _bound(name, args)
    call.keep_alive = (sh, n, q, k, valid, chan_idx, scores, ws)
    return call


def bind_topk_select(scores, k, n_tail, idx, ws, stream):
    n = scores.shape[-1]
    rows = scores.numel() // n
    nb = ctypes.c_size_t(ws.numel() * ws.element_size())
    args = (_ptr(scores), rows, n, k, n_tail, _ptr(idx), _ptr(ws), ctypes.byref(nb),
            ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_topk_select", args)
    call.keep_alive = (nb, scores, idx, ws)
    return call


def bind_gather_compact(k, v, idx, k_out, v_out, stream, chan_idx=None):
    B, Hkv, S, D = k.shape
    sh = KvcShape(B, Hkv, Hkv, S, D, 1)
    d_keep = 0 if chan_idx is None else chan_idx.shape[2]
    args = (ctypes.byref(sh), _dtype_code(k), _ptr(k), _ptr(v), _ptr(idx), idx.shape[2], _ptr(chan_idx), d_keep,
            _ptr(k_out), _ptr(v_out), ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_gather_compact", args)
    call.keep_alive = (sh, k, v, idx, chan_idx, k_out, v_out)
    return call


def bind_gather_compress(k, v, idx, chan_idx, k_out, v_out, stream):
    B, Hkv, S, D = k.shape
    sh = KvcShape(B, Hkv, Hkv, S, D, 1)
    args = (ctypes.byref(sh), _dtype_code(k), _ptr(k), _ptr(v), _ptr(idx), idx.shape[2], _ptr(chan_idx),
            chan_idx.shape[2], _ptr(k_out), _ptr(v_out), ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_gather_compress", args)
    call.keep_alive = (sh, k, v, idx, chan_idx, k_out, v_out)
    return call


def bind_query_channels(q, chan_idx, q_c, stream):
    B, H, n, D = q.shape
    args = (B, H, chan_idx.shape[1], n, D, _dtype_code(q), _ptr(q), _ptr(chan_idx), chan_idx.shape[2], _ptr(q_c),
            ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_query_channels", args)
    call.keep_alive = (q, chan_idx, q_c)
    return call


def bind_scissor_update(valid, hist, counts, stream, probs=None, frac_out=None, evict_idx=None, since=None):
    """Pre-bound kvc_scissor_update; returns (call, step) with step a ctypes.c_int64
    whose value the caller sets before each call."""
    B, Hkv, C = valid.shape
    step = ctypes.c_int64(0)
    n_evict = 0 if evict_idx is None else evict_idx.shape[2]
    args = (B, Hkv, C, hist.shape[0], step, _ptr(probs), _ptr(valid), _ptr(hist), _ptr(counts), _ptr(since),
            _ptr(frac_out), _ptr(evict_idx), n_evict, ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_scissor_update", args)
    call.keep_alive = (valid, hist, counts, probs, frac_out, evict_idx, since, step)
    return call, step


def bind_scissor_refill(valid, counts, since, hist_len, n_protect, queue, ws, stream):
    """Pre-bound kvc_scissor_refill; returns (call, step)."""
    B, Hkv, C = valid.shape
    step = ctypes.c_int64(0)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    args = (B, Hkv, C, hist_len, step, _ptr(valid), _ptr(counts), _ptr(since), n_protect, queue.shape[2],
            _ptr(queue), _ptr(ws), ctypes.byref(n), ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_scissor_refill", args)
    call.keep_alive = (valid, counts, since, queue, ws, step, n)
    return call, step


def bind_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, stream, queue=None):
    """Pre-bound kvc_scissor_insert; returns (call, j, fill_pos, rec), ctypes values
    the caller sets before each call (rec: the recordings made before the token)."""
    B, Hkv, C, D = k_cache.shape
    j, fill_pos, rec = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    m = 0 if queue is None else queue.shape[2]
    args = (B, Hkv, C, D, hist.shape[0], _dtype_code(k_cache), _ptr(queue), m, j, fill_pos, rec, _ptr(k_new),
            _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(valid), _ptr(hist), _ptr(counts), _ptr(since),
            ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_scissor_insert", args)
    call.keep_alive = (k_new, v_new, k_cache, v_cache, valid, hist, counts, since, queue, j, fill_pos, rec)
    return call, j, fill_pos, rec


def bind_channel_scores(q, k, out, ws, stream):
    _need(q, "q_win", 4)
    _need(k, "k", 4)
    sh = _shape(q, k)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    args = (ctypes.byref(sh), _dtype_code(k), _ptr(q), _ptr(k), _ptr(out), _ptr(ws), ctypes.byref(n),
            ctypes.c_void_p(stream.cuda_stream))
    call = _bound("kvc_channel_scores", args)
    call.keep_alive = (sh, n, q, k, out, ws)
    return call
