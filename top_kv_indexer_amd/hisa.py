"""Python binding of libhisa.so (ctypes).  Argument marshalling only: shapes are
read off the torch tensors, outputs and the workspace are allocated with torch
on the tensors' device, and every computation runs in the HIP kernels on the
current torch stream.  The names follow the C ABI in include/hisa.h.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhisa.so")

F32, BF16 = 0, 1
MODE_AUTO, MODE_FORCE_FLAT, MODE_FORCE_DENSE = 0, 1, 2
PATH_INVALID, PATH_DENSE, PATH_FLAT, PATH_HISA = -1, 0, 1, 2
(OP_BLOCK_SCORES, OP_SELECT_DECODE, OP_SELECT_PREFILL, OP_FLAT_TOPK, OP_ATTENTION, OP_SELECT_DECODE_CACHED,
 OP_BLOCK_MEANS_UPDATE, OP_DECODE_STEP) = range(8)

EXPORTS = ("hisa_block_scores", "hisa_select_decode", "hisa_select_decode_noalloc", "hisa_select_decode_cached",
           "hisa_block_means_update", "hisa_select_prefill", "flat_topk_select",
           "sparse_local_pooled_attention", "sparse_local_pooled_attention_ring", "hisa_decode_step",
           "hisa_workspace_bytes",
           "hisa_last_error", "hisa_abi_version",
           "hisa_profile_enable", "hisa_profile_collect")


class HisaError(RuntimeError):
    pass


class hisa_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class hisa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "L", "ratio", "window", "topk", "index_block", "index_keep", "H_i", "D_i", "H", "Dk", "Dv",
        "Np_cap", "Wl_cap", "kI", "mode", "idx_dtype", "attn_dtype")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HisaError(f"{LIB_PATH} is missing: build it with top_kv_indexer_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        dp = ctypes.POINTER(hisa_dims)
        sel = [dp, vp, vp, vp, vp]
        L.hisa_block_scores.argtypes = sel + [vp, vp, vp, sz, vp]
        L.hisa_select_decode.argtypes = sel + [vp, vp, vp, vp, sz, vp]
        L.hisa_select_decode_noalloc.argtypes = sel + [vp, vp, vp, vp]
        L.hisa_select_decode_cached.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hisa_block_means_update.argtypes = [dp, vp, vp, vp, vp]
        L.hisa_select_prefill.argtypes = sel + [vp, vp, vp, vp, sz, vp]
        L.flat_topk_select.argtypes = sel + [vp, vp, sz, vp]
        L.sparse_local_pooled_attention.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sparse_local_pooled_attention_ring.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hisa_decode_step.argtypes = [dp] + [vp] * 13 + [sz, vp]
        for f in ("hisa_block_scores", "hisa_select_decode", "hisa_select_decode_noalloc", "hisa_select_decode_cached",
                  "hisa_block_means_update", "hisa_select_prefill", "flat_topk_select",
                  "sparse_local_pooled_attention", "sparse_local_pooled_attention_ring", "hisa_decode_step"):
            getattr(L, f).restype = i32
        L.hisa_workspace_bytes.argtypes = [i32, dp]
        L.hisa_workspace_bytes.restype = sz
        L.hisa_last_error.restype = ctypes.c_char_p
        L.hisa_abi_version.restype = i32
        L.hisa_profile_enable.argtypes = [i32]
        L.hisa_profile_enable.restype = i32
        L.hisa_profile_collect.argtypes = [ctypes.POINTER(hisa_kernel_time), i32]
        L.hisa_profile_collect.restype = i32
        _lib = L
    return _lib


def last_error() -> str:
    return lib().hisa_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise HisaError(f"libhisa error {rc}: {last_error()}")


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise HisaError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, ndim: int, dtype=None, shape=None) -> torch.Tensor:
    """Checks one tensor argument; shape entries that are None are free."""
    if not isinstance(t, torch.Tensor):
        raise HisaError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != ndim:
        raise HisaError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise HisaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        for ax, (have, want) in enumerate(zip(t.shape, shape)):
            if want is not None and have != want:
                raise HisaError(f"{name} has shape {tuple(t.shape)}; dim {ax} must be {want}")
    if not t.is_contiguous():
        raise HisaError(f"{name} must be contiguous")
    return t


def _same_gpu(**tensors) -> torch.device:
    """Every given tensor on one GPU (checked after the shapes, so shape errors
    show on any device); returns that device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise HisaError(f"{name} must be on a GPU, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise HisaError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_bytes(op: int, d: hisa_dims) -> int:
    n = lib().hisa_workspace_bytes(op, ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise HisaError(last_error())
    return int(n)


# One workspace per (device, stream, op), grown on demand and reused by every
# call of that op on that stream (calls on one stream are ordered, so they
# never overlap).  The decode selection's arrival counters start zeroed and
# every call leaves them zero; their region grows with B and Np_cap (and the
# decode step's also with H, topk, index_block and index_keep), so those
# workspaces are kept per such dims as well.
_ws_cache = {}


def _workspace(op: int, d: hisa_dims, dev: torch.device, ws: Optional[torch.Tensor]):
    n = workspace_bytes(op, d)
    if ws is not None:
        if ws.numel() < n:
            raise HisaError(f"workspace of {ws.numel()} bytes < {n} needed")
        return ws, ws.numel()
    if n == 0:
        return None, 0
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream, op)
    if op in (OP_SELECT_DECODE, OP_SELECT_DECODE_CACHED):
        key += (d.B, d.Np_cap)
    elif op == OP_DECODE_STEP:
        key += (d.B, d.Np_cap, d.H, d.topk, d.index_block, d.index_keep)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < n:
        buf = torch.zeros(n, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf, buf.numel()


def selection_dims(q_idx, keys, *, ratio, topk, index_block, index_keep, mode=MODE_AUTO) -> hisa_dims:
    B, L, H_i, D_i = q_idx.shape
    return hisa_dims(B=B, L=L, ratio=ratio, window=0, topk=topk, index_block=index_block, index_keep=index_keep,
                     H_i=H_i, D_i=D_i, H=1, Dk=1, Dv=1, Np_cap=keys.shape[1], Wl_cap=0, kI=0, mode=mode,
                     idx_dtype=_code(keys), attn_dtype=F32)


def _ws_arg(ws):
    if ws is not None:
        _need(ws, "ws", 1, torch.uint8)
    return ws


def _sel_args(q_idx, w, keys, t0):
    _need(q_idx, "q_idx", 4)
    _code(q_idx)
    B, L, H_i, D_i = q_idx.shape
    _need(w, "w", 3, torch.float32, (B, L, H_i))
    _need(keys, "keys", 3, q_idx.dtype, (B, None, D_i))
    _need(t0, "t0", 1, torch.int32, (B,))
    return B, L


def hisa_block_scores(q_idx, w, keys, t0, *, ratio, index_block, want_rep=False, ws=None):
    """Coarse stage: returns cscore (B, L, nb_cap) and rep (B, nb_cap, D_i) or None."""
    B, L = _sel_args(q_idx, w, keys, t0)
    dev = _same_gpu(q_idx=q_idx, w=w, keys=keys, t0=t0, ws=_ws_arg(ws))
    d = selection_dims(q_idx, keys, ratio=ratio, topk=1, index_block=index_block, index_keep=1)
    nb_cap = keys.shape[1] // max(index_block, 1)
    cs = torch.empty((B, L, nb_cap), dtype=torch.float32, device=dev)
    rep = torch.empty((B, nb_cap, q_idx.shape[3]), dtype=torch.float32, device=dev) if want_rep else None
    wsb, n = _workspace(OP_BLOCK_SCORES, d, dev, ws)
    _check(lib().hisa_block_scores(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(t0), _p(cs), _p(rep), _p(wsb), n,
                                   _stream(dev)))
    return cs, rep


def _select(fn, op, q_idx, w, keys, t0, ratio, topk, index_block, index_keep, mode, I, top_blk, path, ws):
    B, L = _sel_args(q_idx, w, keys, t0)
    if I is not None:
        _need(I, "I", 3, torch.int32, (B, L, topk))
    if top_blk is not None:
        _need(top_blk, "top_blk", 3, torch.int32, (B, L, index_keep))
    if path is not None:
        _need(path, "path", 1, torch.int32, (B,))
    dev = _same_gpu(q_idx=q_idx, w=w, keys=keys, t0=t0, I=I, top_blk=top_blk, path=path, ws=_ws_arg(ws))
    d = selection_dims(q_idx, keys, ratio=ratio, topk=topk, index_block=index_block, index_keep=index_keep,
                       mode=mode)
    if I is None:
        I = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
    if top_blk is None:
        top_blk = torch.empty((B, L, index_keep), dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B,), dtype=torch.int32, device=dev)
    wsb, n = _workspace(op, d, dev, ws)
    _check(fn(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(t0), _p(I), _p(top_blk), _p(path), _p(wsb), n,
              _stream(dev)))
    return I, top_blk, path


def hisa_select_decode(q_idx, w, keys, t0, *, ratio, topk, index_block=64, index_keep=16, mode=MODE_AUTO,
                       I=None, top_blk=None, path=None, ws=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Single-token selection; returns I (B,1,topk), top_blk (B,1,index_keep), path (B).
    A caller-given ws must start with zeroed arrival counters (see include/hisa.h)."""
    return _select(lib().hisa_select_decode, OP_SELECT_DECODE, q_idx, w, keys, t0, ratio, topk, index_block,
                   index_keep, mode, I, top_blk, path, ws)


def _rep_arg(rep, keys, index_block):
    B, Np_cap, D_i = keys.shape
    return _need(rep, "rep", 3, torch.float32, (B, Np_cap // max(index_block, 1), D_i))


def hisa_select_decode_cached(q_idx, w, keys, rep, t0, *, ratio, topk, index_block=64, index_keep=16,
                              mode=MODE_AUTO, I=None, top_blk=None, path=None, ws=None):
    """Decode selection on the block-mean cache rep (B, Np_cap // index_block, D_i) f32, which it keeps
    current (see include/hisa.h); returns I (B,1,topk), top_blk (B,1,index_keep), path (B)."""
    B, L = _sel_args(q_idx, w, keys, t0)
    _rep_arg(rep, keys, index_block)
    if I is not None:
        _need(I, "I", 3, torch.int32, (B, L, topk))
    if top_blk is not None:
        _need(top_blk, "top_blk", 3, torch.int32, (B, L, index_keep))
    if path is not None:
        _need(path, "path", 1, torch.int32, (B,))
    dev = _same_gpu(q_idx=q_idx, w=w, keys=keys, rep=rep, t0=t0, I=I, top_blk=top_blk, path=path, ws=_ws_arg(ws))
    d = selection_dims(q_idx, keys, ratio=ratio, topk=topk, index_block=index_block, index_keep=index_keep,
                       mode=mode)
    if I is None:
        I = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
    if top_blk is None:
        top_blk = torch.empty((B, L, index_keep), dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B,), dtype=torch.int32, device=dev)
    wsb, n = _workspace(OP_SELECT_DECODE_CACHED, d, dev, ws)
    _check(lib().hisa_select_decode_cached(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(rep), _p(t0), _p(I),
                                           _p(top_blk), _p(path), _p(wsb), n, _stream(dev)))
    return I, top_blk, path


def hisa_block_means_update(keys, t0, rep, *, ratio, index_block, L) -> None:
    """Writes into rep the means of the blocks that the step's L tokens (from position t0) complete."""
    _need(keys, "keys", 3)
    _code(keys)
    B, Np_cap, D_i = keys.shape
    _need(t0, "t0", 1, torch.int32, (B,))
    _rep_arg(rep, keys, index_block)
    dev = _same_gpu(keys=keys, t0=t0, rep=rep)
    d = hisa_dims(B=B, L=L, ratio=ratio, window=0, topk=1, index_block=index_block, index_keep=1, H_i=1, D_i=D_i,
                  H=1, Dk=1, Dv=1, Np_cap=Np_cap, Wl_cap=0, kI=0, mode=MODE_AUTO, idx_dtype=_code(keys),
                  attn_dtype=F32)
    _check(lib().hisa_block_means_update(ctypes.byref(d), _p(keys), _p(t0), _p(rep), _stream(dev)))


NOALLOC_MAX_BYTES = 16 << 20  # HISA_DECODE_NOALLOC_MAX_BYTES


def hisa_select_decode_noalloc(q_idx, w, keys, t0, I, top_blk, path, *, ratio, topk, index_block=64, index_keep=16,
                               mode=MODE_AUTO) -> None:
    """hisa_select_decode with the library's own per-GPU workspace: the caller
    passes preallocated outputs I (B,1,topk), top_blk (B,1,index_keep) or None,
    path (B) or None; nothing is allocated."""
    B, L = _sel_args(q_idx, w, keys, t0)
    _need(I, "I", 3, torch.int32, (B, L, topk))
    if top_blk is not None:
        _need(top_blk, "top_blk", 3, torch.int32, (B, L, index_keep))
    if path is not None:
        _need(path, "path", 1, torch.int32, (B,))
    dev = _same_gpu(q_idx=q_idx, w=w, keys=keys, t0=t0, I=I, top_blk=top_blk, path=path)
    d = selection_dims(q_idx, keys, ratio=ratio, topk=topk, index_block=index_block, index_keep=index_keep,
                       mode=mode)
    _check(lib().hisa_select_decode_noalloc(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(t0), _p(I), _p(top_blk),
                                            _p(path), _stream(dev)))


def hisa_select_prefill(q_idx, w, keys, t0, *, ratio, topk, index_block=64, index_keep=16, mode=MODE_AUTO,
                        I=None, top_blk=None, path=None, ws=None):
    """Multi-row selection; returns I (B,L,topk), top_blk (B,L,index_keep), path (B)."""
    return _select(lib().hisa_select_prefill, OP_SELECT_PREFILL, q_idx, w, keys, t0, ratio, topk, index_block,
                   index_keep, mode, I, top_blk, path, ws)


def flat_topk_select(q_idx, w, keys, t0, *, ratio, topk, I=None, ws=None) -> torch.Tensor:
    """Flat top-k indexer; returns I (B, L, topk)."""
    B, L = _sel_args(q_idx, w, keys, t0)
    if I is not None:
        _need(I, "I", 3, torch.int32, (B, L, topk))
    dev = _same_gpu(q_idx=q_idx, w=w, keys=keys, t0=t0, I=I, ws=_ws_arg(ws))
    d = selection_dims(q_idx, keys, ratio=ratio, topk=topk, index_block=0, index_keep=1)
    if I is None:
        I = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
    wsb, n = _workspace(OP_FLAT_TOPK, d, dev, ws)
    _check(lib().flat_topk_select(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(t0), _p(I), _p(wsb), n,
                                  _stream(dev)))
    return I


def attention_dims(q, local_kv, pooled_kv, I, *, ratio, window, Dv=None) -> hisa_dims:
    """I None: dense over every visible pooled row (kI = Np_cap)."""
    B, L, H, Dk = q.shape
    return hisa_dims(B=B, L=L, ratio=ratio, window=window, topk=1, index_block=0, index_keep=1, H_i=1, D_i=1,
                     H=H, Dk=Dk, Dv=Dk if Dv is None else Dv, Np_cap=pooled_kv.shape[1],
                     Wl_cap=0 if local_kv is None else local_kv.shape[1],
                     kI=pooled_kv.shape[1] if I is None else I.shape[2], mode=MODE_AUTO,
                     idx_dtype=F32, attn_dtype=_code(q))


def _attn_args(q, local_kv, pooled_kv, I, sinks, t0, window, Dv, out, ws):
    _need(q, "q", 4)
    _code(q)
    B, L, H, Dk = q.shape
    Dv = Dk if Dv is None else Dv
    _need(pooled_kv, "pooled_kv", 3, q.dtype, (B, None, Dk))
    if local_kv is not None:
        _need(local_kv, "local_kv", 3, q.dtype, (B, None, Dk))
    elif window > 0:
        raise HisaError("local_kv is None but window > 0")
    if I is not None:
        _need(I, "I", 3, torch.int32, (B, L, None))
    _need(t0, "t0", 1, torch.int32, (B,))
    if sinks is not None:
        _need(sinks, "sinks", 1, torch.float32, (H,))
    if out is not None:
        _need(out, "out", 4, q.dtype, (B, L, H, Dv))
    return _same_gpu(q=q, local_kv=local_kv, pooled_kv=pooled_kv, I=I, sinks=sinks, t0=t0, out=out, ws=_ws_arg(ws))


def sparse_local_pooled_attention(q, local_kv, pooled_kv, I, sinks, t0, *, ratio, window, Dv=None, out=None,
                                  ws=None) -> torch.Tensor:
    """Sparse local + pooled combine; returns out (B, L, H, Dv).  I None: every visible pooled row."""
    dev = _attn_args(q, local_kv, pooled_kv, I, sinks, t0, window, Dv, out, ws)
    d = attention_dims(q, local_kv, pooled_kv, I, ratio=ratio, window=window, Dv=Dv)
    if out is None:
        out = torch.empty((d.B, d.L, d.H, d.Dv), dtype=q.dtype, device=dev)
    wsb, n = _workspace(OP_ATTENTION, d, dev, ws)
    _check(lib().sparse_local_pooled_attention(ctypes.byref(d), _p(q), _p(local_kv), _p(pooled_kv), _p(I), _p(sinks),
                                               _p(t0), _p(out), _p(wsb), n, _stream(dev)))
    return out


def sparse_local_pooled_attention_ring(q, local_ring, pooled_kv, I, sinks, t0, ring_slot=None, *, ratio, window,
                                       Dv=None, out=None, ws=None) -> torch.Tensor:
    """The combine with the local window as a ring of local_ring.shape[1] slots: position s of sequence b in
    slot (ring_slot[b] + s - t0[b]) mod Wl_cap (ring_slot None: t0[b] mod Wl_cap); returns out (B, L, H, Dv)."""
    dev = _attn_args(q, local_ring, pooled_kv, I, sinks, t0, window, Dv, out, ws)
    if ring_slot is not None:
        _need(ring_slot, "ring_slot", 1, torch.int32, (q.shape[0],))
        _same_gpu(q=q, ring_slot=ring_slot)
    d = attention_dims(q, local_ring, pooled_kv, I, ratio=ratio, window=window, Dv=Dv)
    if out is None:
        out = torch.empty((d.B, d.L, d.H, d.Dv), dtype=q.dtype, device=dev)
    wsb, n = _workspace(OP_ATTENTION, d, dev, ws)
    _check(lib().sparse_local_pooled_attention_ring(ctypes.byref(d), _p(q), _p(local_ring), _p(pooled_kv), _p(I),
                                                    _p(sinks), _p(t0), _p(ring_slot), _p(out), _p(wsb), n,
                                                    _stream(dev)))
    return out


def decode_step_dims(q_idx, keys, q, local_kv, pooled_kv, *, ratio, window, topk, index_block, index_keep,
                     mode=MODE_AUTO) -> hisa_dims:
    B, L, H_i, D_i = q_idx.shape
    H, Dk = q.shape[2], q.shape[3]
    return hisa_dims(B=B, L=L, ratio=ratio, window=window, topk=topk, index_block=index_block,
                     index_keep=index_keep, H_i=H_i, D_i=D_i, H=H, Dk=Dk, Dv=Dk, Np_cap=keys.shape[1],
                     Wl_cap=0 if local_kv is None else local_kv.shape[1], kI=topk, mode=mode,
                     idx_dtype=_code(keys), attn_dtype=_code(q))


def hisa_decode_step(q_idx, w, keys, q, local_kv, pooled_kv, sinks, t0, *, ratio, window, topk, index_block=64,
                     index_keep=16, mode=MODE_AUTO, I=None, top_blk=None, path=None, out=None, ws=None):
    """The whole decode step (selection, then the combine on its index row); returns
    I (B,1,topk), top_blk (B,1,index_keep), path (B), out (B,1,H,Dk).  pooled_kv and
    keys share Np_cap.  A caller-given ws must start with its counter region zeroed
    (see include/hisa.h)."""
    B, L = _sel_args(q_idx, w, keys, t0)
    if L != 1:
        raise HisaError(f"hisa_decode_step takes one query row per sequence (q_idx has L = {L})")
    dev = _attn_args(q, local_kv, pooled_kv, None, sinks, t0, window, None, out, ws)
    _need(q, "q", 4, None, (B, 1, None, None))
    _need(pooled_kv, "pooled_kv", 3, None, (B, keys.shape[1], None))
    if I is not None:
        _need(I, "I", 3, torch.int32, (B, 1, topk))
    if top_blk is not None:
        _need(top_blk, "top_blk", 3, torch.int32, (B, 1, index_keep))
    if path is not None:
        _need(path, "path", 1, torch.int32, (B,))
    _same_gpu(q_idx=q_idx, w=w, keys=keys, q=q, I=I, top_blk=top_blk, path=path)
    d = decode_step_dims(q_idx, keys, q, local_kv, pooled_kv, ratio=ratio, window=window, topk=topk,
                         index_block=index_block, index_keep=index_keep, mode=mode)
    if I is None:
        I = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
    if top_blk is None:
        top_blk = torch.empty((B, 1, index_keep), dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, 1, d.H, d.Dv), dtype=q.dtype, device=dev)
    wsb, n = _workspace(OP_DECODE_STEP, d, dev, ws)
    _check(lib().hisa_decode_step(ctypes.byref(d), _p(q_idx), _p(w), _p(keys), _p(q), _p(local_kv), _p(pooled_kv),
                                  _p(sinks), _p(t0), _p(I), _p(top_blk), _p(path), _p(out), _p(wsb), n, _stream(dev)))
    return I, top_blk, path, out


def hisa_profile_enable(on: bool) -> None:
    """Turns the library's per-kernel event timing on or off (off clears the totals)."""
    _check(lib().hisa_profile_enable(1 if on else 0))


def hisa_profile_collect() -> dict:
    """Waits for the timed launches and returns {kernel: (launches, total_ms)}."""
    buf = (hisa_kernel_time * 64)()
    n = lib().hisa_profile_collect(buf, 64)
    if n < 0:
        _check(n)
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 64))}
