"""CPU oracle for HiSA selection, the flat top-k indexer and the sparse
local+pooled combine (ctypes over hisa_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It imports nothing from the HIP
library and the HIP library imports nothing from it.

Inputs are numpy arrays; bf16 data arrive as float32 arrays holding the same
values.  See hisa_oracle.c for the passage each function follows.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_lib = None

PATH_DENSE, PATH_FLAT, PATH_HISA = 0, 1, 2
NEG = np.float32(-1e30)


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "B", "L", "ratio", "window", "topk", "index_block", "index_keep",
        "H_i", "D_i", "H", "Dk", "Dv", "Np_cap", "force_flat", "force_dense")]


@dataclass
class Dims:
    B: int = 1
    L: int = 1
    ratio: int = 4
    window: int = 128
    topk: int = 512
    index_block: int = 64
    index_keep: int = 16
    H_i: int = 64
    D_i: int = 128
    H: int = 64
    Dk: int = 512
    Dv: int = 512
    Np_cap: int = 0
    force_flat: int = 0
    force_dense: int = 0

    def c(self) -> _Dims:
        return _Dims(*(int(getattr(self, f)) for f, _ in _Dims._fields_))


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.POINTER
        f32p, i32p, f64p = P(ctypes.c_float), P(ctypes.c_int), P(ctypes.c_double)
        dp = P(_Dims)
        L.orc_num_pooled.argtypes = [ctypes.c_int] * 3
        L.orc_visible.argtypes = [ctypes.c_int] * 3
        L.orc_gate.argtypes = [dp, ctypes.c_int]
        L.orc_score.argtypes = [dp, f32p, f32p, f32p]
        L.orc_score.restype = ctypes.c_float
        L.orc_block_mean.argtypes = [dp, f32p, ctypes.c_int, f64p]
        L.orc_topk.argtypes = [f32p, i32p, ctypes.c_int, ctypes.c_int, i32p]
        L.orc_select_row.argtypes = [dp, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, i32p,
                                     i32p, i32p, i32p]
        L.orc_select.argtypes = [dp, f32p, f32p, f32p, i32p, i32p, i32p, i32p]
        L.orc_coarse_row.argtypes = [dp, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, f32p]
        L.orc_block_scores.argtypes = [dp, f32p, f32p, f32p, i32p, f32p, f32p]
        L.orc_scores_of.argtypes = [dp, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, i32p,
                                    ctypes.c_int, f32p]
        L.orc_combine_row.argtypes = [dp, f32p, f32p, f32p, i32p, ctypes.c_int, f32p,
                                      ctypes.c_int, ctypes.c_int, f64p]
        L.orc_combine.argtypes = [dp, f32p, f32p, f32p, i32p, ctypes.c_int, f32p, i32p,
                                  ctypes.c_int, f64p]
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _fp(a):
    return None if a is None else _p(a, ctypes.c_float)


def _ip(a):
    return None if a is None else _p(a, ctypes.c_int)


def num_pooled(t0: int, L: int, ratio: int) -> int:
    return lib().orc_num_pooled(int(t0), int(L), int(ratio))


def visible(t: int, ratio: int, Np: int) -> int:
    return lib().orc_visible(int(t), int(ratio), int(Np))


def gate(d: Dims, Np: int) -> int:
    dc = d.c()
    return lib().orc_gate(ctypes.byref(dc), int(Np))


def score(d: Dims, q_row, w_row, key) -> np.float32:
    """One indexer score; q_row (H_i, D_i), w_row (H_i), key (D_i)."""
    dc = d.c()
    q_row, w_row, key = _f32(q_row), _f32(w_row), _f32(key)
    return np.float32(lib().orc_score(ctypes.byref(dc), _fp(q_row), _fp(w_row), _fp(key)))


def block_mean(d: Dims, keys_b, beta: int) -> np.ndarray:
    dc = d.c()
    keys_b = _f32(keys_b)
    out = np.zeros(d.D_i, np.float64)
    lib().orc_block_mean(ctypes.byref(dc), _fp(keys_b), int(beta), _p(out, ctypes.c_double))
    return out


def topk(s, ids, k: int) -> np.ndarray:
    s, ids = _f32(s), _i32(ids)
    out = np.full(max(k, 1), -1, np.int32)
    n = lib().orc_topk(_fp(s), _ip(ids), len(s), int(k), _ip(out))
    return out[:n]


def select_row(d: Dims, q_row, w_row, keys_b, t0: int, j: int, given_blocks=None):
    """One row of the selector; returns (I_row, blk_row, path)."""
    dc = d.c()
    q_row, w_row, keys_b = _f32(q_row), _f32(w_row), _f32(keys_b)
    gb = None if given_blocks is None else _i32(given_blocks)
    I = np.empty(d.topk, np.int32)
    blk = np.empty(max(d.index_keep, 1), np.int32)
    path = np.zeros(1, np.int32)
    lib().orc_select_row(ctypes.byref(dc), _fp(q_row), _fp(w_row), _fp(keys_b), int(t0), int(j),
                         _ip(gb), _ip(I), _ip(blk), _ip(path))
    return I, blk[:d.index_keep], int(path[0])


def select(d: Dims, q, w, keys, t0):
    """All rows: q (B,L,H_i,D_i), w (B,L,H_i), keys (B,Np_cap,D_i), t0 (B).
    Returns I (B,L,topk), blk (B,L,index_keep), path (B,L)."""
    dc = d.c()
    q, w, keys, t0 = _f32(q), _f32(w), _f32(keys), _i32(t0)
    I = np.empty((d.B, d.L, d.topk), np.int32)
    blk = np.empty((d.B, d.L, max(d.index_keep, 1)), np.int32)
    path = np.empty((d.B, d.L), np.int32)
    lib().orc_select(ctypes.byref(dc), _fp(q), _fp(w), _fp(keys), _ip(t0), _ip(I), _ip(blk),
                     _ip(path))
    return I, blk[..., :d.index_keep], path


def block_scores(d: Dims, q, w, keys, t0):
    """cscore (B,L,nb_cap) and rep (B,nb_cap,D_i), nb_cap = Np_cap // index_block."""
    dc = d.c()
    q, w, keys, t0 = _f32(q), _f32(w), _f32(keys), _i32(t0)
    nb_cap = d.Np_cap // d.index_block
    cs = np.empty((d.B, d.L, nb_cap), np.float32)
    rep = np.empty((d.B, nb_cap, d.D_i), np.float32)
    lib().orc_block_scores(ctypes.byref(dc), _fp(q), _fp(w), _fp(keys), _ip(t0), _fp(cs), _fp(rep))
    return cs, rep


def coarse_row(d: Dims, q_row, w_row, keys_b, t0: int, j: int) -> np.ndarray:
    """Coarse scores (nb_cap,) of one query row, batched mask applied."""
    dc = d.c()
    q_row, w_row, keys_b = _f32(q_row), _f32(w_row), _f32(keys_b)
    out = np.empty(d.Np_cap // d.index_block, np.float32)
    lib().orc_coarse_row(ctypes.byref(dc), _fp(q_row), _fp(w_row), _fp(keys_b), int(t0), int(j), _fp(out))
    return out


def scores_of(d: Dims, q_row, w_row, keys_b, t0: int, j: int, ids) -> np.ndarray:
    dc = d.c()
    q_row, w_row, keys_b, ids = _f32(q_row), _f32(w_row), _f32(keys_b), _i32(ids)
    out = np.empty(len(ids), np.float32)
    lib().orc_scores_of(ctypes.byref(dc), _fp(q_row), _fp(w_row), _fp(keys_b), int(t0), int(j),
                        _ip(ids), len(ids), _fp(out))
    return out


def combine_row(d: Dims, q_row, local_b, pooled_b, I_row, sinks, t0: int, j: int) -> np.ndarray:
    """One query row: q_row (H,Dk), local_b (Wl_cap,Dk), pooled_b (Np_cap,Dk), I_row (kI)."""
    dc = d.c()
    q_row, local_b, pooled_b, I_row = _f32(q_row), _f32(local_b), _f32(pooled_b), _i32(I_row)
    s = None if sinks is None else _f32(sinks)
    out = np.empty((d.H, d.Dv), np.float64)
    lib().orc_combine_row(ctypes.byref(dc), _fp(q_row), _fp(local_b), _fp(pooled_b), _ip(I_row),
                          len(I_row), _fp(s), int(t0), int(j), _p(out, ctypes.c_double))
    return out


def combine(d: Dims, q, local_kv, pooled_kv, I, sinks, t0) -> np.ndarray:
    """All rows -> out (B,L,H,Dv) float64."""
    dc = d.c()
    q, local_kv, pooled_kv, I, t0 = _f32(q), _f32(local_kv), _f32(pooled_kv), _i32(I), _i32(t0)
    s = None if sinks is None else _f32(sinks)
    out = np.empty((d.B, d.L, d.H, d.Dv), np.float64)
    lib().orc_combine(ctypes.byref(dc), _fp(q), _fp(local_kv), _fp(pooled_kv), _ip(I), I.shape[-1],
                      _fp(s), _ip(t0), local_kv.shape[1], _p(out, ctypes.c_double))
    return out
