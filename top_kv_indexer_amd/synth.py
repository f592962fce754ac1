"""Seeded synthetic inputs for the HiSA selector and the sparse combine.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic and is shared, read-only, by the tests, the benchmark and
the CPU oracle's callers.  Every tensor is drawn in float32 from one
numpy Generator(PCG64(seed)) in a fixed order, then rounded once to bf16
(round to nearest even) where the workload is bf16, so every consumer sees the
same values.  Rows past a sequence's pooled count (padding of ragged batches)
hold NaN: nothing may read them.

Workload shapes follow the DeepSeek-V4-Flash indexer configuration (HiSA issue,
Configuration table: index_topk 512, 64 indexer heads of dim 128, window 128,
index_block 64, index_keep 16) and the DSA indexer issue (flat top-k over
per-token keys).
"""
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np


@dataclass
class Workload:
    name: str
    B: int
    L: int
    ratio: int
    window: int
    topk: int
    index_block: int
    index_keep: int
    H_i: int
    D_i: int
    H: int
    Dk: int
    Dv: int
    bf16: bool
    t0: Optional[List[int]] = None          # fixed per-sequence offsets, or None to draw
    t0_range: Optional[tuple] = None        # (lo, hi) inclusive, drawn first when t0 is None
    planted: int = 0                        # planted high-score blocks per sequence
    layernorm_keys: bool = False
    sinks: bool = True
    Np_cap: Optional[int] = None            # padded pooled rows per sequence (default: max Np)
    force_flat: int = 0
    extra: Dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny decode: f32, Np = 1024 (t0 = 4096, r = 4), H_i 4 x D_i 32, topk 64, b 16.
TINY_DECODE = Workload("tiny_decode_np1024_f32", B=1, L=1, ratio=4, window=128, topk=64,
                       index_block=16, index_keep=16, H_i=4, D_i=32, H=4, Dk=64, Dv=64,
                       bf16=False, t0=[4096], planted=6)
# V4-Flash-shaped single decode step, Np = 16384.
FLASH_DECODE = Workload("v4flash_decode_np16384", B=1, L=1, ratio=4, window=128, topk=512,
                        index_block=64, index_keep=16, H_i=64, D_i=128, H=64, Dk=512, Dv=512,
                        bf16=True, t0=[65536], planted=32)
# Batched ragged decode: B = 32, t0 ~ U{16384..131072}, Np up to 32768.
BATCHED_DECODE = Workload("batched_decode_b32_ragged", B=32, L=1, ratio=4, window=128, topk=512,
                          index_block=64, index_keep=16, H_i=64, D_i=128, H=64, Dk=512, Dv=512,
                          bf16=True, t0_range=(16384, 131072), planted=32, Np_cap=32768)
# Batched HiSA prefill chunk: L = 2048 rows at t0 = 63488 (Np = 16384).
PREFILL = Workload("hisa_prefill_l2048_np16384", B=1, L=2048, ratio=4, window=128, topk=512,
                   index_block=64, index_keep=16, H_i=64, D_i=128, H=64, Dk=512, Dv=512,
                   bf16=True, t0=[63488], planted=0)
# Flat DSA baseline over per-token keys (ratio 1), kv_len 32768, topk 2048.
DSA_DECODE = Workload("dsa_flat_decode_kv32768", B=1, L=1, ratio=1, window=0, topk=2048,
                      index_block=0, index_keep=16, H_i=64, D_i=128, H=128, Dk=576, Dv=576,
                      bf16=True, t0=[32767], layernorm_keys=True, sinks=False)
DSA_PREFILL = DSA_DECODE.with_(name="dsa_flat_prefill_l4096_kv32768", L=4096, t0=[28672])

# Multi-token verify chunks on the V4-Flash decode shapes: 4 rows (the short-
# chunk selection) and 9 rows (just past it: the prefill row selection).
VERIFY_L4 = FLASH_DECODE.with_(name="v4flash_verify_l4_np16384", L=4, t0=[65532])
VERIFY_L9 = FLASH_DECODE.with_(name="v4flash_verify_l9_np16384", L=9, t0=[65527])

WORKLOADS = {w.name: w for w in (TINY_DECODE, FLASH_DECODE, BATCHED_DECODE, PREFILL,
                                 DSA_DECODE, DSA_PREFILL, VERIFY_L4, VERIFY_L9)}
# Seeds: one stream per workload family.
SEEDS = {TINY_DECODE.name: 1001, FLASH_DECODE.name: 1002, BATCHED_DECODE.name: 1003,
         PREFILL.name: 1004, DSA_DECODE.name: 1005, DSA_PREFILL.name: 1005,
         VERIFY_L4.name: 1002, VERIFY_L9.name: 1002}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(x.shape)


def pooled_count(t0: int, L: int, ratio: int) -> int:
    """Pooled rows present after the step (whole windows only)."""
    return (t0 + L) // ratio


def local_start(t0: int, window: int) -> int:
    """Absolute position held by local-window row 0."""
    return max(0, t0 - window + 1)


def make_inputs(w: Workload, seed: int, need_attention: bool = True) -> Dict[str, np.ndarray]:
    """Draws one workload.  Returns float32 arrays (bf16-valued where w.bf16):
    q_idx (B,L,H_i,D_i), w (B,L,H_i), keys (B,Np_cap,D_i), q (B,L,H,Dk),
    local_kv (B,Wl_cap,Dk), pooled_kv (B,Np_cap,Dk), sinks (H,) or None, and
    t0 (B,) int32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rnd = round_bf16 if w.bf16 else (lambda a: np.ascontiguousarray(a, np.float32))
    if w.t0 is not None:
        t0 = np.array(w.t0, dtype=np.int64)
        assert len(t0) == w.B
    else:
        lo, hi = w.t0_range
        t0 = rng.integers(lo, hi + 1, size=w.B)
    Np = np.array([pooled_count(int(t), w.L, w.ratio) for t in t0])
    Np_cap = int(w.Np_cap if w.Np_cap is not None else Np.max())
    assert Np.max() <= Np_cap
    ls = np.array([local_start(int(t), w.window) for t in t0])
    Wl = np.array([int(t) + w.L - int(s) for t, s in zip(t0, ls)]) if w.window > 0 else np.zeros(w.B, int)
    Wl_cap = max(int(Wl.max()), 1)

    def normal(shape):
        return rng.standard_normal(size=shape, dtype=np.float32)

    out = {}
    if w.layernorm_keys:
        keys = normal((w.B, Np_cap, w.D_i))
        mu = keys.mean(axis=-1, keepdims=True, dtype=np.float64)
        var = ((keys - mu) ** 2).mean(axis=-1, keepdims=True)
        keys = ((keys - mu) / np.sqrt(var + 1e-6)).astype(np.float32)
        q_idx = normal((w.B, w.L, w.H_i, w.D_i))
        wts = normal((w.B, w.L, w.H_i))
    else:
        q_idx = normal((w.B, w.L, w.H_i, w.D_i))
        wts = normal((w.B, w.L, w.H_i))
        keys = normal((w.B, Np_cap, w.D_i))
    q_idx = rnd(q_idx)
    planted = np.full((w.B, max(w.planted, 1)), -1, np.int64)
    if w.planted > 0 and w.index_block > 0:
        for b in range(w.B):
            nb = int(Np[b]) // w.index_block
            n = min(w.planted, nb)
            ids = rng.choice(nb, size=n, replace=False)
            planted[b, :n] = ids
            u = q_idx[b, 0].astype(np.float64).sum(axis=0)
            qhat = (u / np.linalg.norm(u)).astype(np.float32)
            for beta in ids:
                keys[b, beta * w.index_block:(beta + 1) * w.index_block, :] += 2.0 * qhat
    keys = rnd(keys)
    for b in range(w.B):
        keys[b, Np[b]:, :] = np.nan
    out.update(q_idx=q_idx, w=wts.astype(np.float32), keys=keys)
    if need_attention:
        q = rnd(normal((w.B, w.L, w.H, w.Dk)))
        local_kv = rnd(normal((w.B, Wl_cap, w.Dk)))
        pooled_kv = rnd(normal((w.B, Np_cap, w.Dk)))
        for b in range(w.B):
            local_kv[b, Wl[b]:, :] = np.nan
            pooled_kv[b, Np[b]:, :] = np.nan
        sinks = normal((w.H,)) if w.sinks else None
        out.update(q=q, local_kv=local_kv, pooled_kv=pooled_kv, sinks=sinks)
    out.update(t0=t0.astype(np.int32), Np=Np.astype(np.int32), Wl=Wl.astype(np.int32),
               planted=planted.astype(np.int32), Np_cap=Np_cap, Wl_cap=Wl_cap)
    return out
