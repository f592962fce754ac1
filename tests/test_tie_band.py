"""The 1e-5 relative tie band of the comparison rules against f32 rounding.

The oracle sums in double and rounds each selection score once to f32; the
GPU sums the same products in f32 (bf16 products are exact in f32, so only the
additions round).  A selection can then differ from the oracle's only when two
scores lie within twice the largest GPU-vs-oracle gap of each other, and the
comparison accepts a swap only when the swapped ids score within
1e-5 * |tau| of the k-th score tau.  These tests show, on the V4-Flash decode
workload (64 heads x 128 dims, bf16 inputs, head weights ~ N(0, 1) so heads
cancel in the sum), that twice the gap of two f32 summation orders stays well
inside that band, for the fine scores (tau = 512th of 16384) and for the block
scores (tau = 16th of 256 block means).

It is an empirical margin, not a proof: the worst-case bound of f32 summation
((n-1) u sum|x| per sum) is about 30 times the band at these sizes, so the
band relies on rounding errors adding up like a random walk, as they do here.
"""
import math

import numpy as np
import pytest

import oracle
from top_kv_indexer_amd import synth

TIE_RTOL = 1e-5


@pytest.fixture(scope="module")
def flash():
    w = synth.FLASH_DECODE
    x = synth.make_inputs(w, synth.SEEDS[w.name], need_attention=False)
    d = oracle.Dims(B=1, L=1, ratio=4, topk=512, index_block=64, index_keep=16, H_i=64, D_i=128,
                    Np_cap=int(x["Np_cap"]))
    return w, x, d


def _f32_dots_sequential(q, keys):
    """Per-head dot products accumulated in f32, one dimension at a time."""
    acc = np.zeros((q.shape[0], keys.shape[0]), np.float32)
    for e in range(q.shape[1]):
        acc = (acc + q[:, e, None] * keys[None, :, e]).astype(np.float32)
    return acc


def _f32_head_sum(dots, weff, reverse=False):
    s = np.zeros(dots.shape[1], np.float32)
    hs = range(dots.shape[0] - 1, -1, -1) if reverse else range(dots.shape[0])
    for h in hs:
        s = (s + np.maximum(dots[h], np.float32(0)) * weff[h]).astype(np.float32)
    return s


def test_fine_scores_f32_gap_inside_the_band(flash):
    w, x, d = flash
    q, ww, keys = x["q_idx"][0, 0], x["w"][0, 0], x["keys"][0]
    Np = int(x["Np"][0])
    orc = oracle.scores_of(d, q, ww, keys, int(x["t0"][0]), 0, np.arange(Np, dtype=np.int32)).astype(np.float64)
    tau = np.sort(orc)[-w.topk]
    band = TIE_RTOL * abs(tau)
    weff = (ww * np.float32(1.0 / math.sqrt(w.H_i * w.D_i))).astype(np.float32)
    gaps = []
    for dots in (_f32_dots_sequential(q, keys), (q @ keys.T).astype(np.float32)):
        for rev in (False, True):
            gaps.append(np.abs(_f32_head_sum(dots, weff, rev).astype(np.float64) - orc).max())
    assert 2 * max(gaps) <= 0.25 * band, (gaps, band)


def test_block_scores_f32_gap_inside_the_band(flash):
    # The decode scan forms a block's score from the f32 mean of its rows'
    # per-head dot products (the mean is linear, so this is the dot with the
    # block mean); the oracle takes the double mean of the keys.
    w, x, d = flash
    q, ww = x["q_idx"][0, 0], x["w"][0, 0]
    cs_orc = oracle.block_scores(d, x["q_idx"], x["w"], x["keys"], x["t0"])[0][0, 0].astype(np.float64)
    nb = int(x["Np"][0]) // w.index_block
    tau = np.sort(cs_orc[:nb])[-w.index_keep]
    band = TIE_RTOL * abs(tau)
    dots = _f32_dots_sequential(q, x["keys"][0, :nb * w.index_block]).reshape(w.H_i, nb, w.index_block)
    sums = np.zeros((w.H_i, nb), np.float32)
    for r in range(w.index_block):
        sums = (sums + dots[:, :, r]).astype(np.float32)
    means = (sums * np.float32(1.0 / w.index_block)).astype(np.float32)
    weff = (ww * np.float32(1.0 / math.sqrt(w.H_i * w.D_i))).astype(np.float32)
    gap = np.abs(_f32_head_sum(means, weff).astype(np.float64) - cs_orc[:nb]).max()
    assert 2 * gap <= 0.25 * band, (gap, band)
