"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-derived
worked examples (tests/golden/*.json, each with its citation and derivation),
closed forms, special cases that reduce to a library routine (numpy dot,
numpy sorts, torch scaled_dot_product_attention in float64), invariants the
pages state (hierarchy equivalence, causality, tail exclusion, gate table,
dense equivalence), and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Dims, PATH_DENSE, PATH_FLAT, PATH_HISA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- a1, a2: integers

def test_pooled_counts_of_the_workloads():
    # Tiny decode t0 = 4096 -> 1024 pooled rows; V4-Flash decode t0 = 65536 -> 16384.
    assert oracle.num_pooled(4096, 1, 4) == 1024
    assert oracle.num_pooled(65536, 1, 4) == 16384
    # Prefill chunk t0 = 63488, L = 2048: Np = 16384, per-row prefix 15872 .. 16384.
    Np = oracle.num_pooled(63488, 2048, 4)
    assert Np == 16384
    assert oracle.visible(63488 + 0, 4, Np) == 15872
    assert oracle.visible(63488 + 2047, 4, Np) == 16384
    # Ratio 1 (per-token DSA keys): V(t) = t + 1.
    assert oracle.num_pooled(32767, 1, 1) == 32768
    assert oracle.num_pooled(28672, 4096, 1) == 32768
    for t in (0, 5, 28672, 32767):
        assert oracle.visible(t, 1, 32768) == t + 1


def test_visibility_closed_form():
    # p visible iff p < floor((t+1)/r): the pooled row p closes at token p*r + r - 1.
    for r in (1, 4, 128):
        for t in range(0, 3 * r + 2):
            V = oracle.visible(t, r, 10 ** 6)
            for p in range(0, 5):
                closes = p * r + r - 1
                assert (p < V) == (closes <= t)
    # Clamped by Np.
    assert oracle.visible(10 ** 6, 4, 7) == 7


def test_engagement_table():
    # HiSA issue, Engagement thresholds (r = 4, topk 512, b 64, keep 16).
    d = Dims(topk=512, index_block=64, index_keep=16)
    assert oracle.gate(d, 0) == PATH_DENSE
    assert oracle.gate(d, 512) == PATH_DENSE
    assert oracle.gate(d, 513) == PATH_FLAT
    assert oracle.gate(d, 1023) == PATH_FLAT
    assert oracle.gate(d, 1024) == PATH_HISA
    assert oracle.gate(d, 16384) == PATH_HISA
    # index_block == 0 disables the hierarchy.
    assert oracle.gate(Dims(topk=512, index_block=0), 4096) == PATH_FLAT
    # b * keep < k: not enough fine candidates to fill the top-k.
    assert oracle.gate(Dims(topk=512, index_block=16, index_keep=16), 4096) == PATH_FLAT
    # The force-flat switch replaces only the hierarchy.
    assert oracle.gate(Dims(topk=512, force_flat=1), 4096) == PATH_FLAT
    assert oracle.gate(Dims(topk=512, force_flat=1), 300) == PATH_DENSE
    # The dense-fallback switch turns the indexer off at every length.
    for Np in (0, 300, 700, 4096, 16384):
        assert oracle.gate(Dims(topk=512, force_dense=1), Np) == PATH_DENSE


def test_force_dense_selects_every_pooled_row():
    # HiSA issue, Implementation plan item 1 (dense fallback): with the indexer
    # off, a row's index list is every pooled row, in order, padded with -1
    # (the index row is sized to the pooled capacity).
    rng = np.random.default_rng(23)
    H, D, Np_cap = 2, 4, 40
    d = Dims(B=2, L=3, ratio=1, topk=Np_cap, H_i=H, D_i=D, index_block=4, index_keep=2, window=0, Np_cap=Np_cap,
             force_dense=1)
    q, w, keys, t0 = _rand_problem(rng, 2, 3, Np_cap, H, D, [10, 37])
    I, blk, path = oracle.select(d, q, w, keys, t0)
    assert (path == PATH_DENSE).all() and (blk == -1).all()
    for b, Np in enumerate((13, 40)):
        for j in range(3):
            np.testing.assert_array_equal(I[b, j], np.r_[np.arange(Np), -np.ones(Np_cap - Np, int)])


# ---------------------------------------------------------------- scoring

def test_score_hand_example():
    g = _load("flat_select_hand.json")
    d = Dims(H_i=1, D_i=2)
    for key, want in zip(g["keys"], g["scores"]):
        got = oracle.score(d, np.array(g["q"]), np.array(g["w"]), np.array(key, np.float32))
        assert got == pytest.approx(want, rel=1e-7, abs=0)


def test_score_two_head_hand_example():
    # d0 = 1*3 + 2*(-1) = 1, d1 = -3 - 1 = -4 -> relu 1, 0; (1*1 + 0*2) / sqrt(2*2) = 0.5.
    d = Dims(H_i=2, D_i=2)
    assert oracle.score(d, np.array([[1, 2], [-1, 1]]), np.array([1, 2]), np.array([3, -1])) == 0.5


def test_score_single_head_is_relu_of_library_dot():
    rng = np.random.default_rng(0)
    for D in (1, 7, 32, 128):
        d = Dims(H_i=1, D_i=D)
        for _ in range(20):
            q, k = rng.standard_normal((1, D)), rng.standard_normal(D)
            q, k = q.astype(np.float32), k.astype(np.float32)
            w = np.float32(rng.standard_normal())
            ref = max(float(np.dot(q[0].astype(np.float64), k.astype(np.float64))), 0.0) * float(w) / math.sqrt(D)
            assert oracle.score(d, q, np.array([w]), k) == np.float32(ref)


def test_score_one_hot_weight_picks_one_head():
    # w = e_h selects head h; pins the (H_i, D_i) row-major indexing of q.
    rng = np.random.default_rng(1)
    H, D = 3, 5
    d = Dims(H_i=H, D_i=D)
    q = rng.standard_normal((H, D)).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    for h in range(H):
        w = np.zeros(H, np.float32)
        w[h] = 1
        ref = max(float(np.dot(q[h].astype(np.float64), k)), 0.0) / math.sqrt(H * D)
        assert oracle.score(d, q, w, k) == np.float32(ref)


def test_score_invariants():
    rng = np.random.default_rng(2)
    H, D = 8, 16
    d = Dims(H_i=H, D_i=D)
    for _ in range(50):
        q = rng.standard_normal((H, D)).astype(np.float32)
        k = rng.standard_normal(D).astype(np.float32)
        w1 = rng.standard_normal(H).astype(np.float32)
        w2 = rng.standard_normal(H).astype(np.float32)
        s1, s2 = oracle.score(d, q, w1, k), oracle.score(d, q, w2, k)
        s12 = oracle.score(d, q, (w1.astype(np.float64) + w2).astype(np.float32), k)
        # linear in the head weights
        assert s12 == pytest.approx(float(s1) + float(s2), abs=1e-5)
        # positively homogeneous in q (exact for a power-of-two factor)
        assert oracle.score(d, 2 * q, w1, k) == 2 * s1
        # a head permutation applied to q and w together changes nothing
        perm = rng.permutation(H)
        assert oracle.score(d, q[perm], w1[perm], k) == pytest.approx(float(s1), rel=1e-6, abs=1e-7)
    # relu: all head dots negative -> exactly zero, with the +0 sign
    q = np.ones((H, D), np.float32)
    k = -np.ones(D, np.float32)
    s = oracle.score(d, q, -np.ones(H, np.float32), k)
    assert s == 0 and not np.signbit(s)


def test_block_mean_is_library_mean():
    rng = np.random.default_rng(3)
    d = Dims(D_i=8, index_block=4)
    keys = rng.standard_normal((20, 8)).astype(np.float32)
    for beta in range(5):
        ref = keys[beta * 4:(beta + 1) * 4].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(oracle.block_mean(d, keys, beta), ref, rtol=0, atol=1e-15)


def test_coarse_score_is_mean_of_pre_relu_dots():
    # One head, w = 1, keys in a cone around q so every dot is positive:
    # cscore(beta) = relu(q . rep) * scale = mean_p(q . k_p) * scale = mean_p score(p).
    rng = np.random.default_rng(4)
    D, b = 16, 8
    d = Dims(B=1, L=1, ratio=1, topk=4, H_i=1, D_i=D, index_block=b, index_keep=2, Np_cap=64)
    q = np.abs(rng.standard_normal((1, 1, 1, D))).astype(np.float32)
    keys = (np.abs(rng.standard_normal((1, 64, D))) + 0.1).astype(np.float32)
    w = np.ones((1, 1, 1), np.float32)
    cs, rep = oracle.block_scores(d, q, w, keys, np.array([63], np.int32))
    for beta in range(8):
        per_row = [float(oracle.score(d, q[0, 0], w[0, 0], keys[0, p])) for p in range(beta * b, (beta + 1) * b)]
        assert cs[0, 0, beta] == pytest.approx(np.mean(per_row), rel=1e-6)
        np.testing.assert_allclose(rep[0, beta], keys[0, beta * b:(beta + 1) * b].astype(np.float64).mean(0), rtol=1e-7)


# ---------------------------------------------------------------- top-k

def test_topk_matches_library_sort():
    rng = np.random.default_rng(5)
    for n in (1, 2, 17, 300):
        for k in (0, 1, 5, n, n + 3):
            s = rng.integers(-5, 5, size=n).astype(np.float32)  # many exact ties
            ids = rng.permutation(10 * n)[:n].astype(np.int32)
            got = oracle.topk(s, ids, k)
            order = np.lexsort((ids, -s))  # score desc, id asc
            want = np.sort(ids[order[:min(k, n)]])
            np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- flat selection

def test_flat_hand_example_decode_and_batched():
    g = _load("flat_select_hand.json")
    keys = np.array(g["keys"], np.float32)[None]
    base = dict(H_i=1, D_i=2, topk=3, ratio=1, index_block=0, window=0, Np_cap=6)
    q = np.array(g["q"], np.float32)
    w = np.array(g["w"], np.float32)
    dd = Dims(B=1, L=1, **base)
    I, _, path = oracle.select(dd, q[None, None], w[None, None], keys, np.array([g["decode"]["t0"]]))
    assert path[0, 0] == PATH_FLAT
    assert sorted(I[0, 0]) == g["decode"]["expect_I"]
    db = Dims(B=1, L=4, **base)
    L = 4
    I, _, _ = oracle.select(db, np.repeat(q[None, None], L, 1), np.repeat(w[None, None], L, 1), keys,
                            np.array([g["batched"]["t0"]]))
    assert sorted(I[0, g["batched"]["row"]]) == g["batched"]["expect_I"]
    assert sorted(I[0, 0]) == g["batched"]["row0_expect_I"]


def test_flat_equals_brute_force_sort_with_and_without_cutoff():
    # One head, D_i = 1, q = 1, w = 1: score(p) = relu(key_p) in closed form, so
    # the flat top-k is a library sort of relu(keys) (HiSA issue, Validation,
    # first selector test), with the causal cutoff p < V(t0 + j) for L > 1.
    rng = np.random.default_rng(6)
    for trial in range(20):
        Np = int(rng.integers(5, 200))
        topk = int(rng.integers(1, Np))
        L = int(rng.integers(1, 6))
        t0 = Np - L  # ratio 1
        keys = rng.integers(-4, 6, size=(1, Np, 1)).astype(np.float32)  # ties
        d = Dims(B=1, L=L, ratio=1, topk=topk, H_i=1, D_i=1, index_block=0, window=0, Np_cap=Np)
        I, _, path = oracle.select(d, np.ones((1, L, 1, 1)), np.ones((1, L, 1)), keys, np.array([t0]))
        s = np.maximum(keys[0, :, 0], 0)
        for j in range(L):
            V = min(Np, t0 + j + 1)
            sj = np.where(np.arange(Np) < V, s, -1e30).astype(np.float32)
            order = np.lexsort((np.arange(Np), -sj))
            np.testing.assert_array_equal(I[0, j][:topk], np.sort(order[:topk]))
            if V >= topk:
                assert (I[0, j][:topk] < V).all()


# ---------------------------------------------------------------- HiSA

def test_hisa_hand_example():
    g = _load("hisa_hand.json")
    keys = np.array(g["keys"], np.float32).reshape(1, -1, 1)
    d = Dims(B=1, L=1, ratio=1, topk=2, H_i=1, D_i=1, index_block=2, index_keep=2, window=0, Np_cap=7)
    I, blk, path = oracle.select(d, np.ones((1, 1, 1, 1)), np.ones((1, 1, 1)), keys, np.array([g["t0"]]))
    assert path[0, 0] == PATH_HISA
    assert sorted(blk[0, 0]) == g["expect_blocks"]
    assert sorted(I[0, 0]) == g["expect_I"]
    d.force_flat = 1
    I, _, path = oracle.select(d, np.ones((1, 1, 1, 1)), np.ones((1, 1, 1)), keys, np.array([g["t0"]]))
    assert path[0, 0] == PATH_FLAT
    assert sorted(I[0, 0]) == g["expect_flat_I"]


def _rand_problem(rng, B, L, Np_cap, H, D, t0s):
    q = rng.standard_normal((B, L, H, D)).astype(np.float32)
    w = rng.standard_normal((B, L, H)).astype(np.float32)
    keys = rng.standard_normal((B, Np_cap, D)).astype(np.float32)
    return q, w, keys, np.array(t0s, np.int32)


def test_hisa_keep_all_blocks_equals_flat():
    # nb == keep and Np == nb * b: the candidate table is every row, so the
    # fine top-k is the flat top-k exactly.
    rng = np.random.default_rng(7)
    b, keep = 16, 16
    Np = b * keep
    for L in (1, 3):
        d = Dims(B=2, L=L, ratio=1, topk=40, H_i=4, D_i=8, index_block=b, index_keep=keep, window=0, Np_cap=Np)
        q, w, keys, t0 = _rand_problem(rng, 2, L, Np, 4, 8, [Np - L, Np - L])
        I_h, _, path_h = oracle.select(d, q, w, keys, t0)
        assert (path_h == PATH_HISA).all()
        d.force_flat = 1
        I_f, _, path_f = oracle.select(d, q, w, keys, t0)
        assert (path_f == PATH_FLAT).all()
        np.testing.assert_array_equal(I_h, I_f)


def test_hisa_planted_mass_equals_flat():
    # HiSA issue, Validation: plant score mass so the true top-k lies inside the
    # top-Kb blocks; decode and batched selections equal the flat scan.
    rng = np.random.default_rng(8)
    H, D, b, keep, topk = 4, 16, 8, 4, 20
    Np = 40 * b
    for L in (1, 4):
        q = np.abs(rng.standard_normal((1, L, H, D))).astype(np.float32)
        w = np.abs(rng.standard_normal((1, L, H))).astype(np.float32)
        keys = rng.standard_normal((1, Np, D)).astype(np.float32)
        planted = rng.choice(Np // b - 1, size=3, replace=False)  # 3 <= keep blocks, never the last
        for beta in planted:
            keys[0, beta * b:(beta + 1) * b] = np.abs(keys[0, beta * b:(beta + 1) * b]) + 4.0
        d = Dims(B=1, L=L, ratio=1, topk=topk, H_i=H, D_i=D, index_block=b, index_keep=keep, window=0, Np_cap=Np)
        t0 = np.array([Np - L], np.int32)
        I_h, blk, path = oracle.select(d, q, w, keys, t0)
        assert (path == PATH_HISA).all()
        d.force_flat = 1
        I_f, _, _ = oracle.select(d, q, w, keys, t0)
        np.testing.assert_array_equal(I_h, I_f)
        for j in range(L):
            assert set(planted) <= set(blk[0, j])


def test_hisa_batched_causality_and_tail_exclusion():
    rng = np.random.default_rng(9)
    H, D, b, keep, topk, r = 4, 8, 8, 6, 24, 4
    L = 64
    t0 = 1000
    Np = (t0 + L) // r  # 266: not a multiple of b, so there is a tail
    d = Dims(B=1, L=L, ratio=r, topk=topk, H_i=H, D_i=D, index_block=b, index_keep=keep, window=0, Np_cap=Np)
    q, w, keys, t0a = _rand_problem(rng, 1, L, Np, H, D, [t0])
    I, blk, path = oracle.select(d, q, w, keys, t0a)
    assert (path == PATH_HISA).all()
    nb = Np // b
    assert nb * b < Np
    for j in range(L):
        V = min(Np, (t0 + j + 1) // r)
        sel = I[0, j]
        assert (sel >= 0).all()
        if V >= topk:
            assert (sel < V).all(), j          # causality
        assert (sel < nb * b).all(), j         # tail exclusion
        assert (blk[0, j] * b < V).all()       # eligible blocks only (enough are visible here)


def test_hisa_last_prefill_row_equals_decode():
    rng = np.random.default_rng(10)
    H, D, b, keep, topk, r = 4, 8, 8, 6, 24, 4
    L, t0 = 9, 1203
    Np = (t0 + L) // r
    d = Dims(B=1, L=L, ratio=r, topk=topk, H_i=H, D_i=D, index_block=b, index_keep=keep, window=0, Np_cap=Np)
    q, w, keys, t0a = _rand_problem(rng, 1, L, Np, H, D, [t0])
    I, blk, _ = oracle.select(d, q, w, keys, t0a)
    dd = Dims(B=1, L=1, ratio=r, topk=topk, H_i=H, D_i=D, index_block=b, index_keep=keep, window=0, Np_cap=Np)
    I1, blk1, path1 = oracle.select(dd, q[:, -1:], w[:, -1:], keys, np.array([t0 + L - 1], np.int32))
    assert path1[0, 0] == PATH_HISA
    np.testing.assert_array_equal(I[0, -1], I1[0, 0])
    np.testing.assert_array_equal(blk[0, -1], blk1[0, 0])


def test_hisa_blocks_are_library_sort_of_cscore():
    rng = np.random.default_rng(11)
    H, D, b, keep, topk, r = 4, 8, 8, 5, 30, 4
    L, t0 = 6, 2000
    Np = (t0 + L) // r
    d = Dims(B=1, L=L, ratio=r, topk=topk, H_i=H, D_i=D, index_block=b, index_keep=keep, window=0, Np_cap=Np)
    q, w, keys, t0a = _rand_problem(rng, 1, L, Np, H, D, [t0])
    _, blk, _ = oracle.select(d, q, w, keys, t0a)
    cs, _ = oracle.block_scores(d, q, w, keys, t0a)
    for j in range(L):
        order = np.lexsort((np.arange(cs.shape[-1]), -cs[0, j]))
        np.testing.assert_array_equal(np.sort(blk[0, j]), np.sort(order[:keep]))


def _np_score(q_row, w_row, key_or_mean):
    """The indexer score written out with numpy in float64, rounded once to f32."""
    H, D = q_row.shape
    dots = q_row.astype(np.float64) @ np.asarray(key_or_mean, np.float64)
    return np.float32(np.sum(np.maximum(dots, 0.0) * w_row.astype(np.float64)) / math.sqrt(H * D))


def test_scores_of_visible_ids_and_masks():
    # The tie-band judge: every id visible to row j gets that row's score of
    # its own key; negative ids and ids at or past V(t0 + j) get the mask.
    # t0 = 40, ratio 4, L = 6: Np = 11 but rows j < 3 see only 10 rows.
    rng = np.random.default_rng(21)
    H, D, r, L, t0 = 3, 8, 4, 6, 40
    Np, Np_cap = (t0 + L) // r, (t0 + L) // r + 5
    d = Dims(B=1, L=L, ratio=r, topk=4, H_i=H, D_i=D, index_block=0, window=0, Np_cap=Np_cap)
    q, w, keys, _ = _rand_problem(rng, 1, L, Np_cap, H, D, [t0])
    seen_partial = False
    for j in range(L):
        V = min(Np, (t0 + j + 1) // r)
        seen_partial |= V < Np
        ids = np.array([-3, -1, 0, 1, V - 1, V, V + 1, Np - 1, Np, Np_cap - 1], np.int32)
        got = oracle.scores_of(d, q[0, j], w[0, j], keys[0], t0, j, ids)
        for i, p in enumerate(ids.tolist()):
            if 0 <= p < V:
                np.testing.assert_allclose(got[i], _np_score(q[0, j], w[0, j], keys[0, p]), rtol=1e-6, atol=1e-7)
            else:
                assert got[i] == oracle.NEG, (j, p)
    assert seen_partial


def test_coarse_row_eligibility_and_past_nb_masks():
    # HiSA batched path: block beta takes part for row j iff its first row is
    # visible (beta * b < V), so a partly visible block is scored; blocks past
    # nb = floor(Np / b) (allocated capacity, or the incomplete tail block) are
    # masked as well, and their block means read as zero.
    rng = np.random.default_rng(22)
    H, D, b, L, t0 = 2, 8, 4, 12, 30
    Np, Np_cap = t0 + L, 60          # ratio 1: V = t0 + j + 1 = 31 .. 42; nb = 10 < nb_cap = 15
    nb = Np // b
    d = Dims(B=1, L=L, ratio=1, topk=8, H_i=H, D_i=D, index_block=b, index_keep=3, window=0, Np_cap=Np_cap)
    q, w, keys, t0a = _rand_problem(rng, 1, L, Np_cap, H, D, [t0])
    cs, rep = oracle.block_scores(d, q, w, keys, t0a)
    partly, tail = 0, 0
    for j in range(L):
        V = t0 + j + 1
        row = oracle.coarse_row(d, q[0, j], w[0, j], keys[0], t0, j)
        np.testing.assert_array_equal(row, cs[0, j])
        for beta in range(Np_cap // b):
            if beta < nb and beta * b < V:
                mean = keys[0, beta * b:(beta + 1) * b].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(cs[0, j, beta], _np_score(q[0, j], w[0, j], mean), rtol=1e-6, atol=1e-7)
                partly += (beta + 1) * b > V
            else:
                assert cs[0, j, beta] == oracle.NEG, (j, beta)
                tail += beta == nb and beta * b < V
    assert partly > 0 and tail > 0
    np.testing.assert_allclose(rep[0, :nb], keys[0, :nb * b].astype(np.float64).reshape(nb, b, D).mean(axis=1),
                               rtol=1e-6, atol=1e-7)
    assert (rep[0, nb:] == 0).all()


def test_hisa_select_uses_the_coarse_masks():
    # With index_keep above the number of eligible blocks, the retained blocks
    # of a row are all its eligible blocks plus the lowest masked ones: the
    # selector's own mask must equal the coarse stage's (a library sort of the
    # coarse scores, ties to the lowest block).
    rng = np.random.default_rng(24)
    H, D, b, L, t0 = 2, 8, 4, 10, 22
    Np = t0 + L                      # 32, nb = 8; row j sees 23 + j rows
    d = Dims(B=1, L=L, ratio=1, topk=6, H_i=H, D_i=D, index_block=b, index_keep=7, window=0, Np_cap=Np)
    q, w, keys, t0a = _rand_problem(rng, 1, L, Np, H, D, [t0])
    _, blk, path = oracle.select(d, q, w, keys, t0a)
    cs, _ = oracle.block_scores(d, q, w, keys, t0a)
    assert (path == PATH_HISA).all()
    for j in range(L):
        order = np.lexsort((np.arange(cs.shape[-1]), -cs[0, j]))
        np.testing.assert_array_equal(np.sort(blk[0, j]), np.sort(order[:7]))


def test_selectors_dense_case_and_given_blocks():
    rng = np.random.default_rng(12)
    H, D = 2, 4
    d = Dims(B=1, L=1, ratio=4, topk=64, H_i=H, D_i=D, index_block=8, index_keep=4, window=0, Np_cap=50)
    q, w, keys, _ = _rand_problem(rng, 1, 1, 50, H, D, [0])
    I, blk, path = oracle.select(d, q, w, keys, np.array([4 * 50 - 1], np.int32))
    assert path[0, 0] == PATH_DENSE
    np.testing.assert_array_equal(I[0, 0][:50], np.arange(50))
    assert (I[0, 0][50:] == -1).all() and (blk == -1).all()
    # given_blocks reproduces the row's own fine stage
    d2 = Dims(B=1, L=1, ratio=1, topk=8, H_i=H, D_i=D, index_block=4, index_keep=3, window=0, Np_cap=40)
    q, w, keys, _ = _rand_problem(rng, 1, 1, 40, H, D, [0])
    I_a, blk_a, _ = oracle.select_row(d2, q[0, 0], w[0, 0], keys[0], 39, 0)
    I_b, _, _ = oracle.select_row(d2, q[0, 0], w[0, 0], keys[0], 39, 0, given_blocks=blk_a[::-1].copy())
    np.testing.assert_array_equal(I_a, I_b)


# ---------------------------------------------------------------- combine

def test_combine_hand_example():
    g = _load("combine_hand.json")
    d = Dims(B=1, L=1, ratio=1, window=1, H=1, Dk=2, Dv=2, Np_cap=2)
    out = oracle.combine_row(d, np.array(g["q"], np.float32), np.array(g["local"], np.float32),
                             np.array(g["pooled"], np.float32), np.array(g["I"]),
                             np.array(g["sinks"], np.float32), g["t0"], 0)
    np.testing.assert_allclose(out, np.array(g["expect"]), rtol=1e-6)


def _sdpa_f64(q, keys, vals, bias):
    """torch SDPA in float64 on the CPU. q (H, Dk), keys (n, Dk), vals (n, Dv), bias (H, n)."""
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]          # (1, H, 1, Dk)
    kt = torch.from_numpy(keys.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(vals.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    mt = torch.from_numpy(bias.astype(np.float64))[None, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("with_sink", [False, True])
def test_combine_equals_library_softmax_attention(with_sink):
    # Every pooled row selected and the sink folded in as one more key with a
    # zero key/value row and an additive logit sink[h] (the sink absorbs mass
    # but contributes no value).
    rng = np.random.default_rng(13)
    H, Dk, window, r = 3, 16, 8, 4
    L, t0 = 5, 37
    Np = (t0 + L) // r
    ls = max(0, t0 - window + 1)
    Wl = t0 + L - ls
    d = Dims(B=1, L=L, ratio=r, window=window, H=H, Dk=Dk, Dv=Dk, Np_cap=Np)
    q = rng.standard_normal((1, L, H, Dk)).astype(np.float32)
    local = rng.standard_normal((1, Wl, Dk)).astype(np.float32)
    pooled = rng.standard_normal((1, Np, Dk)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32) if with_sink else None
    I = np.tile(np.arange(Np, dtype=np.int32), (1, L, 1))
    out = oracle.combine(d, q, local, pooled, I, sinks, np.array([t0], np.int32))
    for j in range(L):
        t = t0 + j
        V = min(Np, (t + 1) // r)
        pos = ls + np.arange(Wl)
        lmask = (pos > t - window) & (pos <= t)
        keys = np.concatenate([local[0], pooled[0]])
        bias = np.concatenate([np.where(lmask, 0.0, -np.inf), np.where(np.arange(Np) < V, 0.0, -np.inf)])
        bias = np.tile(bias, (H, 1))
        if with_sink:
            keys = np.concatenate([keys, np.zeros((1, Dk), np.float32)])
            bias = np.concatenate([bias, sinks.astype(np.float64)[:, None]], axis=1)
        ref = _sdpa_f64(q[0, j], keys, keys, bias)
        np.testing.assert_allclose(out[0, j], ref, rtol=1e-10, atol=1e-12)


def test_combine_invariants():
    rng = np.random.default_rng(14)
    H, Dk, window, r = 2, 8, 4, 4
    L, t0 = 3, 200
    Np = (t0 + L) // r
    ls = max(0, t0 - window + 1)
    Wl = t0 + L - ls
    d = Dims(B=1, L=L, ratio=r, window=window, H=H, Dk=Dk, Dv=Dk, Np_cap=Np)
    q = rng.standard_normal((1, L, H, Dk)).astype(np.float32)
    local = rng.standard_normal((1, Wl, Dk)).astype(np.float32)
    pooled = rng.standard_normal((1, Np, Dk)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    I = np.stack([rng.choice(Np, 10, replace=False) for _ in range(L)])[None].astype(np.int32)
    t0a = np.array([t0], np.int32)
    base = oracle.combine(d, q, local, pooled, I, sinks, t0a)
    # permuting I within a row changes nothing
    perm = I[:, :, rng.permutation(10)]
    np.testing.assert_allclose(oracle.combine(d, q, local, pooled, perm, sinks, t0a), base, rtol=1e-12, atol=1e-14)
    # -1 entries and invisible ids are masked
    padded = np.concatenate([I, -np.ones((1, L, 3), np.int32), np.full((1, L, 2), Np + 5, np.int32)], axis=-1)
    np.testing.assert_allclose(oracle.combine(d, q, local, pooled, padded, sinks, t0a), base, rtol=1e-12, atol=1e-14)
    # all keys equal to one row v: out = v * n e^s / (n e^s + e^sink)
    v = rng.standard_normal(Dk).astype(np.float32)
    loc_eq = np.tile(v, (1, Wl, 1))
    pool_eq = np.tile(v, (1, Np, 1))
    out = oracle.combine(d, q, loc_eq, pool_eq, I, sinks, t0a)
    for j in range(L):
        for h in range(H):
            s = float(np.dot(q[0, j, h].astype(np.float64), v)) / math.sqrt(Dk)
            n = window + 10
            frac = n * math.exp(s) / (n * math.exp(s) + math.exp(float(sinks[h])))
            np.testing.assert_allclose(out[0, j, h], frac * v.astype(np.float64), rtol=1e-10)
    # no key and no sink -> 0; no key with a sink -> 0 (the sink has no value)
    d0 = Dims(B=1, L=1, ratio=r, window=0, H=H, Dk=Dk, Dv=Dk, Np_cap=Np)
    noI = -np.ones((1, 1, 4), np.int32)
    assert (oracle.combine(d0, q[:, :1], local, pooled, noI, None, t0a) == 0).all()
    assert (oracle.combine(d0, q[:, :1], local, pooled, noI, sinks, t0a) == 0).all()
    # one visible local key, no sink -> that row's value exactly
    d1 = Dims(B=1, L=1, ratio=r, window=1, H=H, Dk=Dk, Dv=4, Np_cap=Np)
    out = oracle.combine(d1, q[:, :1], local, pooled, noI, None, np.array([t0], np.int32))
    ls1 = max(0, t0 - 1 + 1)
    np.testing.assert_array_equal(out[0, 0], np.tile(local[0, t0 - ls1, :4].astype(np.float64), (H, 1)))


def test_combine_all_selected_equals_dense():
    # HiSA issue, Validation: with k == Np (every row selected) the sparse
    # combine reproduces dense local + pooled attention; dense here is the
    # library SDPA over [local window; all visible pooled rows] plus the sink.
    rng = np.random.default_rng(15)
    H, Dk, window, r = 2, 8, 6, 4
    t0 = 60
    Np = (t0 + 1) // r
    d = Dims(B=1, L=1, ratio=r, window=window, H=H, Dk=Dk, Dv=Dk, Np_cap=Np)
    q = rng.standard_normal((1, 1, H, Dk)).astype(np.float32)
    local = rng.standard_normal((1, window, Dk)).astype(np.float32)
    pooled = rng.standard_normal((1, Np, Dk)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    I = rng.permutation(Np).astype(np.int32)[None, None]
    out = oracle.combine(d, q, local, pooled, I, sinks, np.array([t0], np.int32))
    keys = np.concatenate([local[0], pooled[0], np.zeros((1, Dk), np.float32)])
    bias = np.concatenate([np.zeros((H, window + Np)), sinks.astype(np.float64)[:, None]], axis=1)
    np.testing.assert_allclose(out[0, 0], _sdpa_f64(q[0, 0], keys, keys, bias), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- planted mutations

def test_pins_catch_planted_mistakes(tmp_path):
    """Builds copies of the oracle with one plausible mistake each (on the CPU)
    and checks that the pins above would fail for every one of them."""
    import ctypes
    import subprocess
    src = open(os.path.join(os.path.dirname(oracle.__file__), "hisa_oracle.c")).read()
    mutations = {
        "dropped relu": ("double s = dot > 0.0 ? dot : 0.0;\n    acc += s * ((double)w_row[h] * c);\n  }\n  return finish_score(acc);\n}\n\n/* The same",
                         "double s = dot;\n    acc += s * ((double)w_row[h] * c);\n  }\n  return finish_score(acc);\n}\n\n/* The same"),
        "transposed q": ("dot += (double)q_row[h * d->D_i + e] * (double)key[e];",
                         "dot += (double)q_row[e * d->H_i + h] * (double)key[e];"),
        "wrong scale": ("const double c = 1.0 / sqrt((double)d->H_i * (double)d->D_i);\n  double acc = 0.0;\n  for (int h = 0; h < d->H_i; h++) {\n    double dot = 0.0;\n    for (int e = 0; e < d->D_i; e++) dot += (double)q_row[h * d->D_i + e] * (double)key[e];",
                        "const double c = 1.0 / sqrt((double)d->D_i);\n  double acc = 0.0;\n  for (int h = 0; h < d->H_i; h++) {\n    double dot = 0.0;\n    for (int e = 0; e < d->D_i; e++) dot += (double)q_row[h * d->D_i + e] * (double)key[e];"),
        "ascending topk": ("if (a->s > b->s) return -1;\n  if (a->s < b->s) return 1;",
                           "if (a->s < b->s) return -1;\n  if (a->s > b->s) return 1;"),
        "no causal mask": ("s[q] = q < valid ?", "s[q] = q < Np ?"),
        "visible off by one": ("return imin(Np, (int)(((long long)t + 1) / ratio));",
                               "return imin(Np, (int)(((long long)t) / ratio));"),
        "block mean divisor": ("rep[e] = s / (double)b;", "rep[e] = s / (double)(b - 1);"),
        "tail candidate": ("const int nb = Np / b;\n  const int Kb", "const int nb = (Np + b - 1) / b;\n  const int Kb"),
        "no sink": ("double Z = sinks ? exp((double)sinks[h] - m) : 0.0;", "double Z = 0.0;"),
        "window too wide": ("const int s_lo = imax(ls, t - d->window + 1);", "const int s_lo = imax(ls, t - d->window);"),
        "no pooled re-mask": ("if (id >= 0 && id < V) rows[n++]", "if (id >= 0) rows[n++]"),
        "scores_of masks at Np": ("out[i] = (p >= 0 && p < valid) ?", "out[i] = (p >= 0 && p < Np) ?"),
        "scores_of ignores the row": ("const int valid = orc_visible(t0 + j, d->ratio, Np);\n  for (int i = 0; i < n; i++) {",
                                      "const int valid = orc_visible(t0, d->ratio, Np);\n  for (int i = 0; i < n; i++) {"),
        "coarse row without eligibility": ("if (beta < nb && beta * b < valid) {", "if (beta < nb) {"),
        "coarse row without nb mask": ("if (beta < nb && beta * b < valid) {", "if (beta * b < valid) {"),
        "coarse eligibility on the last row": ("if (beta * b < valid) {\n        orc_block_mean",
                                               "if (beta * b + b <= valid) {\n        orc_block_mean"),
        "force-dense ignored": ("if (d->force_dense) return ORC_PATH_DENSE;", ""),
    }
    import importlib
    import sys
    tests = [test_scores_of_visible_ids_and_masks, test_coarse_row_eligibility_and_past_nb_masks,
             test_hisa_select_uses_the_coarse_masks, test_engagement_table, test_force_dense_selects_every_pooled_row,
             test_score_hand_example, test_score_two_head_hand_example, test_score_single_head_is_relu_of_library_dot,
             test_score_one_hot_weight_picks_one_head, test_score_invariants, test_block_mean_is_library_mean,
             test_coarse_score_is_mean_of_pre_relu_dots, test_topk_matches_library_sort,
             test_flat_hand_example_decode_and_batched, test_flat_equals_brute_force_sort_with_and_without_cutoff,
             test_hisa_hand_example, test_hisa_keep_all_blocks_equals_flat, test_hisa_planted_mass_equals_flat,
             test_hisa_batched_causality_and_tail_exclusion, test_hisa_last_prefill_row_equals_decode,
             test_visibility_closed_form, test_pooled_counts_of_the_workloads, test_combine_hand_example,
             lambda: test_combine_equals_library_softmax_attention(True), test_combine_invariants,
             test_combine_all_selected_equals_dense]
    real = oracle._lib
    try:
        for name, (old, new) in mutations.items():
            assert src.count(old) == 1, name
            cfile = tmp_path / "m.c"
            cfile.write_text(src.replace(old, new))
            so = tmp_path / f"m_{abs(hash(name))}.so"
            subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-I",
                            os.path.dirname(oracle.__file__), str(cfile), "-o", str(so), "-lm"], check=True)
            oracle._lib = None
            saved = oracle._build.LIB
            oracle._build.LIB = str(so)
            try:
                caught = False
                for t in tests:
                    try:
                        t()
                    except AssertionError:
                        caught = True
                        break
                assert caught, f"no pin fails for the planted mistake: {name}"
            finally:
                oracle._build.LIB = saved
                oracle._lib = None
    finally:
        oracle._lib = real
