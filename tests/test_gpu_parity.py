"""Parity of the HIP library (through its C ABI) with the CPU oracle on the
same seeded inputs: the five workloads at full size (oracle on sampled rows
where it is slow) plus edge cases (ragged batches mixing the dense / flat /
HiSA / invalid paths, early prefill rows with fewer than k visible rows, tail
blocks, window 0, no sinks, masked and -1 ids, the generic VALU kernels)."""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
from tests import parity
from top_kv_indexer_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hisa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from top_kv_indexer_amd import hisa as h
    h.lib()  # fails loudly when the library is missing
    return h


_cache = {}


def inputs(w, seed):
    key = (repr(w), seed)
    if key not in _cache:
        say(f"[gen] {w.name} seed={seed}")
        x = synth.make_inputs(w, seed)
        dt = torch.bfloat16 if w.bf16 else torch.float32
        g = {}
        for k in ("q_idx", "keys", "q", "local_kv", "pooled_kv"):
            g[k] = torch.from_numpy(x[k]).to("cuda").to(dt).contiguous()
        g["w"] = torch.from_numpy(x["w"]).to("cuda")
        g["sinks"] = None if x["sinks"] is None else torch.from_numpy(x["sinks"]).to("cuda")
        g["t0"] = torch.from_numpy(x["t0"]).to("cuda")
        _cache.clear()
        _cache[key] = (x, g)
    return _cache[key]


def odims(w, x, kI=0, force_flat=0):
    return oracle.Dims(B=w.B, L=w.L, ratio=w.ratio, window=w.window, topk=w.topk, index_block=w.index_block,
                       index_keep=w.index_keep, H_i=w.H_i, D_i=w.D_i, H=w.H, Dk=w.Dk, Dv=w.Dv,
                       Np_cap=int(x["Np_cap"]), force_flat=force_flat)


def sel_kw(w, mode=0):
    return dict(ratio=w.ratio, topk=w.topk, index_block=w.index_block, index_keep=w.index_keep, mode=mode)


def rows_of(w, sample):
    if sample is None or w.B * w.L <= sample:
        return [(b, j) for b in range(w.B) for j in range(w.L)]
    rng = np.random.default_rng(123)
    picks = {(0, 0), (w.B - 1, w.L - 1), (0, w.L // 2)}
    while len(picks) < sample:
        picks.add((int(rng.integers(w.B)), int(rng.integers(w.L))))
    return sorted(picks)


def oracle_rows(d, x, rows):
    """The oracle's selection of each (b, j) in rows, on host threads (the C
    oracle releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(bj):
        b, j = bj
        return oracle.select_row(d, x["q_idx"][b, j], x["w"][b, j], x["keys"][b], int(x["t0"][b]), j)

    with ThreadPoolExecutor(max_workers=8) as ex:
        return dict(zip(rows, ex.map(one, rows)))


def check_selection(w, x, I, blk, path, mode=0, sample=None, rows=None):
    d = odims(w, x, force_flat=mode)
    I, blk, path = parity.to_np(I), parity.to_np(blk), parity.to_np(path)
    rows = rows if rows is not None else rows_of(w, sample)
    ref = oracle_rows(d, x, rows)
    for b, j in rows:
        Io, blko, po = ref[(b, j)]
        assert path[b] == po, (b, path[b], po)
        parity.check_selection_row(d, x, b, j, I[b, j], blk[b, j] if blk is not None else None, po, Io, blko, po)


def slot_rows(L, per_slot=8, seed=7, slots=8):
    """Query rows of a single sequence covering every row slot of an 8-row (or
    4-row) workgroup several times, plus the first and last workgroups whole."""
    rng = np.random.default_rng(seed)
    js = set(range(min(slots, L))) | set(range(max(0, L - slots), L))
    for sl in range(slots):
        cand = np.arange(sl, L, slots)
        js |= set(rng.choice(cand, size=min(per_slot, len(cand)), replace=False).tolist())
    return [(0, int(j)) for j in sorted(js)]


def check_rows_invariants(I, t0, ratio, topk, Np):
    """All rows of a one-sequence flat or HiSA selection whose rows all see at
    least k pooled rows: ids ascending, unique, visible, exactly k of them."""
    I = parity.to_np(I)[0]
    L = I.shape[0]
    V = np.minimum(Np, (t0 + np.arange(L) + 1) // ratio)
    k = np.minimum(topk, V)
    valid = I >= 0
    assert (valid.sum(axis=1) == k).all()
    assert (np.where(valid, I, -1) < V[:, None]).all()
    # ascending and unique among the valid entries (which come first)
    assert (valid[:, :-1] | ~valid[:, 1:]).all(), "-1 padding before a valid id"
    d = np.diff(I, axis=1)
    assert ((d > 0) | ~valid[:, 1:]).all()


def check_attention(w, x, I, out, sample=None, tol=None):
    I = parity.to_np(I)
    out = parity.to_np(out)
    d = odims(w, x)
    tol = tol if tol is not None else (2e-2 if w.bf16 else 1e-4)
    worst = 0.0
    for b, j in rows_of(w, sample):
        ref = oracle.combine_row(d, x["q"][b, j], x["local_kv"][b], x["pooled_kv"][b], I[b, j], x["sinks"],
                                 int(x["t0"][b]), j)
        err = parity.max_abs(out[b, j], ref)
        worst = max(worst, err)
        assert err <= tol, (b, j, err)
    return worst


def run_attention(hisa, w, g, I):
    return hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], I, g["sinks"], g["t0"],
                                              ratio=w.ratio, window=w.window)


DECODE = [synth.TINY_DECODE, synth.FLASH_DECODE, synth.BATCHED_DECODE]


@pytest.mark.parametrize("w", DECODE, ids=lambda w: w.name)
def test_decode_selection_and_attention(hisa, w):
    x, g = inputs(w, synth.SEEDS[w.name])
    say(f"[run] hisa_select_decode {w.name}")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_HISA).all()
    check_selection(w, x, I, blk, path)
    say(f"[run] sparse_local_pooled_attention {w.name}")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    say(f"  max-abs {check_attention(w, x, I, out):.3g}")


@pytest.mark.parametrize("w", [synth.TINY_DECODE, synth.FLASH_DECODE], ids=lambda w: w.name)
def test_decode_force_flat_and_flat_indexer(hisa, w):
    x, g = inputs(w, synth.SEEDS[w.name])
    say(f"[run] hisa_select_decode force-flat {w.name}")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w, mode=1))
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_FLAT).all()
    assert (parity.to_np(blk) == -1).all()
    check_selection(w, x, I, blk, path, mode=1)
    say(f"[run] flat_topk_select {w.name}")
    If = hisa.flat_topk_select(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio, topk=w.topk)
    torch.cuda.synchronize()
    check_selection(w, x, If, None, path, mode=1)


def test_prefill_selection_and_attention(hisa):
    w = synth.PREFILL
    x, g = inputs(w, synth.SEEDS[w.name])
    say(f"[run] hisa_select_prefill {w.name}")
    I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_HISA).all()
    # every row: ascending, unique, visible, k of them (every row sees >= k rows here)
    check_rows_invariants(I, int(x["t0"][0]), w.ratio, w.topk, int(x["Np"][0]))
    # retained blocks of every row: ascending, eligible (first row visible)
    Bn = parity.to_np(blk)[0]
    V = (int(x["t0"][0]) + np.arange(w.L) + 1) // w.ratio
    assert (np.diff(Bn, axis=1) > 0).all() and (Bn * w.index_block < V[:, None]).all()
    # the oracle on rows covering each of the four row slots of a workgroup
    rows = slot_rows(w.L, per_slot=16, slots=4)
    assert len(rows) >= 64
    check_selection(w, x, I, blk, path, rows=rows)
    say(f"[run] sparse_local_pooled_attention {w.name}")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    say(f"  max-abs {check_attention(w, x, I, out, sample=64):.3g}")


@pytest.mark.parametrize("w", [synth.DSA_DECODE, synth.DSA_PREFILL], ids=lambda w: w.name)
def test_flat_dsa(hisa, w):
    x, g = inputs(w, synth.SEEDS[w.name])
    say(f"[run] flat_topk_select {w.name}")
    I = hisa.flat_topk_select(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio, topk=w.topk)
    torch.cuda.synchronize()
    d = dataclasses.replace(odims(w, x), index_block=0)
    In = parity.to_np(I)
    if w.L > 1:
        # every row: ascending, unique, visible, exactly k
        check_rows_invariants(I, int(x["t0"][0]), w.ratio, w.topk, int(x["Np"][0]))
        # the oracle on 64+ rows covering all 8 row slots of a flat-scoring workgroup
        rows = slot_rows(w.L, per_slot=7, slots=8)
        assert len(rows) >= 64
    else:
        rows = rows_of(w, None)
    say(f"  oracle on {len(rows)} rows")
    ref = oracle_rows(d, x, rows)
    for b, j in rows:
        q, ww, kb, t0 = x["q_idx"][b, j], x["w"][b, j], x["keys"][b], int(x["t0"][b])
        parity.compare_sets(In[b, j], ref[(b, j)][0], lambda ids: oracle.scores_of(d, q, ww, kb, t0, j, ids),
                            what=f"({b},{j})")
    say(f"[run] sparse_local_pooled_attention {w.name}")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    say(f"  max-abs {check_attention(w, x, I, out, sample=16):.3g}")


def test_flat_topk_long_rows_masked_and_ties(hisa):
    # Rows longer than 8192 keys take the register-resident top-k.  Sequence
    # 0 (t0 = 100, ratio 1, 700 pooled rows) sees only 101 + j keys on row j,
    # fewer than k = 512 on rows j < 411, which are completed with the
    # lowest-index masked ids; sequence 1 has 2500 copies of one key row, so
    # thousands of exactly equal scores straddle the k-th score on many rows
    # and the lowest ids must win.  (Tiny attention shapes: unused here.)
    w = synth.DSA_DECODE.with_(name="dsa_long_rows_edges", B=2, L=600, t0=[100, 6000], Np_cap=9000, topk=512,
                               H=4, Dk=64, Dv=64)
    x, g = inputs(w, 31)
    x = dict(x)
    keys = x["keys"].copy()
    keys[1, 3000:5500] = keys[1, 3000]
    x["keys"] = keys
    gk = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
    say("[run] flat top-k on long rows with masked fill and heavy ties")
    I = hisa.flat_topk_select(g["q_idx"], g["w"], gk, g["t0"], ratio=1, topk=w.topk)
    torch.cuda.synchronize()
    d = dataclasses.replace(odims(w, x), index_block=0)
    In = parity.to_np(I)
    rows = rows_of(w, 14) + [(0, 0), (0, 200), (0, 410), (0, 411), (0, 599)]
    for b, j in rows:
        q, ww, kb, t0 = x["q_idx"][b, j], x["w"][b, j], x["keys"][b], int(x["t0"][b])
        Io, _, _ = oracle.select_row(d, q, ww, kb, t0, j)
        V = t0 + j + 1
        if b == 0 and V < w.topk:  # every visible id, then the lowest masked ids
            np.testing.assert_array_equal(In[b, j], np.arange(w.topk))
        parity.compare_sets(In[b, j], Io, lambda ids: oracle.scores_of(d, q, ww, kb, t0, j, ids), what=f"({b},{j})")
        assert (np.diff(In[b, j][In[b, j] >= 0]) > 0).all()


@pytest.mark.parametrize("case", ["flash_cap_past_np", "tiny_f32", "prefill_l96", "early_rows_ragged"])
def test_block_scores(hisa, case):
    # The coarse stage alone, including its masks: blocks past nb (capacity
    # above the pooled count: flash_cap_past_np, and the shorter sequence of
    # early_rows_ragged) and blocks whose first row a prefill row cannot see
    # yet (early_rows_ragged: t0 = 300, ratio 1, so row j sees 301 + j rows,
    # 5 of 17 blocks on row 0).
    w = {"flash_cap_past_np": synth.FLASH_DECODE.with_(name="flash_cap20000", Np_cap=20000),
         "tiny_f32": synth.TINY_DECODE,
         "prefill_l96": synth.PREFILL.with_(L=96),
         "early_rows_ragged": EARLY.with_(L=300)}[case]
    seed = 77
    x, g = inputs(w, seed)
    say(f"[run] hisa_block_scores {w.name}")
    cs, rep = hisa.hisa_block_scores(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio,
                                     index_block=w.index_block, want_rep=True)
    torch.cuda.synchronize()
    d = odims(w, x)
    cso, repo = oracle.block_scores(d, x["q_idx"], x["w"], x["keys"], x["t0"])
    np.testing.assert_allclose(parity.to_np(rep), repo, rtol=1e-6, atol=1e-7)
    csg = parity.to_np(cs)
    masked = cso == np.float32(-1e30)
    if case in ("flash_cap_past_np", "early_rows_ragged"):
        assert masked.sum() > 0
    np.testing.assert_array_equal(csg[masked], cso[masked])
    assert (csg[~masked] > np.float32(-1e30)).all()
    scale = np.abs(cso[~masked]).max()
    np.testing.assert_allclose(csg[~masked], cso[~masked], rtol=1e-4, atol=1e-5 * scale)


# ------------------------------------------------------------------ edge cases

MIXED = synth.Workload("mixed_paths_b6", B=6, L=1, ratio=4, window=128, topk=512, index_block=64, index_keep=16,
                       H_i=64, D_i=128, H=64, Dk=512, Dv=512, bf16=True,
                       # Np = 300 (dense), 700 (flat), 1024 (HiSA, no tail), 1500 (HiSA + tail),
                       # 5000 and 4100 (HiSA)
                       t0=[1200, 2800, 4096, 6000, 20000, 16400], planted=4, Np_cap=5000)


def test_mixed_paths_decode(hisa):
    w = MIXED
    x, g = inputs(w, 5)
    x = dict(x)
    say("[run] mixed-path decode")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    p = parity.to_np(path)
    assert p.tolist() == [hisa.PATH_DENSE, hisa.PATH_FLAT, hisa.PATH_HISA, hisa.PATH_HISA, hisa.PATH_HISA,
                          hisa.PATH_HISA], p
    d = odims(w, x)
    In, bn = parity.to_np(I), parity.to_np(blk)
    for b in range(6):
        parity.check_selection_row(d, x, b, 0, In[b, 0], bn[b, 0], p[b])
    # tail exclusion where Np is not a multiple of the block
    assert (In[3, 0] < (1500 // 64) * 64).all()
    say("[run] mixed-path attention")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    o = parity.to_np(out)
    dd = odims(w, x)
    for b in range(6):
        ref = oracle.combine_row(dd, x["q"][b, 0], x["local_kv"][b], x["pooled_kv"][b], In[b, 0], x["sinks"],
                                 int(x["t0"][b]), 0)
        assert parity.max_abs(o[b, 0], ref) <= 2e-2, b


def test_decode_workspace_reuse(hisa):
    # The fused decode scan + selection counts the waves that finished each
    # sequence in the workspace and returns the counters to zero: three calls
    # on one workspace, with pooled counts that change the number of waves per
    # sequence between calls, each match the oracle, and the counters end zero.
    w = MIXED
    x, g = inputs(w, 5)
    d = hisa.selection_dims(g["q_idx"], g["keys"], ratio=4, topk=512, index_block=64, index_keep=16)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d), dtype=torch.uint8, device="cuda")
    od = odims(w, x)
    # each sequence's pooled count stays within its own (non-NaN) rows
    for t0s in ([1200, 2800, 4096, 6000, 20000, 16400], [1200, 2100, 4096, 4500, 12000, 9000],
                [1000, 2800, 3000, 6000, 20000, 16000]):
        say(f"[run] decode on a reused workspace, t0 = {t0s}")
        t0 = torch.tensor(t0s, dtype=torch.int32, device="cuda")
        I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], t0, **sel_kw(w), ws=ws)
        torch.cuda.synchronize()
        xx = dict(x)
        xx["t0"] = np.array(t0s, np.int32)
        In, bn, p = parity.to_np(I), parity.to_np(blk), parity.to_np(path)
        for b in range(w.B):
            Io, blko, po = oracle.select_row(od, xx["q_idx"][b, 0], xx["w"][b, 0], xx["keys"][b], t0s[b], 0)
            assert p[b] == po, (b, p[b], po)
            parity.check_selection_row(od, xx, b, 0, In[b, 0], bn[b, 0], p[b], Io, blko, po)
    assert (ws[: counter_bytes(w)].view(torch.int32) == 0).all()


def counter_bytes(w):
    # arrival counters of the fused decode: B x (1 + ceil(slabs / 16)), 64 bytes each
    slabs = -(-w.Np_cap // 64)
    return w.B * (1 + -(-slabs // 16)) * 64


MIXED_STREAM = MIXED.with_(name="mixed_paths_b7_stream", B=7, t0=[1200, 2800, 4096, 6000, 160000, 16400, 90000],
                           Np_cap=40000)


def test_mixed_paths_decode_stream(hisa):
    # Many 64-row slabs (7 x 625) take the persistent scan over the flattened
    # live slabs: dense (Np 300), flat (700), HiSA with and without a tail
    # block and with long pooled prefixes; one sequence then turns invalid
    # (Np > Np_cap) on a reused workspace.
    w = MIXED_STREAM
    x, g = inputs(w, 21)
    od = odims(w, x)
    d = hisa.selection_dims(g["q_idx"], g["keys"], ratio=4, topk=512, index_block=64, index_keep=16)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d), dtype=torch.uint8, device="cuda")
    for t0s in (list(w.t0), [1200, 2800, 4096, 6000, 200000, 16400, 60000]):
        say(f"[run] streaming decode scan, t0 = {t0s}")
        t0 = torch.tensor(t0s, dtype=torch.int32, device="cuda")
        I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], t0, **sel_kw(w), ws=ws)
        torch.cuda.synchronize()
        xx = dict(x)
        xx["t0"] = np.array(t0s, np.int32)
        In, bn, p = parity.to_np(I), parity.to_np(blk), parity.to_np(path)
        for b in range(w.B):
            if t0s[b] == 200000:  # Np = 50000 > Np_cap
                assert p[b] == hisa.PATH_INVALID and (In[b] == -1).all() and (bn[b] == -1).all()
                continue
            Io, blko, po = oracle.select_row(od, xx["q_idx"][b, 0], xx["w"][b, 0], xx["keys"][b], t0s[b], 0)
            assert p[b] == po, (b, p[b], po)
            parity.check_selection_row(od, xx, b, 0, In[b, 0], bn[b, 0], p[b], Io, blko, po)
    assert (ws[: counter_bytes(w)].view(torch.int32) == 0).all()


def test_decode_stream_many_short_sequences(hisa):
    # 300 sequences of 1100..1400 pooled rows (about 6000 slabs: the streaming
    # scan), so each workgroup's share of about 12 slabs crosses into another
    # sequence: runs of every length from one slab, the steps after the loop
    # of whole three-slab steps, and one published count per run.
    rng = np.random.default_rng(5)
    t0 = [int(v) for v in rng.integers(4400, 5600, size=300)]
    w = MIXED.with_(name="stream_b300_short", B=300, t0=t0, Np_cap=1400, planted=2, H=4, Dk=64, Dv=64)
    x, g = inputs(w, 23)
    say("[run] streaming decode scan over 300 short sequences")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_HISA).all()
    check_selection(w, x, I, blk, path, sample=48)


@pytest.mark.parametrize("case", [(MIXED, 5), (MIXED_STREAM, 21)], ids=["latency_scan", "streaming_scan"])
def test_decode_exact_ties(hisa, case):
    # Exact score ties straddle both top-k boundaries of the decode selection:
    # the best-scoring row of each HiSA sequence is copied over rows 640 ..
    # 2559 (blocks 10 .. 39), so up to 30 blocks share the top coarse score
    # and up to 1920 rows the top fine score; the flat sequence gets 500 equal
    # rows.  Both sides break ties by the lowest id, so the tied ids that are
    # kept must be exactly the oracle's.
    w, seed = case
    x, g = inputs(w, seed)
    od = odims(w, x)
    keys = x["keys"].copy()
    dup = {}
    for b in range(w.B):
        t0 = int(w.t0[b])
        Np = oracle.num_pooled(t0, 1, w.ratio)
        _, _, po = oracle.select_row(od, x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], t0, 0)
        if po == oracle.PATH_FLAT:
            lo, hi = 100, 600
        elif po == oracle.PATH_HISA:
            lo, hi = 640, min(2560, Np)
        else:
            continue
        sc = oracle.scores_of(od, x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], t0, 0, np.arange(Np, dtype=np.int32))
        keys[b, lo:hi] = x["keys"][b, int(np.argmax(sc))]
        dup[b] = (lo, hi)
    xx = dict(x)
    xx["keys"] = keys
    gk = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
    say(f"[run] decode with exact ties, {w.name}")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], gk, g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    In, bn, p = parity.to_np(I), parity.to_np(blk), parity.to_np(path)
    for b, (lo, hi) in dup.items():
        t0 = int(w.t0[b])
        Io, blko, po = oracle.select_row(od, xx["q_idx"][b, 0], xx["w"][b, 0], keys[b], t0, 0)
        assert p[b] == po, (b, p[b], po)
        parity.check_selection_row(od, xx, b, 0, In[b, 0], bn[b, 0], p[b], Io, blko, po)
        tied = lambda ids: set(i for i in ids.tolist() if lo <= i < hi)
        assert tied(In[b, 0]) == tied(Io), b
        assert len(tied(Io)) > 0
        if po == oracle.PATH_HISA:
            tb = lambda ids: set(i for i in ids.tolist() if lo // 64 <= i < -(-hi // 64))
            assert tb(bn[b, 0]) == tb(blko), b


def test_attention_split_merge_paths(hisa):
    # Few query rows split their 640-row lists over several workgroups whose
    # partial results a second kernel merges: three calls on one workspace
    # give bit-identical outputs that match the oracle; 6 sequences (16-head
    # workgroups, 10 splits) and 40 sequences (64-head workgroups, 4 splits)
    # match it on sampled rows.
    w = synth.FLASH_DECODE
    x, g = inputs(w, synth.SEEDS[w.name])
    I, _, _ = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    d = hisa.attention_dims(g["q"], g["local_kv"], g["pooled_kv"], I, ratio=w.ratio, window=w.window)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_ATTENTION, d), dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(3):
        say(f"[run] split attention on one workspace, call {rep}")
        outs.append(hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], I, g["sinks"], g["t0"],
                                                       ratio=w.ratio, window=w.window, ws=ws))
        torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    check_attention(w, x, I, outs[0])
    for wl, seed in ((MIXED, 5), (MIXED.with_(name="mixed_b40", B=40, t0=[1200 + 337 * b for b in range(40)],
                                              Np_cap=5000), 8)):
        x, g = inputs(wl, seed)
        say(f"[run] attention split merge, {wl.name}")
        I, _, _ = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(wl))
        out = run_attention(hisa, wl, g, I)
        torch.cuda.synchronize()
        check_attention(wl, x, I, out, sample=12)


def test_invalid_sequence_outputs(hisa):
    x, g = inputs(MIXED, 5)
    w = MIXED
    g = dict(g)
    g["t0"] = g["t0"].clone()
    g["t0"][5] = 30000  # Np = 7500 > Np_cap = 5000
    say("[run] invalid t0 (Np > Np_cap)")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    Ip, _, pp = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    If = hisa.flat_topk_select(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=4, topk=512)
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    assert parity.to_np(path)[5] == hisa.PATH_INVALID and parity.to_np(pp)[5] == hisa.PATH_INVALID
    assert (parity.to_np(I)[5] == -1).all() and (parity.to_np(blk)[5] == -1).all()
    assert (parity.to_np(Ip)[5] == -1).all() and (parity.to_np(If)[5] == -1).all()
    assert (parity.to_np(out)[5] == 0).all()
    # the valid sequences are unaffected and prefill at L = 1 equals decode
    np.testing.assert_array_equal(np.sort(parity.to_np(I)[:5], -1), np.sort(parity.to_np(Ip)[:5], -1))


EARLY = synth.Workload("early_rows_prefill", B=2, L=800, ratio=1, window=128, topk=512, index_block=64,
                       index_keep=16, H_i=64, D_i=128, H=64, Dk=512, Dv=512, bf16=True, t0=[300, 70],
                       planted=0, Np_cap=1100)


def test_prefill_early_rows_and_small_t0(hisa):
    # t0 = 300, ratio 1: Np = 1100 (HiSA) but row j sees only 301 + j rows, so
    # rows j < 211 hold masked ids; t0 = 70 < window: short local streams and a
    # flat sequence (Np = 870).
    w = EARLY
    x, g = inputs(w, 9)
    say("[run] early-row prefill")
    I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert parity.to_np(path).tolist() == [hisa.PATH_HISA, hisa.PATH_FLAT]
    check_selection(w, x, I, blk, path, sample=60)
    In = parity.to_np(I)
    for j in (0, 100, 210, 211, 500):
        V = 301 + j
        vis = In[0, j][(In[0, j] >= 0) & (In[0, j] < V)]
        assert len(vis) == min(V, 512), (j, len(vis))
    say("[run] early-row attention")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    check_attention(w, x, I, out, sample=40)


ROWS = synth.Workload("rows_prefill_b4_l53", B=4, L=53, ratio=4, window=128, topk=64, index_block=8,
                      index_keep=10, H_i=64, D_i=128, H=64, Dk=512, Dv=512, bf16=True,
                      t0=[20000, 3000, 264, 200], planted=0, Np_cap=5016)


def test_prefill_rows_small_blocks_mixed_paths(hisa):
    # The one-row-per-wave batched selection (B * L = 212 rows, past the
    # cached-means kernels' share) with index_block 8 and keep 10: C = 80
    # candidates (a partial 16-row tile and a partial 64-entry key row), nb up
    # to 626 blocks, L = 53 (the last workgroup holds one row), and one
    # sequence on each of the HiSA / flat (Np = 79) / dense (Np = 63) paths.
    w = ROWS
    x, g = inputs(w, 11)
    say("[run] small-block prefill")
    hisa.hisa_profile_enable(True)
    try:
        I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
        torch.cuda.synchronize()
        names = set(hisa.hisa_profile_collect())
    finally:
        hisa.hisa_profile_enable(False)
    assert "select_rows" in names, names
    assert parity.to_np(path).tolist() == [hisa.PATH_HISA, hisa.PATH_HISA, hisa.PATH_FLAT, hisa.PATH_DENSE]
    check_selection(w, x, I, blk, path)
    Bk = parity.to_np(blk)
    assert (Bk[2:] == -1).all() and (Bk[:2] >= 0).all()
    assert (np.diff(Bk[:2], axis=-1) > 0).all()  # retained blocks ascending
    In = parity.to_np(I)
    assert (np.diff(In[:3], axis=-1) > 0).all()  # ids ascending, k = 64 of each visible prefix
    np.testing.assert_array_equal(In[3], np.broadcast_to(np.r_[np.arange(63), -np.ones(1, int)], (53, 64)))


def test_attention_masks_window0_no_sinks(hisa):
    w = synth.FLASH_DECODE.with_(name="flash_b3_window0", B=3, t0=[65536, 40000, 9000], window=0, sinks=False,
                                 planted=0, Np_cap=16384)
    x, g = inputs(w, 11)
    rng = np.random.default_rng(3)
    kI = 300
    Iw = np.stack([rng.choice(int(n), kI, replace=False) for n in x["Np"]])[:, None, :].astype(np.int32)
    Iw[:, :, :17] = -1
    Iw[:, :, 17:30] = x["Np"][:, None, None] + 5      # invisible ids
    Ig = torch.from_numpy(Iw).to("cuda")
    say("[run] attention window 0, no sinks, masked ids")
    out = hisa.sparse_local_pooled_attention(g["q"], None, g["pooled_kv"], Ig, None, g["t0"], ratio=4, window=0)
    torch.cuda.synchronize()
    d = odims(w, x)
    o = parity.to_np(out)
    for b in range(3):
        ref = oracle.combine_row(d, x["q"][b, 0], np.zeros((1, w.Dk), np.float32), x["pooled_kv"][b], Iw[b, 0], None,
                                 int(x["t0"][b]), 0)
        assert parity.max_abs(o[b, 0], ref) <= 2e-2


def test_generic_kernels_prefill_f32(hisa):
    # f32 inputs take the VALU kernels; L > 1 with a tail block and ragged t0.
    w = synth.TINY_DECODE.with_(name="tiny_prefill_f32", B=2, L=37, t0=[4000, 2500], Np_cap=1100, planted=3)
    x, g = inputs(w, 13)
    say("[run] generic prefill selection")
    I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    check_selection(w, x, I, blk, path)
    say("[run] generic attention")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    check_attention(w, x, I, out)
    If = hisa.flat_topk_select(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio, topk=w.topk)
    torch.cuda.synchronize()
    d = odims(w, x, force_flat=1)
    In = parity.to_np(If)
    for b in range(2):
        for j in (0, 17, 36):
            Io, _, _ = oracle.select_row(d, x["q_idx"][b, j], x["w"][b, j], x["keys"][b], int(x["t0"][b]), j)
            parity.compare_sets(In[b, j], Io, lambda ids: oracle.scores_of(d, x["q_idx"][b, j], x["w"][b, j],
                                                                           x["keys"][b], int(x["t0"][b]), j, ids))


@pytest.mark.parametrize("shape", ["wide_rows", "odd_width", "many_index_heads"])
def test_generic_kernels_shapes_f32(hisa, shape):
    # f32 VALU kernels off the tiny shape: rows wider than a workgroup
    # (Dk = Dv = 300: one thread per value column, and a dot-product tail past
    # the 16-wide steps), a value width that does not divide 256 (96), and
    # more than 64 indexer heads (block scores from block means of the keys).
    kw = {"wide_rows": dict(H=3, Dk=300, Dv=300),
          "odd_width": dict(H=5, Dk=96, Dv=96),
          "many_index_heads": dict(H_i=72, D_i=20, index_block=8)}[shape]
    w = synth.TINY_DECODE.with_(name="generic_" + shape, B=2, L=1, t0=[4000, 2600], Np_cap=1000, planted=3, **kw)
    x, g = inputs(w, 19)
    say(f"[run] generic decode selection {shape}")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    check_selection(w, x, I, blk, path)
    say(f"[run] generic attention {shape}")
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    check_attention(w, x, I, out)


def test_dense_equivalence(hisa):
    # HiSA issue, Validation: with every pooled row selected (k == Np) the
    # sparse combine equals dense local + pooled attention.
    w = synth.FLASH_DECODE.with_(name="dense_np400", t0=[1600], planted=0, Np_cap=400)
    x, g = inputs(w, 17)
    I, _, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert parity.to_np(path)[0] == hisa.PATH_DENSE
    In = parity.to_np(I)
    np.testing.assert_array_equal(In[0, 0, :400], np.arange(400))
    assert (In[0, 0, 400:] == -1).all()
    out = run_attention(hisa, w, g, I)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(400).astype(np.int32)[None, None]).to("cuda")
    out2 = hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], perm, g["sinks"], g["t0"],
                                              ratio=4, window=128)
    torch.cuda.synchronize()
    check_attention(w, x, I, out)
    assert parity.max_abs(parity.to_np(out2), parity.to_np(out)) <= 2e-2
