"""Edge cases of the HIP library against the CPU oracle, through the C ABI:
no pooled rows at all (local-only attention), ratio-128 layers (dense pooled
lists and HiSA on a long ratio-128 stream), a ratio that is not a power of
two, value rows narrower than key rows (Dv < Dk), HiSA blocks of 8, 16 and 32
rows on both decode scans, a 1024-sequence streaming decode scan, the dense
fallback switch, a decode step replayed from a captured HIP graph, and the
flat top-k's coarse-bin path (including samples that mislead it)."""
import sys

import numpy as np
import pytest

import oracle
from tests import parity
from tests.test_gpu_parity import (EARLY, MIXED, MIXED_STREAM, ROWS, check_attention, check_selection, counter_bytes,
                                   inputs, odims, run_attention, sel_kw)
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
    h.lib()
    return h


def selection_then_attention(hisa, w, x, g, prefill, sample=None, att_sample=None):
    fn = hisa.hisa_select_prefill if prefill else hisa.hisa_select_decode
    I, blk, path = fn(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    check_selection(w, x, I, blk, path, sample=sample)
    out = hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], I, g["sinks"], g["t0"],
                                             ratio=w.ratio, window=w.window, Dv=w.Dv)
    torch.cuda.synchronize()
    say(f"  attention max-abs {check_attention(w, x, I, out, sample=att_sample):.3g}")
    return parity.to_np(I), parity.to_np(path)


# ---------------------------------------------------------------- no pooled rows

NP0 = synth.Workload("np0_local_only", B=3, L=1, ratio=4, window=128, topk=512, index_block=64, index_keep=16,
                     H_i=64, D_i=128, H=64, Dk=512, Dv=512, bf16=True, t0=[2, 0, 70], planted=0, Np_cap=64)


def test_no_pooled_rows_decode(hisa):
    # HiSA issue, Consuming the selection, branch 1 (Np == 0): the selector
    # lists nothing and the combine attends to the local window alone
    # (t0 = 2 and 0: Np = 0 with 3 and 1 local rows; t0 = 70: Np = 17, dense).
    w = NP0
    x, g = inputs(w, 41)
    say("[run] decode with Np = 0")
    I, path = selection_then_attention(hisa, w, x, g, prefill=False)
    assert path.tolist() == [hisa.PATH_DENSE] * 3
    assert (I[:2] == -1).all()
    np.testing.assert_array_equal(I[2, 0, :17], np.arange(17))


def test_no_pooled_rows_prefill(hisa):
    # t0 = 0, L = 16, ratio 4: Np = 4, and rows 0..2 see no pooled row yet.
    w = NP0.with_(name="np0_prefill", B=2, L=16, t0=[0, 5])
    x, g = inputs(w, 42)
    say("[run] prefill whose first rows see no pooled row")
    I, path = selection_then_attention(hisa, w, x, g, prefill=True)
    assert path.tolist() == [hisa.PATH_DENSE] * 2


# ---------------------------------------------------------------- ratio 128 and ratio 3

def test_ratio128_layers(hisa):
    # DeepSeek-V4's ratio-128 layers (HiSA issue, Dependency): Np = 512 at
    # t0 = 65536 (dense: I = iota), Np = 1093 at t0 = 140000 (HiSA), Np = 0 at
    # t0 = 100; then a 256-row prefill chunk on the dense branch.
    w = synth.FLASH_DECODE.with_(name="ratio128_decode_b3", B=3, ratio=128, t0=[65536, 140000, 100], planted=4,
                                 Np_cap=1100)
    x, g = inputs(w, 43)
    say("[run] ratio-128 decode")
    I, path = selection_then_attention(hisa, w, x, g, prefill=False)
    assert path.tolist() == [hisa.PATH_DENSE, hisa.PATH_HISA, hisa.PATH_DENSE]
    np.testing.assert_array_equal(I[0, 0], np.arange(512))
    w = synth.PREFILL.with_(name="ratio128_prefill_l256", L=256, ratio=128, t0=[65000], Np_cap=512)
    x, g = inputs(w, 44)
    say("[run] ratio-128 prefill (dense pooled list, rows see 507..509)")
    I, path = selection_then_attention(hisa, w, x, g, prefill=True, sample=24, att_sample=24)
    assert path.tolist() == [hisa.PATH_DENSE]
    np.testing.assert_array_equal(I[0], np.broadcast_to(np.r_[np.arange(509), -np.ones(3, int)], (256, 512)))


def test_ratio3_division(hisa):
    # A ratio that is not a power of two takes the division in the pooled
    # count and the visibility: Np = 16384 (HiSA) and 1000 (flat) in decode,
    # 10021 (HiSA) and 521 (flat) in a 64-row prefill.
    w = synth.FLASH_DECODE.with_(name="ratio3_decode_b2", B=2, ratio=3, t0=[49152, 3000], planted=8, Np_cap=16384)
    x, g = inputs(w, 45)
    say("[run] ratio-3 decode")
    _, path = selection_then_attention(hisa, w, x, g, prefill=False)
    assert path.tolist() == [hisa.PATH_HISA, hisa.PATH_FLAT]
    w = synth.PREFILL.with_(name="ratio3_prefill_b2_l64", B=2, L=64, ratio=3, t0=[30000, 1500], Np_cap=10100)
    x, g = inputs(w, 46)
    say("[run] ratio-3 prefill")
    _, path = selection_then_attention(hisa, w, x, g, prefill=True, sample=32, att_sample=16)
    assert path.tolist() == [hisa.PATH_HISA, hisa.PATH_FLAT]


# ---------------------------------------------------------------- Dv < Dk

@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_value_narrower_than_key(hisa, bf16):
    # MLA-style rows: 576-wide keys whose first 512 entries are the value.
    w = MIXED.with_(name="dv512_dk576", B=2, L=3, H=16, Dk=576, Dv=512, t0=[20000, 9000], bf16=bf16, planted=2)
    x, g = inputs(w, 47)
    say(f"[run] attention Dk 576 / Dv 512 ({'bf16' if bf16 else 'f32'})")
    selection_then_attention(hisa, w, x, g, prefill=True)


# ---------------------------------------------------------------- small HiSA blocks

@pytest.mark.parametrize("block,keep", [(1, 512), (2, 256), (4, 128), (8, 64), (16, 32), (32, 16)])
@pytest.mark.parametrize("scan", ["latency", "streaming"])
def test_decode_small_blocks(hisa, block, keep, scan):
    # index_block below 64 on the bf16 MFMA decode scans: blocks of <= 16 rows
    # are summed across the lanes of one wave, 32-row blocks across two waves.
    # index_block * index_keep = 512 = topk keeps the HiSA path.  Latency scan:
    # one sequence of 256 slabs; streaming: 5 sequences of up to 256 slabs.
    # (Blocks of 16 and 32 rows keep the selection fused into both scans; with
    # more than 64 kept blocks the selection runs in a launch of its own.)
    if scan == "latency":
        w = synth.FLASH_DECODE.with_(name=f"flash_b{block}", index_block=block, index_keep=keep, planted=24)
        seed = 48
    else:
        w = MIXED_STREAM.with_(name=f"stream_b{block}", B=5, t0=[65000, 16400, 40000, 30000, 5000], Np_cap=16384,
                               index_block=block, index_keep=keep, planted=24, H=4, Dk=64, Dv=64)
        seed = 49
    x, g = inputs(w, seed)
    say(f"[run] {scan} decode scan with index_block {block}, keep {keep}")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_HISA).all()
    check_selection(w, x, I, blk, path)


# ---------------------------------------------------------------- 1024 sequences

def test_decode_stream_b1024(hisa):
    # The streaming scan's largest batch: 1024 sequences of 1025..1100 pooled
    # rows (about 18000 slabs).  The end of the last sequence's slab list sits
    # past every thread's four sequences of the prefix table.
    rng = np.random.default_rng(50)
    t0 = [int(v) for v in rng.integers(4100, 4400, size=1024)]
    w = MIXED.with_(name="stream_b1024", B=1024, t0=t0, Np_cap=1100, planted=2, H=4, Dk=64, Dv=64)
    x, g = inputs(w, 51)
    d = hisa.selection_dims(g["q_idx"], g["keys"], ratio=4, topk=512, index_block=64, index_keep=16)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d), dtype=torch.uint8, device="cuda")
    say("[run] streaming decode scan, B = 1024")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w), ws=ws)
    torch.cuda.synchronize()
    assert (parity.to_np(path) == hisa.PATH_HISA).all()
    rows = sorted({(0, 0), (1023, 0), (511, 0)} | {(int(b), 0) for b in rng.choice(1024, 45, replace=False)})
    check_selection(w, x, I, blk, path, rows=rows)
    assert (ws[: counter_bytes(w)].view(torch.int32) == 0).all()


# ---------------------------------------------------------------- dense fallback switch

def test_force_dense_switch(hisa):
    # HiSA issue, Implementation plan item 1: with the indexer off, every row
    # lists all pooled rows (the index width is the pooled capacity) and the
    # combine is dense attention over the window and every visible pooled row.
    w = synth.FLASH_DECODE.with_(name="flash_force_dense", B=2, t0=[65536, 20000], planted=0, Np_cap=16384,
                                 topk=16384)
    x, g = inputs(w, 52)
    say("[run] decode, dense fallback")
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w, mode=2))
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    In = parity.to_np(I)
    assert (parity.to_np(path) == hisa.PATH_DENSE).all() and (parity.to_np(blk) == -1).all()
    for b, Np in enumerate(x["Np"].tolist()):
        np.testing.assert_array_equal(In[b, 0], np.r_[np.arange(Np), -np.ones(16384 - Np, int)])
    say(f"  attention max-abs {check_attention(w, x, I, out):.3g}")
    w = EARLY.with_(name="early_force_dense", topk=1100)
    x, g = inputs(w, 53)
    say("[run] prefill, dense fallback")
    I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w, mode=2))
    out = run_attention(hisa, w, g, I)
    torch.cuda.synchronize()
    d = odims(w, x)
    d.force_dense = 1
    Io, blko, po = oracle.select(d, x["q_idx"], x["w"], x["keys"], x["t0"])
    np.testing.assert_array_equal(parity.to_np(I), Io)
    assert (parity.to_np(path) == hisa.PATH_DENSE).all() and (parity.to_np(blk) == -1).all()
    say(f"  attention max-abs {check_attention(w, x, I, out, sample=24):.3g}")


# ---------------------------------------------------------------- HIP graph replay

def test_decode_step_graph_replay(hisa):
    # The two calls of a decode step captured once into a HIP graph (outputs
    # and workspaces allocated beforehand, the selection's counters zeroed
    # before capture) and replayed three times, with eager work and a
    # synchronisation between replays: every replay equals the eager step.
    w = synth.FLASH_DECODE
    x, g = inputs(w, synth.SEEDS[w.name])
    dev = torch.device("cuda")
    sd = hisa.selection_dims(g["q_idx"], g["keys"], ratio=w.ratio, topk=w.topk, index_block=w.index_block,
                             index_keep=w.index_keep)
    ws_sel = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE, sd), dtype=torch.uint8, device=dev)
    I = torch.empty((1, 1, w.topk), dtype=torch.int32, device=dev)
    blk = torch.empty((1, 1, w.index_keep), dtype=torch.int32, device=dev)
    path = torch.empty((1,), dtype=torch.int32, device=dev)
    ad = hisa.attention_dims(g["q"], g["local_kv"], g["pooled_kv"], I, ratio=w.ratio, window=w.window)
    ws_att = torch.zeros(max(hisa.workspace_bytes(hisa.OP_ATTENTION, ad), 256), dtype=torch.uint8, device=dev)
    out = torch.empty((1, 1, w.H, w.Dv), dtype=torch.bfloat16, device=dev)

    def step():
        hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w), I=I, top_blk=blk, path=path,
                                ws=ws_sel)
        hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], I, g["sinks"], g["t0"],
                                           ratio=w.ratio, window=w.window, out=out, ws=ws_att)

    say("[run] eager decode step")
    step()
    torch.cuda.synchronize()
    I_ref, out_ref = I.clone(), out.clone()
    check_attention(w, x, I_ref, out_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say("[run] capture")
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        I.fill_(-7)
        out.fill_(0.5)
        torch.cuda.synchronize()
        say(f"[run] replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(I, I_ref), rep
        assert torch.equal(out, out_ref), rep
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(I, I_ref) and torch.equal(out, out_ref)
    assert (ws_sel[: counter_bytes(w.with_(Np_cap=int(x["Np_cap"])))].view(torch.int32) == 0).all()


# ---------------------------------------------------------------- dense attention (no index list)

@pytest.mark.parametrize("case", ["ratio128_decode", "ratio128_prefill", "ratio4_decode_b2"])
def test_dense_attention_without_index_list(hisa, case):
    # I = NULL: every visible pooled row (the sparse combine's dense branch and
    # the ratio-128 layers, which have no indexer).  Against the oracle with
    # the list 0..Np_cap-1 (it masks ids at or past V(t)), and equal to the
    # attention over the dense fallback's index list.
    w = {"ratio128_decode": synth.FLASH_DECODE.with_(name="r128_dense_b3", B=3, ratio=128,
                                                     t0=[65536, 140000, 100], planted=0, Np_cap=1100),
         "ratio128_prefill": synth.PREFILL.with_(name="r128_dense_prefill", L=256, ratio=128, t0=[65000],
                                                 Np_cap=512),
         "ratio4_decode_b2": synth.FLASH_DECODE.with_(name="flash_dense_b2", B=2, t0=[16000, 9000], planted=0,
                                                      Np_cap=4000)}[case]
    x, g = inputs(w, 58)
    say(f"[run] dense attention, no index list, {w.name}")
    out = hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], None, g["sinks"], g["t0"],
                                             ratio=w.ratio, window=w.window)
    torch.cuda.synchronize()
    Np_cap = int(x["Np_cap"])
    full = torch.from_numpy(np.broadcast_to(np.arange(Np_cap, dtype=np.int32), (w.B, w.L, Np_cap)).copy())
    say(f"  max-abs {check_attention(w, x, full, out, sample=24):.3g}")
    Id, _, _ = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"],
                                        **sel_kw(w.with_(topk=Np_cap), mode=2))
    out2 = run_attention(hisa, w, g, Id)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


# ---------------------------------------------------------------- local window as a ring

def ring_from_linear(x, w, R, slot0):
    """The ring layout of the linear local rows: position s in slot (slot0[b] + s - t0[b]) mod R; every other
    slot NaN (never read)."""
    lin = x["local_kv"]
    ring = np.full((w.B, R, lin.shape[2]), np.nan, np.float32)
    for b in range(w.B):
        t0 = int(x["t0"][b])
        ls = max(0, t0 - w.window + 1)
        for s in range(ls, t0 + w.L):
            ring[b, (slot0[b] + s - t0) % R] = lin[b, s - ls]
    return ring


@pytest.mark.parametrize("case", ["decode_ring_is_window", "verify_l4", "prefill_l37_b4", "f32_generic"])
def test_ring_window_equals_linear(hisa, case):
    w = {"decode_ring_is_window": synth.FLASH_DECODE.with_(name="ring_flash", B=2, t0=[65536, 100], planted=4,
                                                           Np_cap=16384),
         "verify_l4": synth.FLASH_DECODE.with_(name="ring_verify_l4", B=3, L=4, t0=[65000, 5000, 60], planted=4,
                                               Np_cap=16384),
         "prefill_l37_b4": ROWS,
         "f32_generic": synth.TINY_DECODE.with_(name="ring_tiny_f32", B=2, L=5, t0=[4000, 70], Np_cap=1100,
                                                planted=2)}[case]
    x, g = inputs(w, 61)
    R = w.window + w.L - 1 + (0 if case == "decode_ring_is_window" else 19)
    rng = np.random.default_rng(62)
    slot0 = rng.integers(0, R, size=w.B).astype(np.int32)
    dt = torch.bfloat16 if w.bf16 else torch.float32
    ring = torch.from_numpy(ring_from_linear(x, w, R, slot0)).to("cuda").to(dt).contiguous()
    say(f"[run] selection + ring attention, {w.name}, {R} slots")
    fn = hisa.hisa_select_prefill if w.L > 1 else hisa.hisa_select_decode
    I, _, _ = fn(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    out_lin = run_attention(hisa, w, g, I)
    s0 = torch.from_numpy(slot0).to("cuda")
    out_ring = hisa.sparse_local_pooled_attention_ring(g["q"], ring, g["pooled_kv"], I, g["sinks"], g["t0"], s0,
                                                       ratio=w.ratio, window=w.window)
    torch.cuda.synchronize()
    assert torch.equal(out_ring, out_lin)
    say(f"  max-abs {check_attention(w, x, I, out_ring, sample=24):.3g}")
    # the default slot of position t0 is t0 mod Wl_cap
    ring2 = torch.from_numpy(ring_from_linear(x, w, R, (x["t0"] % R).astype(np.int32))).to("cuda").to(dt)
    out2 = hisa.sparse_local_pooled_attention_ring(g["q"], ring2.contiguous(), g["pooled_kv"], I, g["sinks"],
                                                   g["t0"], None, ratio=w.ratio, window=w.window)
    # a slot outside the ring: that sequence is not computed
    bad = s0.clone()
    bad[0] = R
    out3 = hisa.sparse_local_pooled_attention_ring(g["q"], ring, g["pooled_kv"], I, g["sinks"], g["t0"], bad,
                                                   ratio=w.ratio, window=w.window)
    torch.cuda.synchronize()
    assert torch.equal(out2, out_lin)
    assert (out3[0] == 0).all() and torch.equal(out3[1:], out_lin[1:])


# ---------------------------------------------------------------- flat top-k of long rows

@pytest.mark.parametrize("case", ["ragged_b4", "heavy_ties"])
def test_flat_topk_long_rows_decode(hisa, case):
    # Decode rows of up to 32768 scores: a ragged batch (rows of 32768,
    # 20001, 9001 and 5000 scores) and 3000 equal top scores straddling the
    # k-th (the best key row copied over rows 1000..3999 of sequence 0: the
    # 2048 kept must be the lowest ids).
    w = {"ragged_b4": synth.DSA_DECODE.with_(name="dsa_decode_b4", B=4, t0=[32767, 20000, 9000, 4999], H=4, Dk=64,
                                             Dv=64),
         "heavy_ties": synth.DSA_DECODE.with_(name="dsa_decode_ties", B=2, t0=[32767, 15000], H=4, Dk=64,
                                              Dv=64)}[case]
    x, g = inputs(w, 65)
    x = dict(x)
    keys = x["keys"]
    if case == "heavy_ties":
        keys = keys.copy()
        d0 = odims(w, x)
        sc = oracle.scores_of(d0, x["q_idx"][0, 0], x["w"][0, 0], x["keys"][0], int(x["t0"][0]), 0,
                              np.arange(32768, dtype=np.int32))
        keys[0, 1000:4000] = x["keys"][0, int(np.argmax(sc))]
        x["keys"] = keys
    gk = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
    say(f"[run] flat top-k of long decode rows, {case}")
    I = hisa.flat_topk_select(g["q_idx"], g["w"], gk, g["t0"], ratio=1, topk=w.topk)
    torch.cuda.synchronize()
    d = odims(w, x)
    In = parity.to_np(I)
    for b in range(w.B):
        q, ww, kb, t0 = x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], int(x["t0"][b])
        Io, _, _ = oracle.select_row(d, q, ww, kb, t0, 0)
        parity.compare_sets(In[b, 0], Io, lambda ids: oracle.scores_of(d, q, ww, kb, t0, 0, ids), what=f"({b},0)")
        v = In[b, 0][In[b, 0] >= 0]
        assert (np.diff(v) > 0).all()
        if case == "heavy_ties" and b == 0:
            np.testing.assert_array_equal(v, np.arange(1000, 3048))



# ---------------------------------------------------------------- the flat top-k's coarse-bin path

@pytest.mark.parametrize("case", ["ragged_b2", "sample_misleads", "one_coarse_bin", "retry_one_bin"])
def test_flat_topk_coarse_bin_path(hisa, case):
    # Rows of 8193..32768 scores: the row top-k takes the coarse key bin (top
    # 8 key bits) of the k-th key from one sample per thread (scores 0, 32,
    # 64, ...), checks it with its own counts and moves it up or down (three
    # tries) before falling back to the exact path.  A ragged batch (rows of
    # 32768 and 9001 scores); samples that mislead (the best key copied onto
    # 300 sampled rows of sequence 0, so the sample puts the k-th key in the
    # top bin: the tries move down, then the exact path takes over); rows
    # whose scores are all equal (one coarse bin holds every key: 32768 and
    # 9001 ties, the lowest 2048 ids kept); and rows built so that the first
    # guess is one bin too high: every head's q is one unit vector u, every
    # head weight 1 and key row i is a_i u, so the score is about 0.71 a_i;
    # the sampled rows and 1000 others score in [2, 8), one coarse bin, all
    # the rest in [0.5, 2), the bin below, so the sample names the upper bin,
    # which holds fewer than k entries, and one move down finds the k-th key.
    # A repeated call is identical.
    w = synth.DSA_DECODE.with_(name=f"dsa_decode_coarse_{case}", B=2, t0=[32767, 9000], H=4, Dk=64, Dv=64)
    x, g = inputs(w, 77)
    x = dict(x)
    gk = g["keys"]
    if case == "retry_one_bin":
        rng = np.random.default_rng(9)
        u = rng.standard_normal(128).astype(np.float32)
        u /= np.linalg.norm(u)
        q_idx = np.repeat(synth.round_bf16(u)[None, None, None, :], 64, axis=2).repeat(w.B, axis=0)
        keys = np.empty_like(x["keys"])
        high = []
        for b in range(w.B):
            n_b = int(x["Np"][b])
            a = rng.uniform(0.8, 2.7, keys.shape[1]).astype(np.float32)
            hi = np.zeros(keys.shape[1], dtype=bool)
            hi[0:n_b:32] = True
            hi[rng.choice(np.flatnonzero(~hi[:n_b]), 1000, replace=False)] = True
            a[hi] = rng.uniform(3.0, 10.0, int(hi.sum())).astype(np.float32)
            keys[b] = synth.round_bf16(a[:, None] * u[None, :])
            high.append(np.flatnonzero(hi[:n_b]))
            assert len(high[b]) < w.topk
        x["q_idx"], x["w"], x["keys"] = q_idx.astype(np.float32), np.ones_like(x["w"]), keys
        gq = torch.from_numpy(x["q_idx"]).to("cuda").to(torch.bfloat16).contiguous()
        gw = torch.from_numpy(x["w"]).to("cuda")
        gk = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
        g = dict(g, q_idx=gq, w=gw)
    elif case != "ragged_b2":
        keys = x["keys"].copy()
        if case == "sample_misleads":
            d0 = odims(w, x)
            sc = oracle.scores_of(d0, x["q_idx"][0, 0], x["w"][0, 0], x["keys"][0], int(x["t0"][0]), 0,
                                  np.arange(32768, dtype=np.int32))
            keys[0, 0:9600:32] = x["keys"][0, int(np.argmax(sc))]
        else:
            keys[0, :] = keys[0, 5]
            keys[1, :] = keys[1, 7]
        x["keys"] = keys
        gk = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
    say(f"[run] flat top-k, coarse-bin path: {case}")
    I1 = hisa.flat_topk_select(g["q_idx"], g["w"], gk, g["t0"], ratio=1, topk=w.topk)
    I2 = hisa.flat_topk_select(g["q_idx"], g["w"], gk, g["t0"], ratio=1, topk=w.topk)
    torch.cuda.synchronize()
    assert torch.equal(I1, I2)
    d = odims(w, x)
    In = parity.to_np(I1)
    for b in range(w.B):
        q, ww, kb, t0 = x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], int(x["t0"][b])
        Io, _, _ = oracle.select_row(d, q, ww, kb, t0, 0)
        parity.compare_sets(In[b, 0], Io, lambda ids: oracle.scores_of(d, q, ww, kb, t0, 0, ids), what=f"({b},0)")
        v = In[b, 0][In[b, 0] >= 0]
        assert len(v) == w.topk and (np.diff(v) > 0).all()
        if case == "one_coarse_bin":
            np.testing.assert_array_equal(v, np.arange(w.topk))
        if case == "sample_misleads" and b == 0:
            assert set(range(0, 9600, 32)) <= set(v.tolist())  # the 300 copies of the best key are kept
        if case == "retry_one_bin":
            assert set(high[b].tolist()) <= set(v.tolist())  # every row of the upper bin, then the best below
