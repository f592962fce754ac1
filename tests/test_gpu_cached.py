"""Decode selection on cached block means (hisa_select_decode_cached) and the
cache update (hisa_block_means_update) against the CPU oracle, through the C
ABI: the V4-Flash decode step and the ragged batch, mixed dense / flat / HiSA /
invalid sequences, exact ties, steps that complete a block (the call writes
the new mean into the cache and leaves the others alone), and the cache's
contents against the oracle's block means."""
import sys

import numpy as np
import pytest

import oracle
from tests import parity
from tests.test_gpu_parity import MIXED, MIXED_STREAM, check_selection, inputs, odims, sel_kw
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


def full_cache(hisa, w, g):
    """A cache holding every complete block of each sequence at its t0."""
    _, rep = hisa.hisa_block_scores(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio,
                                    index_block=w.index_block, want_rep=True)
    return rep


@pytest.mark.parametrize("case", ["flash", "batched", "mixed", "mixed_stream"])
def test_cached_decode_matches_oracle(hisa, case):
    w, seed = {"flash": (synth.FLASH_DECODE, synth.SEEDS[synth.FLASH_DECODE.name]),
               "batched": (synth.BATCHED_DECODE, synth.SEEDS[synth.BATCHED_DECODE.name]),
               "mixed": (MIXED, 5), "mixed_stream": (MIXED_STREAM, 21)}[case]
    x, g = inputs(w, seed)
    rep = full_cache(hisa, w, g)
    rep0 = rep.clone()
    say(f"[run] cached decode selection, {w.name}")
    I, blk, path = hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    p = parity.to_np(path)
    ref_paths = [oracle.gate(odims(w, x), int(n)) for n in x["Np"]]
    assert p.tolist() == ref_paths
    check_selection(w, x, I, blk, path)
    # the blocks the cache already held are untouched; only the block this
    # step's token completes (if any) was rewritten, with the same mean
    nb = x["Np"] // w.index_block
    first_new = (x["t0"] // w.ratio) // w.index_block
    for b in range(w.B):
        assert torch.equal(rep[b, :first_new[b]], rep0[b, :first_new[b]])
        if nb[b] > first_new[b] and ref_paths[b] == oracle.PATH_HISA:
            np.testing.assert_allclose(parity.to_np(rep[b, first_new[b]:nb[b]]),
                                       parity.to_np(rep0[b, first_new[b]:nb[b]]), rtol=1e-6, atol=1e-7)
    say("[run] stateless decode selection for comparison")
    Is, _, ps = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    assert torch.equal(ps, path)
    same = (np.sort(parity.to_np(Is), -1) == np.sort(parity.to_np(I), -1)).mean()
    say(f"  ids equal to the stateless path: {same:.5f}")


def cached_counter_bytes(w):
    """The cached selection's counter region: per query row a coarse counter
    and its group counters (16 coarse workgroups of 16 blocks to a group) and a
    fine counter, one 64-byte line each, then the error line and 16 descriptor
    words per row."""
    rows = w.B * w.L
    wgs = -(-(w.Np_cap // w.index_block) // 16)
    groups = -(-wgs // 16)
    return rows * (1 + groups) * 64 + rows * 64 + 64 + rows * 16 * 8


@pytest.mark.parametrize("block,keep", [(8, 64), (16, 64), (32, 32)])
def test_cached_decode_small_blocks(hisa, block, keep):
    # Blocks of 8 rows take the two-launch form (eight block ids per 64
    # candidates do not fit one descriptor word); blocks of 16 and 32 the
    # one-launch form, four and two kept blocks per descriptor word.  Two
    # calls on one workspace: its counters, error word and descriptors are
    # back to zero after each.
    w = synth.FLASH_DECODE.with_(name=f"flash_cached_b{block}", B=2, t0=[65536, 30001], Np_cap=16384,
                                 index_block=block, index_keep=keep, planted=24)
    x, g = inputs(w, 77)
    rep = full_cache(hisa, w, g)
    d = hisa.selection_dims(g["q_idx"], g["keys"], **sel_kw(w))
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE_CACHED, d), dtype=torch.uint8, device="cuda")
    nbytes = cached_counter_bytes(w)
    for call in range(2):
        say(f"[run] cached decode, blocks of {block}, call {call}")
        I, blk, path = hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, g["t0"], **sel_kw(w),
                                                      ws=ws)
        torch.cuda.synchronize()
        assert parity.to_np(path).tolist() == [hisa.PATH_HISA, hisa.PATH_HISA]
        check_selection(w, x, I, blk, path)
        assert (ws[:nbytes].view(torch.int32) == 0).all()


def test_cached_decode_graph_replay(hisa):
    # The one-launch cached selection of the B = 32 ragged batch captured once
    # into a HIP graph (outputs, cache and workspace allocated beforehand) and
    # replayed three times with eager calls and synchronisations between
    # replays: every replay equals the eager call, the blocks it completes are
    # rewritten with the same means, and the workspace words end at zero.
    w = synth.BATCHED_DECODE
    x, g = inputs(w, synth.SEEDS[w.name])
    dev = torch.device("cuda")
    rep = full_cache(hisa, w, g)
    d = hisa.selection_dims(g["q_idx"], g["keys"], **sel_kw(w))
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE_CACHED, d), dtype=torch.uint8, device=dev)
    I = torch.empty((w.B, 1, w.topk), dtype=torch.int32, device=dev)
    blk = torch.empty((w.B, 1, w.index_keep), dtype=torch.int32, device=dev)
    path = torch.empty((w.B,), dtype=torch.int32, device=dev)

    def call():
        hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, g["t0"], **sel_kw(w), I=I, top_blk=blk,
                                       path=path, ws=ws)

    say("[run] eager cached selection")
    call()
    torch.cuda.synchronize()
    check_selection(w, x, I, blk, path)
    I_ref, blk_ref, path_ref, rep_ref = I.clone(), blk.clone(), path.clone(), rep.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say("[run] capture")
    with torch.cuda.graph(graph, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        I.fill_(-7)
        blk.fill_(-7)
        path.fill_(-7)
        torch.cuda.synchronize()
        say(f"[run] replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(I, I_ref) and torch.equal(blk, blk_ref) and torch.equal(path, path_ref), r
        assert torch.equal(rep, rep_ref), r
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(I, I_ref)
    assert (ws[:cached_counter_bytes(w.with_(Np_cap=int(x["Np_cap"])))].view(torch.int32) == 0).all()


def test_cached_decode_exact_ties(hisa):
    # The best row of each HiSA sequence copied over blocks 10..39, so the
    # coarse and the fine top-k both cut through exact ties; the lowest ids win
    # on both sides.
    w = MIXED
    x, g = inputs(w, 5)
    od = odims(w, x)
    keys = x["keys"].copy()
    for b in range(w.B):
        t0 = int(w.t0[b])
        Np = oracle.num_pooled(t0, 1, w.ratio)
        if oracle.gate(od, Np) != oracle.PATH_HISA:
            continue
        sc = oracle.scores_of(od, x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], t0, 0, np.arange(Np, dtype=np.int32))
        keys[b, 640:min(2560, Np)] = x["keys"][b, int(np.argmax(sc))]
    xx = dict(x)
    xx["keys"] = keys
    gg = dict(g)
    gg["keys"] = torch.from_numpy(keys).to("cuda").to(torch.bfloat16).contiguous()
    rep = full_cache(hisa, w, gg)
    say("[run] cached decode with exact ties")
    I, blk, path = hisa.hisa_select_decode_cached(gg["q_idx"], gg["w"], gg["keys"], rep, gg["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    In, bn = parity.to_np(I), parity.to_np(blk)
    for b in range(w.B):
        Io, blko, po = oracle.select_row(od, xx["q_idx"][b, 0], xx["w"][b, 0], keys[b], int(w.t0[b]), 0)
        parity.check_selection_row(od, xx, b, 0, In[b, 0], bn[b, 0], int(parity.to_np(path)[b]), Io, blko, po)
        if po == oracle.PATH_HISA:
            assert set(In[b, 0].tolist()) == set(Io.tolist()), b
            assert set(bn[b, 0].tolist()) == set(blko.tolist()), b


def test_cached_decode_steps_complete_a_block(hisa):
    # Decode steps at t0 = 65532 .. 65535 on the V4-Flash keys: the cache is
    # built by hisa_block_means_update for the first 65532 tokens (255 complete
    # blocks); the last step's token completes pooled row 16383 and with it
    # block 255, whose mean the selection computes and stores.
    w = synth.FLASH_DECODE
    x, g = inputs(w, synth.SEEDS[w.name])
    dev = torch.device("cuda")
    rep = torch.full((1, 256, 128), float("nan"), dtype=torch.float32, device=dev)
    say("[run] block means of the first 65532 tokens")
    hisa.hisa_block_means_update(g["keys"], torch.zeros(1, dtype=torch.int32, device=dev), rep, ratio=4,
                                 index_block=64, L=65532)
    torch.cuda.synchronize()
    _, rep_orc = oracle.block_scores(odims(w, x), x["q_idx"], x["w"], x["keys"], x["t0"])
    np.testing.assert_allclose(parity.to_np(rep[0, :255]), rep_orc[0, :255], rtol=1e-6, atol=1e-7)
    assert torch.isnan(rep[0, 255]).all()
    d = hisa.selection_dims(g["q_idx"], g["keys"], **sel_kw(w))
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE_CACHED, d), dtype=torch.uint8, device=dev)
    od = odims(w, x)
    for t0 in (65532, 65533, 65534, 65535):
        say(f"[run] cached decode at t0 = {t0}")
        before = rep.clone()
        tt = torch.tensor([t0], dtype=torch.int32, device=dev)
        I, blk, path = hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, tt, **sel_kw(w), ws=ws)
        torch.cuda.synchronize()
        xx = dict(x)
        xx["t0"] = np.array([t0], np.int32)
        Io, blko, po = oracle.select_row(od, x["q_idx"][0, 0], x["w"][0, 0], x["keys"][0], t0, 0)
        parity.check_selection_row(od, xx, 0, 0, parity.to_np(I)[0, 0], parity.to_np(blk)[0, 0],
                                   int(parity.to_np(path)[0]), Io, blko, po)
        assert torch.equal(rep[0, :255], before[0, :255])
        if t0 < 65535:  # Np = 16383: block 255 is not complete and stays untouched
            assert parity.to_np(I)[0, 0].max() < 255 * 64
            assert torch.isnan(rep[0, 255]).all()
    np.testing.assert_allclose(parity.to_np(rep[0, 255]), rep_orc[0, 255], rtol=1e-6, atol=1e-7)
    # the step's mean and the update call's mean are the same numbers
    rep2 = torch.zeros_like(rep)
    hisa.hisa_block_means_update(g["keys"], torch.zeros(1, dtype=torch.int32, device=dev), rep2, ratio=4,
                                 index_block=64, L=65536)
    torch.cuda.synchronize()
    assert torch.equal(rep2, rep)
    # counters, the error word (a hand-off never timed out) and the kept-block
    # descriptors of the one-launch form: all back to zero
    assert (ws[:2 * 64 + 64 + 64 + 16 * 8].view(torch.int32) == 0).all()


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_block_means_update_ragged(hisa, bf16):
    # A prefill chunk of 300 tokens (75 pooled rows) completes blocks
    # [floor(floor(t0/r)/b), floor(floor((t0+300)/r)/b)) of each sequence;
    # everything else keeps its value.
    w = MIXED.with_(name="means_update", bf16=bf16, index_block=16, t0=[1200, 2800, 4096, 6000, 19900, 16400],
                    L=1)
    x, g = inputs(w, 55)
    dev = torch.device("cuda")
    nb_cap = int(x["Np_cap"]) // 16
    rep = torch.full((w.B, nb_cap, w.D_i), -3.0, dtype=torch.float32, device=dev)
    t0 = torch.tensor([t - 299 for t in w.t0], dtype=torch.int32, device=dev)
    say(f"[run] block means update ({'bf16' if bf16 else 'f32'})")
    hisa.hisa_block_means_update(g["keys"], t0, rep, ratio=4, index_block=16, L=300)
    torch.cuda.synchronize()
    R = parity.to_np(rep)
    for b in range(w.B):
        t0b = w.t0[b] - 299
        lo = (t0b // 4) // 16
        hi = ((t0b + 300) // 4) // 16
        assert hi > lo, b
        mean = x["keys"][b, :hi * 16].astype(np.float64).reshape(hi, 16, w.D_i).mean(axis=1)
        np.testing.assert_allclose(R[b, lo:hi], mean[lo:hi], rtol=1e-6, atol=1e-7)
        assert (R[b, :lo] == -3.0).all() and (R[b, hi:] == -3.0).all()


def test_cached_decode_dense_switch_leaves_cache(hisa):
    w = synth.FLASH_DECODE.with_(name="flash_cached_dense", topk=16384, planted=0)
    x, g = inputs(w, 57)
    rep = full_cache(hisa, w, g)
    rep0 = rep.clone()
    I, blk, path = hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, g["t0"], **sel_kw(w, mode=2))
    torch.cuda.synchronize()
    assert torch.equal(rep, rep0)
    np.testing.assert_array_equal(parity.to_np(I)[0, 0], np.arange(16384))
    assert parity.to_np(path)[0] == hisa.PATH_DENSE


VERIFY = synth.Workload("verify_b4_l8", B=4, L=8, ratio=1, window=128, topk=512, index_block=64, index_keep=16,
                        H_i=64, D_i=128, H=64, Dk=512, Dv=512, bf16=True,
                        # ratio 1: Np = 1083 + L (HiSA; at L = 8 there are 17 blocks and the rows see 1084 ..
                        # 1091, so block 16 is eligible but partly hidden on the first rows), 694 + L (flat),
                        # 294 + L (dense), 16384 + L (HiSA)
                        t0=[1083, 694, 294, 16384], planted=4, Np_cap=16400)


@pytest.mark.parametrize("L", [1, 2, 4, 8, 48])
def test_short_prefill_chunks(hisa, L):
    # hisa_select_prefill with few query rows in all (4 sequences x L <= 192):
    # block means of every complete block into the workspace, then the
    # cached-means selection per row
    w = VERIFY.with_(L=L, Np_cap=max(16400, 16384 + L))
    x, g = inputs(w, 63)
    say(f"[run] short prefill chunk, L = {L}")
    hisa.hisa_profile_enable(True)
    try:
        I, blk, path = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w))
        torch.cuda.synchronize()
        names = set(hisa.hisa_profile_collect())
    finally:
        hisa.hisa_profile_enable(False)
    assert "cached_decode" in names and "select_rows" not in names, names
    assert parity.to_np(path).tolist() == [hisa.PATH_HISA, hisa.PATH_FLAT, hisa.PATH_DENSE, hisa.PATH_HISA]
    check_selection(w, x, I, blk, path)
    # the same call on a workspace holding another call's data (the counters are zeroed by the call itself)
    d = hisa.selection_dims(g["q_idx"], g["keys"], **sel_kw(w))
    ws = torch.full((hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, d),), 0x5A, dtype=torch.uint8, device="cuda")
    I2, blk2, path2 = hisa.hisa_select_prefill(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w), ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(I2, I) and torch.equal(blk2, blk) and torch.equal(path2, path)


def test_cached_verify_chunk_updates_the_cache(hisa):
    # A 4-row verify chunk on a caller cache: rows select on their own, and the
    # blocks the chunk's tokens complete (here block 255 of the ratio-4
    # sequence) are written into the cache.
    w = synth.FLASH_DECODE.with_(name="flash_verify_l4", L=4, t0=[65532], planted=32)
    x, g = inputs(w, synth.SEEDS[synth.FLASH_DECODE.name])
    dev = torch.device("cuda")
    rep = torch.full((1, 256, 128), float("nan"), dtype=torch.float32, device=dev)
    hisa.hisa_block_means_update(g["keys"], torch.zeros(1, dtype=torch.int32, device=dev), rep, ratio=4,
                                 index_block=64, L=65532)
    say("[run] cached verify chunk, L = 4")
    I, blk, path = hisa.hisa_select_decode_cached(g["q_idx"], g["w"], g["keys"], rep, g["t0"], **sel_kw(w))
    torch.cuda.synchronize()
    check_selection(w, x, I, blk, path)
    _, rep_orc = oracle.block_scores(odims(w, x), x["q_idx"], x["w"], x["keys"], x["t0"])
    np.testing.assert_allclose(parity.to_np(rep[0]), rep_orc[0], rtol=1e-6, atol=1e-7)
    # rows 0..2 see 16383 pooled rows: block 255 is eligible there (its first
    # row is visible) but its last row, pooled row 16383, is masked
    assert (parity.to_np(I)[0, :3] < 16383).all()
