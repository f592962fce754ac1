"""hisa_decode_step (the decode selection and the sparse combine in one call)
against the CPU oracle and against the two separate calls, through the C ABI.
The one-kernel step hands the kept blocks and the fine threshold from its
selecting workgroup to its attention workgroups; these tests cover every gate
outcome in one batch (dense, flat, HiSA with and without a tail, invalid),
exact ties at both top-k boundaries, kept blocks of 16 and 32 rows, no window
and no sinks, workspace reuse (every sync word back at zero), HIP-graph
replay, and the batched shapes that take the two calls' kernels."""
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


def to_gpu(x, w):
    dt = torch.bfloat16 if w.bf16 else torch.float32
    g = {k: torch.from_numpy(x[k]).to("cuda").to(dt).contiguous() for k in ("q_idx", "keys", "q", "local_kv",
                                                                            "pooled_kv")}
    g["w"] = torch.from_numpy(x["w"]).to("cuda")
    g["sinks"] = None if x["sinks"] is None else torch.from_numpy(x["sinks"]).to("cuda")
    g["t0"] = torch.from_numpy(x["t0"]).to("cuda")
    return g


def odims(w, x):
    return oracle.Dims(B=w.B, L=1, ratio=w.ratio, window=w.window, topk=w.topk, index_block=w.index_block,
                       index_keep=w.index_keep, H_i=w.H_i, D_i=w.D_i, H=w.H, Dk=w.Dk, Dv=w.Dv,
                       Np_cap=int(x["Np_cap"]))


def step(hisa, w, g, ws=None, local=True):
    return hisa.hisa_decode_step(g["q_idx"], g["w"], g["keys"], g["q"], g["local_kv"] if local else None,
                                 g["pooled_kv"], g["sinks"], g["t0"], ratio=w.ratio, window=w.window, topk=w.topk,
                                 index_block=w.index_block, index_keep=w.index_keep, ws=ws)


def two_calls(hisa, w, g, local=True):
    I, blk, path = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], ratio=w.ratio, topk=w.topk,
                                           index_block=w.index_block, index_keep=w.index_keep)
    out = hisa.sparse_local_pooled_attention(g["q"], g["local_kv"] if local else None, g["pooled_kv"], I,
                                             g["sinks"], g["t0"], ratio=w.ratio, window=w.window)
    return I, blk, path, out


def kernels_of(hisa, fn):
    """Runs fn with the library's kernel timing on; returns the kernel names."""
    hisa.hisa_profile_enable(True)
    try:
        r = fn()
        torch.cuda.synchronize()
        names = set(hisa.hisa_profile_collect())
    finally:
        hisa.hisa_profile_enable(False)
    return r, names


def check_against_oracle(hisa, w, x, res, t0s=None):
    """Selection rows within the tie band of the oracle's and paths equal; the
    attention rows within 2e-2 of the oracle's combine on the same index row."""
    I, blk, path, out = (parity.to_np(t) for t in res)
    d = odims(w, x)
    t0s = [int(t) for t in x["t0"]] if t0s is None else t0s
    for b in range(w.B):
        t0 = t0s[b]
        if t0 < 0:
            continue
        parity.check_selection_row(d, x, b, 0, I[b, 0], blk[b, 0], path[b])
        ref = oracle.combine_row(d, x["q"][b, 0], x["local_kv"][b], x["pooled_kv"][b], I[b, 0], x["sinks"], t0, 0)
        err = parity.max_abs(out[b, 0], ref)
        assert err <= 2e-2, (b, err)


def check_equal_to_two_calls(hisa, w, g, res, local=True, exact_out=False):
    I2, blk2, path2, out2 = two_calls(hisa, w, g, local)
    torch.cuda.synchronize()
    I, blk, path, out = res
    assert torch.equal(I, I2)
    assert torch.equal(blk, blk2)
    assert torch.equal(path, path2)
    if exact_out:
        assert torch.equal(out, out2)
    else:
        err = (out.float() - out2.float()).abs().max().item()
        assert err <= 2e-2, err


def test_step_v4flash_decode(hisa):
    w = synth.FLASH_DECODE
    x = synth.make_inputs(w, synth.SEEDS[w.name])
    g = to_gpu(x, w)
    say(f"[run] hisa_decode_step {w.name}")
    res, names = kernels_of(hisa, lambda: step(hisa, w, g))
    assert names == {"decode_step", "attention_merge"}, names
    assert (parity.to_np(res[2]) == hisa.PATH_HISA).all()
    check_equal_to_two_calls(hisa, w, g, res)
    check_against_oracle(hisa, w, x, res)


# Every gate outcome in one batch (16 heads keep the grid small enough for
# the one-kernel step): Np = 300 (dense), 700 (flat), 1024 (HiSA, no tail),
# 1500 (HiSA + tail), 5000 and 4100 (HiSA), and a sequence made invalid on
# the device (t0 < 0).
MIXED = synth.Workload("step_mixed_b7", B=7, L=1, ratio=4, window=128, topk=512, index_block=64, index_keep=16,
                       H_i=64, D_i=128, H=16, Dk=512, Dv=512, bf16=True,
                       t0=[1200, 2800, 4096, 6000, 20000, 16400, 3000], planted=4, Np_cap=5000)


def test_step_mixed_paths_and_invalid(hisa):
    w = MIXED
    x = synth.make_inputs(w, 11)
    g = to_gpu(x, w)
    g["t0"][6] = -5
    say("[run] hisa_decode_step mixed paths")
    res, names = kernels_of(hisa, lambda: step(hisa, w, g))
    assert names == {"decode_step", "attention_merge"}, names
    path = parity.to_np(res[2]).tolist()
    assert path == [hisa.PATH_DENSE, hisa.PATH_FLAT] + [hisa.PATH_HISA] * 4 + [hisa.PATH_INVALID], path
    I, out = parity.to_np(res[0]), parity.to_np(res[3])
    assert (I[6] == -1).all() and (out[6] == 0).all()
    assert (I[3, 0] < (1500 // 64) * 64).all()  # the tail rows are never selected
    check_equal_to_two_calls(hisa, w, g, res)
    check_against_oracle(hisa, w, x, res, t0s=[int(t) for t in x["t0"][:6]] + [-5])


def test_step_exact_ties_take_the_index_rows(hisa):
    # The best indexer key of each HiSA sequence is copied over rows 640 ..
    # 2559, so 30 blocks tie for the coarse top and more than 512 candidates
    # for the fine top: the selection keeps the lowest ids.  The attention
    # must use exactly those rows: q is zero (every score 0, a uniform softmax)
    # and tied row r carries 256 in value column r % 512, so a row attended
    # instead of another moves an output by about 0.4.
    w = MIXED.with_(name="step_ties_b6", B=6, t0=[1200, 2800, 4096, 6000, 20000, 16400])
    x = synth.make_inputs(w, 12)
    od = odims(w, x)
    keys, pooled, q = x["keys"].copy(), x["pooled_kv"].copy(), np.zeros_like(x["q"])
    for b in range(w.B):
        t0 = int(w.t0[b])
        Np = oracle.num_pooled(t0, 1, w.ratio)
        _, _, po = oracle.select_row(od, x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], t0, 0)
        lo, hi = (100, 600) if po == oracle.PATH_FLAT else (640, min(2560, Np))
        if po == oracle.PATH_DENSE:
            continue
        sc = oracle.scores_of(od, x["q_idx"][b, 0], x["w"][b, 0], x["keys"][b], t0, 0,
                              np.arange(Np, dtype=np.int32))
        keys[b, lo:hi] = x["keys"][b, int(np.argmax(sc))]
        for r in range(lo, hi):
            pooled[b, r, r % 512] = 256.0
    x = dict(x, keys=keys, pooled_kv=pooled, q=q)
    g = to_gpu(x, w)
    say("[run] hisa_decode_step with exact ties")
    res, names = kernels_of(hisa, lambda: step(hisa, w, g))
    assert names == {"decode_step", "attention_merge"}, names
    check_equal_to_two_calls(hisa, w, g, res)
    check_against_oracle(hisa, w, x, res)


@pytest.mark.parametrize("block,keep", [(32, 32), (16, 64)])
def test_step_small_blocks_no_window_no_sinks(hisa, block, keep):
    # several kept blocks per attention split; no local stream and no sinks
    w = synth.FLASH_DECODE.with_(name=f"step_b{block}", index_block=block, index_keep=keep, window=0, sinks=False,
                                 H=16)
    x = synth.make_inputs(w, 13)
    g = to_gpu(x, w)
    say(f"[run] hisa_decode_step index_block {block}")
    res, names = kernels_of(hisa, lambda: step(hisa, w, g, local=False))
    assert names == {"decode_step", "attention_merge"}, names
    assert (parity.to_np(res[2]) == hisa.PATH_HISA).all()
    check_equal_to_two_calls(hisa, w, g, res, local=False)
    check_against_oracle(hisa, w, x, res)


def sync_region_bytes(w, Np_cap):
    """Bytes of the decode step's words that rest at zero: its sync words, then
    hisa_select_decode's arrival counters."""
    r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    nps = -(-max(w.index_keep * w.index_block, w.topk) // 64)
    sync = r256(64 + w.B * 64 * 2 + w.B * nps * 8)
    slabs = -(-Np_cap // 64)
    return sync + r256(w.B * (1 + -(-slabs // 16)) * 64)


def test_step_workspace_reuse(hisa):
    # Three calls on one workspace with pooled counts (and so slab counts,
    # paths and kept lists) that change between calls: each matches the two
    # calls, and every sync word and counter is zero again after each.
    # (inputs drawn at the largest pooled count, so every call's rows are real)
    w = MIXED.with_(name="step_reuse_b3", B=3, t0=[20000, 20000, 20000])
    x = synth.make_inputs(w, 14)
    g = to_gpu(x, w)
    d = hisa.decode_step_dims(g["q_idx"], g["keys"], g["q"], g["local_kv"], g["pooled_kv"], ratio=w.ratio,
                              window=w.window, topk=w.topk, index_block=w.index_block, index_keep=w.index_keep)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_DECODE_STEP, d), dtype=torch.uint8, device="cuda")
    rest = sync_region_bytes(w, int(x["Np_cap"]))
    for t0s in ([20000, 16400, 6000], [2800, 19999, 4096], [20000, 1200, 16400]):
        g["t0"] = torch.tensor(t0s, dtype=torch.int32, device="cuda")
        say(f"[run] hisa_decode_step reuse t0={t0s}")
        res, names = kernels_of(hisa, lambda: step(hisa, w, g, ws=ws))
        assert names == {"decode_step", "attention_merge"}, names
        assert int(ws[:rest].count_nonzero()) == 0
        check_equal_to_two_calls(hisa, w, g, res)


def test_step_graph_replay(hisa):
    # One captured step replayed with other work and synchronisations between
    # the replays: every replay equals the eager call.
    w = synth.FLASH_DECODE
    x = synth.make_inputs(w, synth.SEEDS[w.name])
    g = to_gpu(x, w)
    I0, blk0, path0, out0 = step(hisa, w, g)
    torch.cuda.synchronize()
    I, blk, path, out = (torch.empty_like(t) for t in (I0, blk0, path0, out0))
    d = hisa.decode_step_dims(g["q_idx"], g["keys"], g["q"], g["local_kv"], g["pooled_kv"], ratio=w.ratio,
                              window=w.window, topk=w.topk, index_block=w.index_block, index_keep=w.index_keep)
    ws = torch.zeros(hisa.workspace_bytes(hisa.OP_DECODE_STEP, d), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        hisa.hisa_decode_step(g["q_idx"], g["w"], g["keys"], g["q"], g["local_kv"], g["pooled_kv"], g["sinks"],
                              g["t0"], ratio=w.ratio, window=w.window, topk=w.topk, index_block=w.index_block,
                              index_keep=w.index_keep, I=I, top_blk=blk, path=path, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (I, blk, path, out):
            t.fill_(7 if t.dtype == torch.int32 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[run] replay {rep}")
        assert torch.equal(I, I0) and torch.equal(blk, blk0) and torch.equal(path, path0)
        assert torch.equal(out, out0)


def test_step_batched_takes_two_calls(hisa):
    # 32 sequences of up to 32768 pooled rows: past the one-kernel step's
    # grid, so the call runs the selection's and the attention's kernels;
    # outputs equal those two calls bit for bit.
    w = synth.BATCHED_DECODE
    x = synth.make_inputs(w, synth.SEEDS[w.name])
    g = to_gpu(x, w)
    say("[run] hisa_decode_step batched")
    res, names = kernels_of(hisa, lambda: step(hisa, w, g))
    assert "decode_step" not in names and "attention" in names, names
    check_equal_to_two_calls(hisa, w, g, res, exact_out=True)
    I, out = parity.to_np(res[0]), parity.to_np(res[3])
    d = odims(w, x)
    for b in (0, 13, 31):
        ref = oracle.combine_row(d, x["q"][b, 0], x["local_kv"][b], x["pooled_kv"][b], I[b, 0], x["sinks"],
                                 int(x["t0"][b]), 0)
        assert parity.max_abs(out[b, 0], ref) <= 2e-2, b
