"""hisa_select_decode_noalloc (the decode selection on the library's own
per-GPU workspace, for callers that cannot allocate) against
hisa_select_decode with a caller workspace, through the C ABI: bit-identical
index outputs on consecutive calls whose sizes change (a smaller call after a
larger one, then a larger one again, so the arrival counters must be cleared
over the previous call's scores)."""
import sys

import numpy as np
import pytest

from tests.test_gpu_parity import MIXED, inputs, sel_kw
from top_kv_indexer_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def hisa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from top_kv_indexer_amd import hisa as h
    h.lib()
    return h


def test_noalloc_decode_matches_the_workspace_call(hisa):
    cases = [(MIXED, 5),                                                      # B = 6, Np_cap 5000: all paths
             (MIXED.with_(name="mixed_b2_small", B=2, t0=[4096, 5000], Np_cap=1300), 6),   # smaller
             (synth.BATCHED_DECODE, synth.SEEDS[synth.BATCHED_DECODE.name])]  # larger: B = 32, Np_cap 32768
    for w, seed in cases:
        print(f"[run] noalloc decode selection, {w.name}", flush=True)
        sys.stdout.flush()
        x, g = inputs(w, seed)
        B = w.B
        I = torch.full((B, 1, w.topk), -7, dtype=torch.int32, device="cuda")
        blk = torch.full((B, 1, w.index_keep), -7, dtype=torch.int32, device="cuda")
        path = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        hisa.hisa_select_decode_noalloc(g["q_idx"], g["w"], g["keys"], g["t0"], I, blk, path, **sel_kw(w))
        d = hisa.selection_dims(g["q_idx"], g["keys"], **sel_kw(w))
        ws = torch.zeros(hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d), dtype=torch.uint8, device="cuda")
        Ir, blkr, pathr = hisa.hisa_select_decode(g["q_idx"], g["w"], g["keys"], g["t0"], **sel_kw(w), ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(path, pathr), (path, pathr)
        assert torch.equal(I, Ir)
        assert torch.equal(blk, blkr)
        assert (path.cpu().numpy() >= 0).all()
