"""The Python binding checks every tensor against the sizes it passes to the C
ABI (which carries no shapes) and raises HisaError before anything is
launched: wrong batch, width, index-row, output or length dims, wrong dtypes,
non-contiguous tensors, and tensors that are not on one GPU.  Runs on the
CPU: shape errors are reported whatever the device, and correctly shaped CPU
tensors stop at the device check."""
import pytest
import torch

from top_kv_indexer_amd import hisa

B, L, H_i, D_i, Np, topk, keep = 2, 3, 4, 8, 40, 16, 4
H, Dk, Wl = 2, 16, 10


def sel(**over):
    t = dict(q_idx=torch.zeros(B, L, H_i, D_i, dtype=torch.bfloat16), w=torch.zeros(B, L, H_i),
             keys=torch.zeros(B, Np, D_i, dtype=torch.bfloat16), t0=torch.zeros(B, dtype=torch.int32))
    t.update(over)
    return t


def att(**over):
    t = dict(q=torch.zeros(B, L, H, Dk, dtype=torch.bfloat16), local_kv=torch.zeros(B, Wl, Dk, dtype=torch.bfloat16),
             pooled_kv=torch.zeros(B, Np, Dk, dtype=torch.bfloat16), I=torch.zeros(B, L, topk, dtype=torch.int32),
             sinks=torch.zeros(H), t0=torch.zeros(B, dtype=torch.int32))
    t.update(over)
    return t


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(hisa.LIB_PATH):
        from top_kv_indexer_amd import build
        build.build()


def run_decode(t, **kw):
    return hisa.hisa_select_decode(t["q_idx"], t["w"], t["keys"], t["t0"], ratio=4, topk=topk, index_block=8,
                                   index_keep=keep, **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(w=torch.zeros(B, L, H_i + 1)), "w has shape"),
    (dict(w=torch.zeros(B + 1, L, H_i)), "w has shape"),
    (dict(w=torch.zeros(B, L, H_i, dtype=torch.float64)), "w must be torch.float32"),
    (dict(keys=torch.zeros(B, Np, D_i + 8, dtype=torch.bfloat16)), "keys has shape"),
    (dict(keys=torch.zeros(B + 1, Np, D_i, dtype=torch.bfloat16)), "keys has shape"),
    (dict(keys=torch.zeros(B, Np, D_i)), "keys must be torch.bfloat16"),
    (dict(t0=torch.zeros(B + 1, dtype=torch.int32)), "t0 has shape"),
    (dict(t0=torch.zeros(B, dtype=torch.int64)), "t0 must be torch.int32"),
    (dict(q_idx=torch.zeros(B, L, H_i, D_i, dtype=torch.float16)), "unsupported dtype"),
    (dict(q_idx=torch.zeros(B, L, D_i, H_i, dtype=torch.bfloat16).transpose(2, 3)), "contiguous"),
])
def test_selection_inputs(over, msg):
    with pytest.raises(hisa.HisaError, match=msg):
        run_decode(sel(**over))


@pytest.mark.parametrize("kw,msg", [
    (dict(I=torch.zeros(B, L, topk - 1, dtype=torch.int32)), "I has shape"),
    (dict(I=torch.zeros(B, L, topk, dtype=torch.int64)), "I must be torch.int32"),
    (dict(top_blk=torch.zeros(B, L, keep + 1, dtype=torch.int32)), "top_blk has shape"),
    (dict(path=torch.zeros(B + 1, dtype=torch.int32)), "path has shape"),
    (dict(ws=torch.zeros(1024, dtype=torch.float32)), "ws must be torch.uint8"),
])
def test_selection_outputs(kw, msg):
    with pytest.raises(hisa.HisaError, match=msg):
        run_decode(sel(), **kw)


def test_flat_and_block_scores_inputs():
    t = sel(keys=torch.zeros(B, Np, D_i + 8, dtype=torch.bfloat16))
    with pytest.raises(hisa.HisaError, match="keys has shape"):
        hisa.flat_topk_select(t["q_idx"], t["w"], t["keys"], t["t0"], ratio=1, topk=topk)
    with pytest.raises(hisa.HisaError, match="keys has shape"):
        hisa.hisa_block_scores(t["q_idx"], t["w"], t["keys"], t["t0"], ratio=1, index_block=8)
    t = sel()
    with pytest.raises(hisa.HisaError, match="I has shape"):
        hisa.flat_topk_select(t["q_idx"], t["w"], t["keys"], t["t0"], ratio=1, topk=topk,
                              I=torch.zeros(B, L + 1, topk, dtype=torch.int32))


def run_att(t, **kw):
    return hisa.sparse_local_pooled_attention(t["q"], t["local_kv"], t["pooled_kv"], t["I"], t["sinks"], t["t0"],
                                              ratio=4, window=8, **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(pooled_kv=torch.zeros(B, Np, Dk + 8, dtype=torch.bfloat16)), "pooled_kv has shape"),
    (dict(pooled_kv=torch.zeros(B + 1, Np, Dk, dtype=torch.bfloat16)), "pooled_kv has shape"),
    (dict(local_kv=torch.zeros(B, Wl, Dk - 8, dtype=torch.bfloat16)), "local_kv has shape"),
    (dict(local_kv=torch.zeros(B - 1, Wl, Dk, dtype=torch.bfloat16)), "local_kv has shape"),
    (dict(local_kv=torch.zeros(B, Wl, Dk)), "local_kv must be torch.bfloat16"),
    (dict(I=torch.zeros(B, L + 1, topk, dtype=torch.int32)), "I has shape"),
    (dict(I=torch.zeros(B, L, topk)), "I must be torch.int32"),
    (dict(t0=torch.zeros(B - 1, dtype=torch.int32)), "t0 has shape"),
    (dict(sinks=torch.zeros(H + 1)), "sinks has shape"),
    (dict(sinks=torch.zeros(H, dtype=torch.bfloat16)), "sinks must be torch.float32"),
    (dict(local_kv=None), "window > 0"),
])
def test_attention_inputs(over, msg):
    with pytest.raises(hisa.HisaError, match=msg):
        run_att(att(**over))


def test_attention_output_shape_and_dtype():
    with pytest.raises(hisa.HisaError, match="out has shape"):
        run_att(att(), out=torch.zeros(B, L, H, Dk + 1, dtype=torch.bfloat16))
    with pytest.raises(hisa.HisaError, match="out must be torch.bfloat16"):
        run_att(att(), out=torch.zeros(B, L, H, Dk))
    # a value width below the key width (MLA-style): out is (B, L, H, Dv)
    with pytest.raises(hisa.HisaError, match="out has shape"):
        run_att(att(), Dv=8, out=torch.zeros(B, L, H, Dk, dtype=torch.bfloat16))


def test_well_shaped_cpu_tensors_stop_at_the_device_check():
    with pytest.raises(hisa.HisaError, match="must be on a GPU"):
        run_decode(sel())
    with pytest.raises(hisa.HisaError, match="must be on a GPU"):
        run_att(att())
