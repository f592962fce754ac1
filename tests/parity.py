"""Comparison rules between the HIP library and the CPU oracle.

Index sets (HiSA issue, Conventions: argpartition returns an unordered set):
both sides are compared as sets.  Let tau be the oracle's k-th best visible
score.  Every id in the symmetric difference must score within 1e-5 * |tau| of
tau on the oracle (exact ties included); masked ids (score -1e30) are compared
by count only.  Hierarchical rows compare the retained blocks first with the
same rule on the coarse scores; when the block sets legitimately differ, the
oracle's fine stage is re-run on the GPU's blocks before comparing I.
Attention outputs: max-abs 1e-4 (f32 inputs) or 2e-2 (bf16 inputs), computed
with the GPU's own I fed to the oracle.
"""
import numpy as np

import oracle

TIE_RTOL = 1e-5
NEG = np.float32(-1e30)


def to_np(t):
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


class Mismatch(AssertionError):
    pass


def _ids(row):
    ids = row[row >= 0]
    if len(np.unique(ids)) != len(ids):
        raise Mismatch(f"duplicate ids in {np.sort(ids)[:20]}...")
    return ids


def compare_sets(gpu_ids, orc_ids, score_of, what="I"):
    """gpu_ids / orc_ids: 1-D arrays with -1 padding; score_of(ids) -> oracle scores."""
    G, O = _ids(gpu_ids), _ids(orc_ids)
    if len(G) != len(O):
        raise Mismatch(f"{what}: {len(G)} ids on the GPU, {len(O)} in the oracle")
    if set(G.tolist()) == set(O.tolist()):
        return 0
    union = np.union1d(G, O).astype(np.int32)
    s = dict(zip(union.tolist(), score_of(union).tolist()))
    Gv = [i for i in G.tolist() if s[i] != NEG]
    Ov = [i for i in O.tolist() if s[i] != NEG]
    if len(Gv) != len(Ov):
        raise Mismatch(f"{what}: {len(Gv)} visible ids on the GPU vs {len(Ov)} in the oracle")
    if not Ov:
        return 0
    tau = min(s[i] for i in Ov)
    band = TIE_RTOL * abs(tau)
    diff = set(Gv) ^ set(Ov)
    bad = [(i, s[i]) for i in diff if abs(s[i] - tau) > band]
    if bad:
        raise Mismatch(f"{what}: {len(diff)} ids differ, {len(bad)} outside the tie band around tau={tau!r}: {bad[:8]}")
    return len(diff) // 2


def check_selection_row(d, inp, b, j, I_gpu, blk_gpu, path_gpu, I_orc=None, blk_orc=None, path_orc=None):
    """Checks one (b, j) row.  inp: dict of numpy inputs (synth.make_inputs)."""
    q_row, w_row, keys_b, t0 = inp["q_idx"][b, j], inp["w"][b, j], inp["keys"][b], int(inp["t0"][b])
    if I_orc is None:
        I_orc, blk_orc, path_orc = oracle.select_row(d, q_row, w_row, keys_b, t0, j)
    if path_gpu is not None and path_gpu != path_orc:
        raise Mismatch(f"row ({b},{j}): path {path_gpu} on the GPU, {path_orc} in the oracle")
    Np = oracle.num_pooled(t0, d.L, d.ratio)
    g = I_gpu[I_gpu >= 0]
    if (g >= Np).any():
        raise Mismatch(f"row ({b},{j}): ids past Np={Np}")
    if path_orc == oracle.PATH_HISA and blk_gpu is not None:
        nb = Np // d.index_block
        if (blk_gpu[blk_gpu >= 0] >= nb).any():
            raise Mismatch(f"row ({b},{j}): blocks past nb={nb}")
        cs = coarse_row(d, inp, b, j)
        compare_sets(blk_gpu, blk_orc, lambda ids: cs[ids], what=f"top_blk ({b},{j})")
        if set(blk_gpu[blk_gpu >= 0].tolist()) != set(blk_orc[blk_orc >= 0].tolist()):
            kb = blk_gpu[blk_gpu >= 0]
            I_orc, _, _ = oracle.select_row(d, q_row, w_row, keys_b, t0, j, given_blocks=kb)
        if not np.isin(g // d.index_block, blk_gpu).all():
            raise Mismatch(f"row ({b},{j}): ids outside the retained blocks")
    compare_sets(I_gpu, I_orc, lambda ids: oracle.scores_of(d, q_row, w_row, keys_b, t0, j, ids),
                 what=f"I ({b},{j})")


def coarse_row(d, inp, b, j):
    """Oracle coarse scores (nb_cap,) of row (b, j)."""
    return oracle.coarse_row(d, inp["q_idx"][b, j], inp["w"][b, j], inp["keys"][b], int(inp["t0"][b]), j)


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        raise Mismatch(f"shapes {a.shape} vs {b.shape}")
    if not np.isfinite(a).all():
        raise Mismatch("non-finite values on the GPU")
    return float(np.max(np.abs(a - b))) if a.size else 0.0
