"""The seeded input generator: determinism, shapes, bf16 rounding, planting
and NaN padding of ragged batches."""
import numpy as np

from top_kv_indexer_amd import synth


def test_round_bf16_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, 3.14159], np.float32)
    r = synth.round_bf16(x)
    assert r[0] == 1.0 and r[3] == 1.0            # below half an ulp
    assert r[1] == 1.0                             # tie -> even
    assert r[2] == 1.0 + 4 * 2 ** -8               # tie -> even (up)
    assert r[4] == -2.5 and r[5] == 0.0
    u = r.view(np.uint32)
    assert (u & 0xFFFF == 0).all()
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000).astype(np.float32)
    ry = synth.round_bf16(y)
    assert np.max(np.abs(ry - y) / np.abs(y)) <= 2 ** -8


def test_tiny_decode_layout_and_determinism():
    a = synth.make_inputs(synth.TINY_DECODE, 1001)
    b = synth.make_inputs(synth.TINY_DECODE, 1001)
    for k in ("q_idx", "w", "keys", "q", "local_kv", "pooled_kv", "sinks"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["Np"][0] == 1024 and a["Np_cap"] == 1024
    assert a["q_idx"].shape == (1, 1, 4, 32) and a["keys"].shape == (1, 1024, 32)
    assert a["local_kv"].shape == (1, 128, 64) and a["sinks"].shape == (4,)
    assert (a["planted"][0] >= 0).sum() == 6


def test_ragged_padding_is_nan():
    w = synth.BATCHED_DECODE.with_(B=3, Np_cap=8192, t0_range=(4000, 32000))
    x = synth.make_inputs(w, 7)
    for b in range(3):
        Np = x["Np"][b]
        assert Np == (x["t0"][b] + 1) // 4
        assert np.isfinite(x["keys"][b, :Np]).all() and np.isnan(x["keys"][b, Np:]).all()
        assert np.isnan(x["pooled_kv"][b, Np:]).all()
        v = x["keys"][b, :Np]
        assert (v.view(np.uint32) & 0xFFFF == 0).all()   # bf16 values
