"""The seeded input generator: shapes, dtypes, determinism, recipe."""
import numpy as np
import torch

from block_sparse_backward_amd.synth import CONFIGS, make_inputs, to_f64


def test_tiny_shapes_and_determinism():
    cfg = CONFIGS["tiny"]
    a = make_inputs(cfg, 0)
    b = make_inputs(cfg, 0)
    c = make_inputs(cfg, 1)
    assert a["q"].shape == (1, 2, 256, 64) and a["k"].shape == (1, 2, 256, 64)
    assert a["q"].dtype == torch.float32
    for name in a:
        assert torch.equal(a[name], b[name])
        assert not torch.equal(a[name], c[name])


def test_bf16_cast_is_round_to_nearest_even_of_f32_draw():
    cfg = CONFIGS["mid"].with_(N=256, Hq=4, Hkv=2)
    t = make_inputs(cfg, 0)
    assert t["q"].dtype == torch.bfloat16
    rng = np.random.Generator(np.random.PCG64(0))
    q32 = rng.standard_normal(t["q"].shape, dtype=np.float32)
    # round-to-nearest-even to 8 significant bits, done on the integer bits
    bits = q32.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    want = rounded.astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(to_f64(t["q"]), want.astype(np.float64))


def test_boosted_blocks_recipe():
    cfg = CONFIGS["headline"].with_(N=128 * 40, Hq=2, Hkv=1)
    t = make_inputs(cfg, 0)
    assert round(cfg.boost_frac * cfg.nqb) == 2
    rms = to_f64(t["dout"]).reshape(1, 2, 40, -1).std(axis=-1)
    # the boosted blocks stand out by ~20x in rms over the lognormal(0, 2) rows
    top = np.sort(rms, axis=-1)[..., -2:]
    assert np.all(top > 5 * np.median(rms, axis=-1, keepdims=True))
