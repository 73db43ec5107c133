"""The seeded input generator: storage conversions and the workload recipes."""
import numpy as np
import pytest
import torch

import gdr_inputs as gi


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_and_deterministic():
    w = gi.GDN_PREFILL.scaled(B=1, H=2, T=32)
    a, b = gi.make_prefill(w), gi.make_prefill(w)
    for key in a:
        if a[key] is None:
            assert b[key] is None
        else:
            np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("w", [gi.TINY_GDN_F32, gi.GDN_PREFILL.scaled(B=1, H=4, T=512),
                               gi.KDA_FG2PLUS_PREFILL.scaled(B=1, H=2, T=256),
                               gi.OSDN_LONG_PREFILL.scaled(H=2, T=512)], ids=lambda w: w.name)
def test_prefill_recipe(w):
    x = gi.make_prefill(w)
    f = gi.prefill_f64(w, x)
    assert f["q"].shape == (w.B, w.T, w.H, w.dk) and f["v"].shape == (w.B, w.T, w.H, w.dv)
    # keys are unit-norm before storage rounding
    nk = np.linalg.norm(f["k"], axis=-1)
    assert np.all(np.abs(nk - 1.0) < (1e-6 if w.io == gi.F32 else 1e-2))
    a = f["alpha"]
    assert np.all((a > 0) & (a < 1))
    if w.alpha_flip:  # sigmoid(N(3, 0.5))
        assert 0.93 < a.mean() < 0.96
    else:             # exp(-softplus(N(-4, 1)))
        assert 0.97 < a.mean() < 0.99
    assert 0.4 < f["beta_k"].mean() < 0.6
    assert (x["alpha"].ndim == 4) == (w.alpha_mode == gi.GATE_CHANNEL)
    assert (x["beta_v"] is not None) == (w.beta_mode == gi.BETA_KV)
    assert (x["k_w"] is not None) == w.write_key
    assert (x["S0"] is not None) == (w.s0_std > 0)
    if w.write_key:
        ratio = f["k_w"] / np.where(f["k"] == 0, 1, f["k"])
        assert abs(np.median(ratio) - 1.0) < 0.02
        assert 0.08 < np.std(ratio[np.abs(f["k"]) > 0.05]) < 0.12


def test_decode_recipe():
    w = gi.DECODE_DMEM_R8.scaled(B=64, steps=4)
    x = gi.make_decode(w)
    assert x["q"].shape == (4, 64, 1, 8) and x["S"].shape == (64, 1, 8, 8)
    assert x["alpha"].dtype == np.uint16 and x["S"].dtype == np.float32
