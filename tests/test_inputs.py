"""The seeded generator: determinism, bf16 rounding, config shapes (CPU only)."""
import numpy as np
import pytest
import torch

from generative_recommendation_beam_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 3.0e38], np.float32)])
    x = x.astype(np.float32)
    mine = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(inputs.bf16_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_deterministic():
    a = inputs.config(3)
    b = inputs.config(3)
    for f in ("q", "k_shared", "v_shared", "k_new", "v_new", "parents", "unshared_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = inputs.config(3, layer=1)
    assert not np.array_equal(a.q, c.q)


def test_config_shapes():
    w = inputs.config(1)
    assert (w.R, w.B, w.Hq, w.Hkv, w.D, w.dtype) == (1, 4, 4, 1, 64, "f32")
    assert w.k_shared.shape == (1, 256, 64) and w.k_new.shape == (2, 4, 1, 64)
    w = inputs.config(3)
    assert set(w.unshared_len.tolist()) <= {1, 2, 3}
    assert w.q.dtype == np.uint16 and w.T_max == 3
    # truncated Zipf: beam 0 is the most frequent parent
    counts = np.bincount(w.parents[1:].ravel(), minlength=w.B)
    assert counts.argmax() == 0 and w.parents.max() < w.B


def test_config4_variants_share_values():
    a = inputs.config("4A")
    b = inputs.config("4B")
    assert b.R == 64 and b.B == 1 and a.N_b == b.N_b
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_new, b.k_new)
    for n in range(64):
        r = n // 16
        oa, ob = int(a.prefix_off[r]), int(b.prefix_off[n])
        assert np.array_equal(a.k_shared[:, oa:oa + 4096], b.k_shared[:, ob:ob + 4096])
