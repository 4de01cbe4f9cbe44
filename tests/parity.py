"""Tolerances and comparison helpers for HIP-vs-oracle parity.

Floating point: bf16 inputs with fp32 outputs must match the fp64 oracle to
max|dO| <= 1e-2 and mean|dO| <= 1e-3; the fp32 path to max|dO| <= 1e-4.
Because several workloads draw Q/K/V scaled by 1/sqrt(128) (outputs of order
1e-3, where an absolute bound cannot tell a kernel that returns zeros), every
comparison also bounds the relative Frobenius error ||dO|| / ||O|| (bf16:
1e-2, fp32: 1e-5) and the lse error (bf16: 1e-2, fp32: 1e-5). The bf16 bound
comes from rounding the probabilities to bf16 before the P.V product (relative
error of a sum of rounded terms ~ 2^-8 / sqrt(3) ~ 2.3e-3) plus fp32
accumulation.
"""
import numpy as np

TOL = {
    "bf16": dict(max_abs=1e-2, mean_abs=1e-3, rel_fro=1e-2, lse=1e-2),
    "f32": dict(max_abs=1e-4, mean_abs=1e-5, rel_fro=1e-5, lse=1e-5),
}


def compare(o_gpu, o_ref, lse_gpu, lse_ref, dtype, what=""):
    """Raise AssertionError with a summary if any bound fails; return stats."""
    t = TOL[dtype]
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    d = np.abs(o_gpu - o_ref)
    nref = np.linalg.norm(o_ref)
    stats = dict(max_abs=float(d.max()) if d.size else 0.0,
                 mean_abs=float(d.mean()) if d.size else 0.0,
                 rel_fro=float(np.linalg.norm(o_gpu - o_ref) / nref) if nref > 0 else float(np.linalg.norm(o_gpu)))
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        ninf_g, ninf_r = np.isneginf(lse_gpu), np.isneginf(lse_ref)
        assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf lse pattern differs"
        fin = ~ninf_r
        stats["lse"] = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
        assert not np.isnan(lse_gpu).any(), f"{what}: NaN lse"
    for k, v in stats.items():
        assert v <= t[k], f"{what}: {k} = {v:.3e} exceeds {t[k]:.1e} (all: {stats})"
    return stats
