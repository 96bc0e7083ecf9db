"""Shared helpers for the GPU parity tests: device transfer and comparison
against the fp64 oracle with the tolerances of the parity bar (max-abs 2e-2
on O, 1e-3 on LSE)."""
import math

import numpy as np

O_TOL = 2e-2
LSE_TOL = 1e-3


def to_dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Element-wise comparison; -inf LSE rows must match exactly (and O = 0)."""
    o = np.asarray(o_gpu, dtype=np.float64)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    assert o.shape == o_ref.shape, (what, o.shape, o_ref.shape)
    assert lg.shape == lse_ref.shape, (what, lg.shape, lse_ref.shape)
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), ninf_ref), f"{what}: empty-row pattern differs"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    eo = float(np.abs(o - o_ref).max()) if o.size else 0.0
    fin = ~ninf_ref
    el = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e} > {O_TOL}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e} > {LSE_TOL}"
    return eo, el


def sample_rows(rng, B, H, N, n, must=()):
    """n distinct (b, h, i) triples plus the listed ones (first/last rows...)."""
    rows = set(tuple(m) for m in must)
    while len(rows) < n + len(must):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return np.array(sorted(rows), dtype=np.int32)


def scale_for(d):
    return 1.0 / math.sqrt(d)


# Backward bound, derived in tests/test_gpu_bwd.py's module docstring: per
# tensor, max|g - g_ref| <= GRAD_TOL * max|g_ref| + GRAD_ABS.
GRAD_TOL = 1e-2
GRAD_ABS = 1e-4


def compare_grads(got, ref, lse, what):
    """got, ref: (dq, dk, dv); lse: the GPU forward's LSE (rows at -inf see
    no key, so their dQ must be exactly zero, as must dK and dV of keys that
    no row sees, i.e. whose reference dV row is zero)."""
    empty_rows = np.isneginf(np.asarray(lse))
    unseen = ~np.asarray(ref[2]).any(axis=-1)
    assert not np.asarray(got[0])[empty_rows].any(), f"{what}: dq nonzero on a row with no visible key"
    assert not np.asarray(got[1])[unseen].any(), f"{what}: dk nonzero on a key no row sees"
    assert not np.asarray(got[2])[unseen].any(), f"{what}: dv nonzero on a key no row sees"
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = np.asarray(g, dtype=np.float64)
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        mx = float(np.abs(r).max()) if r.size else 0.0
        err = float(np.abs(g - r).max()) if r.size else 0.0
        assert err <= GRAD_TOL * mx + GRAD_ABS, f"{what}: {name} max err {err:.3e} vs max|ref| {mx:.3e}"
        errs.append(err / max(mx, 1e-30))
    return errs
