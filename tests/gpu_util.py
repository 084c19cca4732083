"""Helpers for the GPU parity tests (not a test module)."""
import numpy as np
import pytest


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


# Tolerance on y: relative L2 error 1e-5 (f32 accumulation against the f64
# oracle), as the workload statement fixes it.
REL_L2_TOL = 1e-5


def assert_y_close(got, ref, tol=REL_L2_TOL):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN pattern differs"
    gi, ri = np.isinf(got), np.isinf(ref)
    assert np.array_equal(gi, ri), "infinity pattern differs"
    assert np.array_equal(got[gi], ref[ri]), "infinity signs differ"
    ok = ~np.isnan(ref) & ~ri
    r = rel_l2(got[ok], ref[ok])
    assert r <= tol, f"rel L2 {r:.3e} > {tol:.0e}"
    return r


def assert_bits_equal(got, ref):
    """Bit-exact f32 comparison (NaNs compared as a set)."""
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    assert got.shape == ref.shape
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), "NaN positions differ"
    bad = (got.view(np.uint32) != ref.view(np.uint32)) & ~rn
    n = int(bad.sum())
    assert n == 0, f"{n} decoded values differ; first at {np.argwhere(bad)[:3].tolist()}"
