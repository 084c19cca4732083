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


# Per-element tolerance: |y - y_ref| / sum_i |w_i x_i| <= 1e-4, the
# magnitude-relative check of colibri PR #457, section 5.
ELEM_TOL = 1e-4


def assert_y_close(got, ref, tol=REL_L2_TOL, mag=None, elem_tol=ELEM_TOL):
    """rel L2 <= tol on the finite entries (same NaN / infinity pattern), and,
    given mag[t][o] = sum_i |w_oi x_ti|, every finite entry within elem_tol of
    its magnitude."""
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
    if mag is not None:
        mag = np.asarray(mag, np.float64).reshape(ref.shape)
        m = ok & (mag > 0)
        d = np.abs(got[m].astype(np.float64) - ref[m].astype(np.float64)) / mag[m]
        worst = float(d.max()) if d.size else 0.0
        assert worst <= elem_tol, f"per-element |dy| / sum|w x| = {worst:.3e} > {elem_tol:.0e}"
        # entries whose terms are all zero must come out zero
        z = ok & (mag == 0)
        assert np.all(got[z] == 0), "a row with no nonzero term is not zero"
    return r


def magnitude(Wdec, x):
    """sum_i |W[o][i] x[t][i]| as f64 [S][O] (Wdec the oracle's decoded weights)."""
    x = np.asarray(x, np.float64).reshape(-1, np.asarray(Wdec).shape[1])
    return np.abs(x) @ np.abs(np.asarray(Wdec, np.float64)).T


def guarded(torch, n, dtype, pad=256, fill=None):
    """A buffer of n elements with `pad` canary elements before and after:
    returns (view of the n elements, whole buffer, canary value)."""
    if dtype == torch.uint8:
        fill = 0xA5 if fill is None else fill
    elif dtype in (torch.int32, torch.int8):
        fill = -77 if fill is None else fill
    else:
        fill = -7.25 if fill is None else fill
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf[pad:pad + n], buf, fill


def assert_guard_intact(buf, n, fill, pad=256):
    """The canaries around a guarded buffer are untouched."""
    b = host(buf)
    head, tail = b[:pad], b[pad + n:]
    assert np.all(head == fill) and np.all(tail == fill), "a write landed outside the output"


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
