"""Shared comparison helpers for the parity tests (no attention arithmetic)."""
import numpy as np
import torch

ATOL_F32, RTOL_F32 = 1e-5, 0.0
ATOL_BF16, RTOL_BF16 = 2e-2, 1e-2


def tol_for(dtype):
    return (ATOL_BF16, RTOL_BF16) if dtype == torch.bfloat16 else (ATOL_F32, RTOL_F32)


def to_f64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def report(got, ref):
    got, ref = to_f64(got), to_f64(ref)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = np.maximum(np.abs(ref), 1e-30)
    max_rel = float((err / denom).max()) if err.size else 0.0
    g, r = got.ravel(), ref.ravel()
    nr = np.linalg.norm(g) * np.linalg.norm(r)
    cos = float(g @ r / nr) if nr > 0 else 1.0
    return dict(max_abs=max_abs, max_rel=max_rel, cos=cos)


def assert_close(got, ref, dtype, what=""):
    """Pass iff |got - ref| <= atol + rtol*|ref| elementwise (all finite)."""
    atol, rtol = tol_for(dtype)
    g, r = to_f64(got), to_f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU output" % what
    bad = np.abs(g - r) > atol + rtol * np.abs(r)
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError("%s: %d of %d elements out of tolerance (atol %g rtol %g); "
                             "first %s; %s" % (what, int(bad.sum()), bad.size, atol, rtol,
                                               idx, report(g, r)))
    return report(g, r)
