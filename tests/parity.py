"""Comparison helpers shared by the GPU parity tests (imported, not collected).

The bar, both parts required, computed in fp64 after decoding both fp16 results:
  * relative Frobenius error  ||G - R||_F / ||R||_F <= 5e-3
    (if ||R||_F == 0: ||G - R||_F <= 5e-3 * sqrt(#elements));
  * per element               |G - R| <= 1e-2 * (1 + |R|);
  * no NaN or Inf in G where R is finite.
"""
from __future__ import annotations

import numpy as np
import torch

REL_FRO = 5e-3
ELEM_ABS = 1e-2


def f64(x) -> np.ndarray:
    """fp16 tensor (any device) or uint16 bit array -> float64 numpy array."""
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy().astype(np.float64)
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.float16)
    return x.astype(np.float64)


def parity_report(got, ref) -> dict:
    G, R = f64(got), f64(ref)
    assert G.shape == R.shape, (G.shape, R.shape)
    d = G - R
    nr = np.linalg.norm(R)
    nd = np.linalg.norm(d)
    rel = nd / nr if nr > 0 else nd / max(np.sqrt(R.size), 1.0)
    bound = ELEM_ABS * (1.0 + np.abs(R))
    viol = np.abs(d) > bound
    finite_bad = (~np.isfinite(G)) & np.isfinite(R)
    return {
        "rel_fro": float(rel),
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "max_scaled": float(np.max(np.abs(d) / bound)) if d.size else 0.0,
        "n_violations": int(viol.sum()),
        "n_nonfinite": int(finite_bad.sum()),
        "first_violation": tuple(int(v) for v in np.argwhere(viol | finite_bad)[0])
        if (viol | finite_bad).any() else None,
    }


def assert_parity(got, ref, what: str = "") -> dict:
    r = parity_report(got, ref)
    ok = r["rel_fro"] <= REL_FRO and r["n_violations"] == 0 and r["n_nonfinite"] == 0
    assert ok, "parity failed %s: %s" % (what, r)
    return r


def assert_bitexact(got, ref_bits, what: str = ""):
    g = got.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    r = np.asarray(ref_bits)
    if r.dtype == np.float16:
        r = r.view(np.uint16)
    # +0 and -0 compare equal
    gz = (g & 0x7FFF) == 0
    rz = (r & 0x7FFF) == 0
    same = (g == r) | (gz & rz)
    if not same.all():
        idx = tuple(int(v) for v in np.argwhere(~same)[0])
        raise AssertionError("bit mismatch %s at %s: got %#06x want %#06x (%d elements differ)"
                             % (what, idx, int(g[idx]), int(r[idx]), int((~same).sum())))
