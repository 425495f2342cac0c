"""Helpers of the GPU parity tests: device transfer, the selection tie-band
rule, and the output error metrics."""
from __future__ import annotations

import sys

import numpy as np

# Output bar (bf16 inputs, fp32 accumulation).
MAX_ABS = 2e-2
REL_L2 = 1e-3
TIE_REL = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_u16(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_selection(s: np.ndarray, K: int, sK: float, sK1: float, got: np.ndarray, nsel: int):
    """Validate a selection against the oracle's fp64 scores of one row.

    Several selections are correct when scores tie within the band: the set
    must hold min(K, nc) distinct ascending blocks < nc, every block scoring
    above sK + delta, and none scoring below sK - delta, where
    delta = 1e-4 * max(|sK|, |sK+1|).  Returns True when the set differs from
    the strict (score desc, index asc) top-K (a tie-band exemption).
    """
    nc = s.size
    want_n = min(K, nc)
    assert nsel == want_n, (nsel, want_n)
    g = got[:nsel]
    assert np.all(got[nsel:] == -1)
    if nsel:
        assert g.min() >= 0 and g.max() < nc
        assert np.all(np.diff(g) > 0), "selection not strictly ascending"
    if nc <= K:
        assert np.array_equal(g, np.arange(nc))
        return False
    delta = TIE_REL * max(abs(sK), abs(sK1))
    inset = np.zeros(nc, dtype=bool)
    inset[g] = True
    must = s > sK + delta
    banned = s < sK - delta
    assert not np.any(must & ~inset), "a block clearly above the K-th score was dropped"
    assert not np.any(banned & inset), "a block clearly below the K-th score was taken"
    order = np.lexsort((np.arange(nc), -s))
    strict = np.sort(order[:K])
    return not np.array_equal(strict, g)


def out_errors(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, what=""):
    m, r = out_errors(got, ref)
    log(f"  {what}: max-abs {m:.3e}  rel-L2 {r:.3e}")
    assert m <= MAX_ABS and r <= REL_L2, (what, m, r)
    return m, r
