"""Comparison of GPU outputs with the fp64 oracle (test infrastructure).

Tolerances (stated for the bf16 output O and the fp32 LSE):
  * max-abs |O_gpu - O_ref| <= 1e-2 over all compared elements;
  * relative L2 ||O_gpu - O_ref|| / ||O_ref|| <= 4e-3;
  * max |LSE_gpu - LSE_ref| <= 1e-3 over rows with a finite reference LSE;
  * a row with no allowed key must give exactly O = 0 and LSE = -inf;
  * no NaN anywhere.
Representability floor: for |O_ref| >= 4 the spacing of bf16 is 2^-5, so
correct rounding alone may be off by up to 2^-6 = 0.0156 > 1e-2.  An element
whose error exceeds 1e-2 is accepted only when |O_ref| >= 4 and its error is
at most half a bf16 spacing of O_ref plus 1e-3; such elements are counted and
reported (``floor_bound``), never hidden.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MAX_ABS = 1e-2
REL_L2 = 4e-3
MAX_DLSE = 1e-3


def bf16_half_spacing(x: np.ndarray) -> np.ndarray:
    """Half the distance between adjacent bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    e = np.floor(np.log2(ax))
    return 0.5 * np.exp2(e - 7)


def compare(got_o, got_lse, ref_o, ref_lse):
    """Return a metrics dict; raise AssertionError when the tolerances fail."""
    go = got_o.detach().float().cpu().numpy().astype(np.float64) if hasattr(got_o, "detach") else np.asarray(got_o, np.float64)
    gl = got_lse.detach().float().cpu().numpy().astype(np.float64) if hasattr(got_lse, "detach") else np.asarray(got_lse, np.float64)
    ref_o = np.asarray(ref_o, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    assert go.shape == ref_o.shape and gl.shape == ref_lse.shape, (go.shape, ref_o.shape)
    assert not np.isnan(go).any(), "NaN in O"
    assert not np.isnan(gl).any(), "NaN in LSE"
    empty = ~np.isfinite(ref_lse)
    assert np.all(gl[empty] == -np.inf), "an empty row did not get LSE = -inf"
    assert np.all(go[empty] == 0.0), "an empty row did not get O = 0"
    assert np.all(np.isfinite(gl[~empty])), "a non-empty row got a non-finite LSE"
    err = np.abs(go - ref_o)
    max_abs = float(err.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref_o))
    rel_l2 = float(np.linalg.norm(go - ref_o) / nref) if nref > 0 else float(np.linalg.norm(go))
    dlse = float(np.abs(gl[~empty] - ref_lse[~empty]).max()) if (~empty).any() else 0.0
    floor = np.abs(torch.from_numpy(ref_o).to(torch.bfloat16).double().numpy() - ref_o)
    over = err > MAX_ABS
    floor_ok = (np.abs(ref_o) >= 4.0) & (err <= bf16_half_spacing(ref_o) + 1e-3)
    metrics = {
        "max_abs": max_abs, "rel_l2": rel_l2, "max_dlse": dlse,
        "bf16_floor_max": float(floor.max()) if floor.size else 0.0,
        "floor_over_1e-2": int((floor > MAX_ABS).sum()),
        "over_1e-2": int(over.sum()), "floor_bound": int((over & floor_ok).sum()),
        "elements": int(err.size), "empty_rows": int(empty.sum()),
    }
    assert not np.any(over & ~floor_ok), f"max-abs above {MAX_ABS} beyond the bf16 floor: {metrics}"
    assert rel_l2 <= REL_L2, f"relative L2 above {REL_L2}: {metrics}"
    assert dlse <= MAX_DLSE, f"|dLSE| above {MAX_DLSE}: {metrics}"
    return metrics


def sample_rows(Lq: int, seed: int, block: int = 128, extra: int = 64):
    """Rows to check on a full-size problem: both ends, every block boundary
    region up to a cap, and seeded random rows."""
    rows = set(range(min(Lq, 40))) | set(range(max(0, Lq - 40), Lq))
    for b0 in range(block, Lq, block * max(1, Lq // (block * 16))):
        rows |= {b0 - 1, b0, b0 + 1, b0 + 31, b0 + 32}
    r = np.random.default_rng(seed)
    rows |= set(int(x) for x in r.integers(0, Lq, extra))
    return np.array(sorted(x for x in rows if 0 <= x < Lq), dtype=np.int64)
