"""Error metrics used to compare a result against the oracle (test infrastructure).

``max_rel_err`` is the gate: max_i |y_i - o_i| / max(|o_i|, rms(o)).  The
floor at rms(o) follows the "Coalesce" README (sections "Triton port" and
"Notes for future sessions"): a plain elementwise relative error is decided
by near-zero entries, where it says nothing about the kernel, so the
denominator never drops below the typical magnitude of the output.

``rel_frobenius`` is the page's own norm ratio ||y - o||_2 / ||o||_2, reported
beside the gate.
"""
from __future__ import annotations

import numpy as np


def rms(o) -> float:
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    return float(np.sqrt(np.mean(o * o)))


def max_rel_err(y, o, floor: float | None = None) -> float:
    """max |y - o| / max(|o|, floor), floor = rms(o) unless given."""
    y = np.asarray(y, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if y.shape != o.shape:
        raise ValueError("shape mismatch %s vs %s" % (y.shape, o.shape))
    if o.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    f = rms(o) if floor is None else float(floor)
    den = np.maximum(np.abs(o), f)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(y - o) / den))


def rel_frobenius(y, o) -> float:
    y = np.asarray(y, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    n = float(np.linalg.norm(o.ravel()))
    d = float(np.linalg.norm((y - o).ravel()))
    return d / n if n > 0 else d


def nonfinite(y) -> int:
    return int(np.size(y) - np.count_nonzero(np.isfinite(np.asarray(y, dtype=np.float64))))
