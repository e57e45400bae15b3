"""Shared helpers of the GPU parity tests (test infrastructure)."""
import numpy as np
import torch

import datagen
import oracle
from oracle.compare import max_rel_err, nonfinite, rel_frobenius

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-2}


def f64(t):
    return datagen.to_f64(t)


def to_gpu(t, padded=True):
    import mlp_megakernel_amd as mk
    if t.dim() == 2 and padded:
        return mk.aligned_copy(t, "cuda")
    return t.to("cuda")


def assert_close(y, o, tol, what=""):
    y = np.asarray(y, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert nonfinite(y) == 0, "%s: non-finite outputs" % what
    e = max_rel_err(y, o)
    assert e <= tol, "%s: max rel err %.3e > %.1e (rel frobenius %.3e)" % (what, e, tol, rel_frobenius(y, o))
    return e


def progress(msg):
    print(msg, flush=True)
