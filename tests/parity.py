"""Parity bars used by the GPU tests (the oracle is the reference).

Per tensor X (an output o or a final state) against the fp64 oracle R, with
eps = max|X - R| and M = max|R|:
  fp32 inputs:  eps <= 1e-5 * max(1, M)
  bf16 inputs:  eps <= 2e-3 * M
"""
import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-3}


def max_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0, 0.0
    return float(np.max(np.abs(x - ref))), float(np.max(np.abs(ref)))


def check(x, ref, dtype, what=""):
    eps, M = max_err(x, ref)
    assert np.all(np.isfinite(np.asarray(x, dtype=np.float64))), "%s: non-finite values" % what
    bound = TOL[dtype] * (max(1.0, M) if dtype == "f32" else M)
    assert eps <= bound, "%s: max|err| = %.3e > %.3e (max|ref| = %.3e)" % (what, eps, bound, M)
    return eps, M
