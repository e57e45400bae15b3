"""Derivation of the rational erf approximation used by the GELU epilogue.

GELU(z) = 0.5 z (1 + erf(z / sqrt 2)) needs erf in fp32 on every GEMM output.
The kernels evaluate

    erf(z / sqrt 2) ~= zc * P(zc^2) / Q(zc^2),  zc = clamp(z, -4 sqrt 2, 4 sqrt 2)

with P of degree 5 and Q of degree 5 (Q(0) = 1) in zc^2.  Beyond |z| = 4 sqrt 2
erf(z / sqrt 2) is +-1 to within 2^-26, so the clamp is exact in fp32.  The
coefficients below were fitted here by linearised least squares on the
relative error of erf(z/sqrt2)/z (Loeb's linearisation, P - f (Q - 1) = f),
with Lawson's iteratively reweighted scheme driving the fit toward the
minimax error; every coefficient comes out positive, so the Horner
evaluation has no cancellation.  Result: 2.5e-8 relative error in fp64 on
the fit interval; 3.3e-7 absolute on erf and 8.7e-7 on GELU (relative, floor
1) when evaluated in fp32 with FMAs and a 1-ulp reciprocal.

A second, shorter fit (P of degree 3, Q of degree 4, same method) serves
the epilogues whose output is bf16 or fp16: 5.1e-6 relative error in fp64,
2.1e-5 absolute on GELU in fp32 -- under 0.03 of an output ulp at |y| = 1
(bf16 ulp 2^-7, fp16 2^-10) -- for 13 VALU operations instead of 16.

    python -m mlp_megakernel_amd.erf_fit      # refits and prints the tables
"""
import numpy as np


def fit(npq: int = 6, nq: int = 5, c: float = 4.0 * np.sqrt(2.0), iters: int = 80):
    from scipy.special import erf
    z = np.cos(np.linspace(0, np.pi, 8000)) * 0.5 * c + 0.5 * c
    z = np.concatenate([z, np.linspace(0, c, 8000)])
    z = z[z > 1e-6]
    u = z * z
    f = erf(z / np.sqrt(2.0)) / z
    Q = np.ones_like(u)
    w = np.ones_like(u)
    for _ in range(iters):
        cols = [u ** i for i in range(npq)] + [-f * u ** j for j in range(1, nq + 1)]
        A = np.stack(cols, 1) / (f * Q)[:, None]
        b = f / (f * Q)
        sw = np.sqrt(w)
        sol, *_ = np.linalg.lstsq(A * sw[:, None], b * sw, rcond=None)
        p = sol[:npq]
        q = np.concatenate([[1.0], sol[npq:]])
        Qn = np.polyval(q[::-1], u)
        err = np.abs(np.polyval(p[::-1], u) / Qn - f) / f
        w = w * (err / err.max() + 1e-3)
        w /= w.mean()
        Q = Qn
    return p, q, float(err.max())


if __name__ == "__main__":
    for npq, nq, what in ((6, 5, "fp32 outputs"), (4, 4, "16-bit outputs")):
        p, q, e = fit(npq, nq)
        print("%s: max relative error (fp64): %.3e" % (what, e))
        print("P:", ", ".join("%.9ef" % v for v in p))
        print("Q:", ", ".join("%.9ef" % v for v in q))
