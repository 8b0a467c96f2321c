"""Coefficients of the erfc exponent polynomial that the GEMM epilogues' GELU evaluates (gemm.hip,
gelu_erf).  Not imported by anything: run it to regenerate or check the constants.

Form (the erfc approximation of W. H. Press et al., Numerical Recipes, section 6.2): with z >= 0 and
t = 1 / (1 + z/2),

    erfc(z) / 2 = t * 2^(-z^2 log2(e) + P(t)),   P(t) = log2(erfcx(z) / (2 t)),

erfcx(z) = exp(z^2) erfc(z) the scaled complement.  P is smooth on (0, 1]; it is fitted here as a
degree-7 polynomial, minimax in absolute error (log2 units, i.e. relative error of erfc) by Lawson's
iteratively reweighted least squares, over t for z in [0, 9.5].  Past z = 9.5 the GELU of a negative
input underflows fp32 and 1 - erfc/2 of a positive one rounds to 1, so the range stops there (the
polynomial stays between -2.83 and -2.56 below it, so the exponent still goes to 0).

    python quantized_video_diffusion_amd/csrc/gelu_erfc_fit.py
"""
import numpy as np
from scipy.special import erfcx

Z_MAX = 9.5
DEGREE = 7


def p_exact(t):
    z = 2.0 * (1.0 / t - 1.0)
    return np.log2(erfcx(z) / (2.0 * t))


def lawson(n, a, b, iters=2000, nodes=4000):
    x = 0.5 * (a + b) + 0.5 * (b - a) * np.cos(np.linspace(0.0, np.pi, nodes))
    f = p_exact(x)
    V = np.vander(x, n + 1, increasing=True)
    w = np.full(x.shape, 1.0 / nodes)
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(V * sw[:, None], f * sw, rcond=None)
        e = np.abs(V @ c - f)
        w = w * e
        w /= w.sum()
    return c


def main():
    t_min = 1.0 / (1.0 + Z_MAX / 2.0)
    c = lawson(DEGREE, t_min, 1.0)
    t = np.linspace(t_min, 1.0, 200001)
    err = np.abs(np.polyval(c[::-1], t) - p_exact(t)).max()
    print(f"degree {DEGREE} on z in [0, {Z_MAX}]: max |P error| {err:.3e} (log2) = relative error of erfc "
          f"{err * np.log(2):.2e}")
    print("coefficients c0 .. c%d (P(t) = sum c_k t^k):" % DEGREE)
    print(", ".join(f"{v:.9g}" for v in c))


if __name__ == "__main__":
    main()
