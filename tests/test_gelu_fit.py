"""The GELU of the GEMM epilogues takes its erfc exponent polynomial from csrc/gelu_erfc_fit.py: the
constants in gemm.hip are that script's output, and the form they are used in reaches the stated
accuracy against scipy's erfc (the function the oracle's GELU rests on) over the fitted range."""
import os
import re
import runpy

import numpy as np
from scipy.special import erfc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_video_diffusion_amd", "csrc")


def _kernel_coefficients():
    src = open(os.path.join(CSRC, "gemm.hip")).read()
    body = src[src.index("QVD_DEV float gelu_erf(float y)"):]
    body = body[:body.index("\n}\n")]
    # Horner from the highest coefficient: fmaf(c7, t, c6), then fmaf(p, t, c_k) down to c0
    first = re.search(r"fmaf\((-?[\d.e-]+)f, t, (-?[\d.e-]+)f\)", body)
    rest = re.findall(r"p = fmaf\(p, t, (-?[\d.e-]+)f\)", body)
    hi_to_lo = [float(first.group(1)), float(first.group(2))] + [float(v) for v in rest]
    return np.array(hi_to_lo[::-1])


def test_kernel_constants_are_the_fit():
    fit = runpy.run_path(os.path.join(CSRC, "gelu_erfc_fit.py"))
    t_min = 1.0 / (1.0 + fit["Z_MAX"] / 2.0)
    c = fit["lawson"](fit["DEGREE"], t_min, 1.0)
    k = _kernel_coefficients()
    assert len(k) == fit["DEGREE"] + 1
    np.testing.assert_allclose(k, c, rtol=1e-8, atol=1e-9)


def test_erfc_form_accuracy_over_the_range():
    """erfc(z) / 2 = t 2^(-z^2 log2 e + P(t)) with the kernel's constants, in float64: relative error
    below 7e-7 for z in [0, 9.5]; past it the exponent still falls (P stays in [-2.9, -2.5])."""
    c = _kernel_coefficients()
    z = np.linspace(0.0, 9.5, 200001)
    t = 1.0 / (1.0 + z / 2.0)
    h = t * np.exp2(-z * z * np.log2(np.e) + np.polyval(c[::-1], t))
    rel = np.abs(h - erfc(z) / 2.0) / (erfc(z) / 2.0)
    assert rel.max() < 7e-7, rel.max()
    tail = np.polyval(c[::-1], np.linspace(1e-9, t.min(), 1001))
    assert tail.min() > -2.9 and tail.max() < -2.5
