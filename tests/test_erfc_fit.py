"""The GeLU epilogues' normal CDF and density (csrc/common.h): erfc(x) =
t * P(t) * exp(-x^2), t = 1 / (1 + p x), with P fitted by csrc/fit_erfc.py.

The constants pasted into common.h are read back from the header, checked to
be the fit script's output, and evaluated in float32 in the kernels' order
(Horner in t, one exponential) against scipy's erfc and the exact GeLU and
its derivative (u * Phi(u) and Phi(u) + u * phi(u), Phi from erfc).  The
bounds are the ones the header states; they are far below bf16's 2^-8 (unit roundoff)
rounding of the epilogue's outputs."""
import os
import re
import sys

import numpy as np
from scipy.special import erfc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "megatron_tensor_transformer_rank_amd", "csrc")


def header_constants():
    text = open(os.path.join(CSRC, "common.h")).read()
    p = float(re.search(r"ERFC_P\s*=\s*([0-9.eE+-]+)f", text).group(1))
    body = re.search(r"ERFC_C\[8\]\s*=\s*\{([^}]*)\}", text).group(1)
    c = [float(v.strip().rstrip("f")) for v in body.split(",")]
    assert len(c) == 8
    return p, np.array(c)


def cdf_pdf_f32(u, p, c):
    """The device code's arithmetic, in float32."""
    f = np.float32
    u = np.asarray(u, f)
    x = (np.abs(u) * f(0.70710678118654752)).astype(f)
    t = (f(1) / (f(p) * x + f(1))).astype(f)
    acc = np.full_like(t, f(c[7]))
    for i in range(6, -1, -1):
        acc = (acc * t + f(c[i])).astype(f)
    e = np.exp((f(-0.5) * u * u).astype(f)).astype(f)
    q = (f(0.5) * (acc * t) * e).astype(f)
    cdf = np.where(u >= 0, f(1) - q, q).astype(f)
    pdf = (f(0.39894228040143268) * e).astype(f)
    return cdf, pdf, q


def test_constants_are_the_fit():
    sys.path.insert(0, CSRC)
    try:
        import fit_erfc
    finally:
        sys.path.remove(CSRC)
    p, c = header_constants()
    assert p == fit_erfc.P_SCALE
    np.testing.assert_allclose(c, fit_erfc.fit(), rtol=1e-8, atol=1e-9)


def test_erfc_relative_error():
    p, c = header_constants()
    u = np.concatenate([np.linspace(-12.7, 0, 400001), np.geomspace(-12.7, -1e-7, 20001)]).astype(np.float32)
    _, _, q = cdf_pdf_f32(u, p, c)
    ref = 0.5 * erfc(np.abs(u.astype(np.float64)) / np.sqrt(2))
    x = np.abs(u) / np.sqrt(2)
    rel = np.abs(q / ref - 1)
    assert rel[x <= 4].max() <= 2e-6
    assert rel[(x > 4) & (x <= 9)].max() <= 6e-6


def test_gelu_and_derivative_against_exact():
    p, c = header_constants()
    u = np.linspace(-12, 12, 200001).astype(np.float32)
    cdf, pdf, _ = cdf_pdf_f32(u, p, c)
    u64 = u.astype(np.float64)
    Phi = 0.5 * erfc(-u64 / np.sqrt(2))
    phi = np.exp(-0.5 * u64 * u64) / np.sqrt(2 * np.pi)
    gelu = u64 * cdf.astype(np.float64)
    grad = (u.astype(np.float32) * pdf + cdf).astype(np.float64)
    # relative to the function's scale: far below the bf16 rounding (2^-8) of the outputs
    assert np.abs(gelu - u64 * Phi).max() <= 2e-6 * np.maximum(np.abs(u64 * Phi), 1e-3).max()
    m = np.abs(u64) > 1e-3
    assert np.max(np.abs(gelu - u64 * Phi)[m] / np.abs(u64 * Phi)[m]) <= 5e-6
    assert np.abs(grad - (Phi + u64 * phi)).max() <= 2e-6
    # the closed forms the oracle is pinned to
    for v, want in ((1.0, 0.8413447460685429), (-1.0, -0.15865525393145707), (2.0, 1.9544997361036416)):
        cd, _, _ = cdf_pdf_f32(np.float32(v), p, c)
        assert abs(float(v) * float(cd) - want) <= 2e-6 * abs(want)
