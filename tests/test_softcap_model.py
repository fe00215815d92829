"""CPU model of the prefill kernel's soft cap for caps up to 64, c * tanh(x / c) formed as
c - 2c / (2^(x * 2 log2(e) / c) + 1) in fp32 with x and c in log2 units.
The form cancels near x = 0 in relative terms; these tests bound its
absolute error (what the softmax sees) over the score range, with the
exponential and the reciprocal each perturbed by one unit in the last place
(the hardware's v_exp_f32 and v_rcp_f32 are accurate to about that)."""
import numpy as np
import pytest

LOG2E = 1.4426950408889634


def capped(x, cap, k2, ulp_e=0, ulp_r=0):
    f = np.float32
    e2 = np.exp2((x * k2).astype(f)).astype(f)
    if ulp_e:
        e2 = np.nextafter(e2, np.float32(np.inf) if ulp_e > 0 else np.float32(-np.inf)).astype(f)
    r = (f(1) / (e2 + f(1))).astype(f)
    if ulp_r:
        r = np.nextafter(r, np.float32(np.inf) if ulp_r > 0 else np.float32(-np.inf)).astype(f)
    return (f(-2) * cap * r + cap).astype(f)


@pytest.mark.parametrize("cap_nat", [0.5, 2.0, 5.0, 20.0, 50.0, 200.0])
@pytest.mark.parametrize("ulps", [(0, 0), (1, 1), (-1, -1), (1, -1), (-1, 1)])
def test_softcap_absolute_error(cap_nat, ulps):
    cap = np.float32(cap_nat * LOG2E)
    k2 = np.float32(2.0 / cap_nat)
    x = np.concatenate([np.linspace(-6 * cap, 6 * cap, 400001),
                        np.logspace(-12, 1, 20000) * cap, -np.logspace(-12, 1, 20000) * cap]).astype(np.float32)
    got = capped(x, cap, k2, *ulps).astype(np.float64)
    exact = float(cap) * np.tanh(x.astype(np.float64) / float(cap))
    err = np.abs(got - exact)
    assert np.all(np.isfinite(got))
    assert float(err.max()) <= 6e-7 * float(cap), float(err.max())
    # the cap bounds the result
    assert float(np.abs(got).max()) <= float(cap) * (1 + 1e-6)


def test_softcap_saturates_without_overflow():
    cap = np.float32(50 * LOG2E)
    k2 = np.float32(2.0 / 50)
    x = np.array([-1e30, -1e6, 1e6, 1e30, np.float32(3e38)], np.float32)
    with np.errstate(over="ignore"):
        got = capped(x, cap, k2)
    assert np.allclose(got, [-cap, -cap, cap, cap, cap], rtol=1e-6)


def tanh_poly_coefficients():
    """The coefficients the prefill kernel's polynomial soft cap uses (attn_kernels.h)."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "online_softmax_fusion_amd", "csrc",
                            "attn_kernels.h")).read()
    m = re.search(r"kTanhPoly\[4\]\s*=\s*\{([^}]*)\}", src)
    assert m, "kTanhPoly not found"
    return [float(v.strip().rstrip("f")) for v in m.group(1).split(",")]


def fma32(a, b, c):
    # a * b is exact in float64 for float32 operands; one rounding to float32 after the add
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


@pytest.mark.parametrize("cap_nat", [0.5, 5.0, 20.0, 50.0, 64.0])
@pytest.mark.parametrize("scale", [0.0883883, 0.125, 1.0, 3.0])
def test_softcap_polynomial_form(cap_nat, scale):
    """The polynomial form on the raw score s (what the q @ k product gives):
    capped (log2 units) = s * P(s^2), P's coefficients scale_log2 * c_i * k^i with
    k = (scale / softcap)^2, used while |s| <= 0.5 softcap / scale, i.e.
    |tanh argument| <= 1/2.  Its absolute error stays below 3e-7 of the cap in
    log2 units (half the exp form's bound), with fp32 evaluation as on the device."""
    c = tanh_poly_coefficients()
    sc = np.float32(scale * LOG2E)
    k = (scale / cap_nat) ** 2
    q = [np.float32(float(sc) * c[i] * k ** i) for i in range(4)]
    s0 = 0.5 * cap_nat / scale
    s = np.concatenate([np.linspace(-s0, s0, 200001), np.logspace(-9, 0, 5000) * s0,
                        -np.logspace(-9, 0, 5000) * s0]).astype(np.float32)
    w = (s * s).astype(np.float32)
    qv = [np.full_like(s, v) for v in q]
    poly = fma32(fma32(fma32(qv[3], w, qv[2]), w, qv[1]), w, qv[0])
    got = (s.astype(np.float64) * poly.astype(np.float64)).astype(np.float32).astype(np.float64)
    cap_l2 = cap_nat * LOG2E
    exact = cap_l2 * np.tanh(s.astype(np.float64) * scale / cap_nat)
    err = np.abs(got - exact)
    assert float(err.max()) <= 3e-7 * cap_l2, (float(err.max()), 3e-7 * cap_l2)


def test_tanh_polynomial_range():
    """The fit itself against tanh on |y| <= 1/2 (1.3e-7 absolute) and its
    failure well outside (so the kernel's range check is needed)."""
    c = np.array(tanh_poly_coefficients())
    y = np.linspace(0, 0.5, 100001)
    p = y * np.polyval(c[::-1], y * y)
    assert float(np.abs(p - np.tanh(y)).max()) <= 1.3e-7
    y2 = np.array([1.5])
    assert abs(float(y2 * np.polyval(c[::-1], y2 * y2)) - float(np.tanh(y2))) > 1e-3
