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
