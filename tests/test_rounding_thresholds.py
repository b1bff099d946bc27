"""Host check of the quantizer kernels' division-free rounding decision.

SpeCache summary §3 gives the codes as the rounded ratio (x - z) / s; the
kernels (quantize.hip, Coder) decide floor(q + 1/2) for the float32 quotient
q = RN(RN(x - z) / s) without dividing: q >= t (t = 1/2, 3/2, 5/2) exactly when
RN(d - t s) >= -h s, d = RN(x - z), h half the float32 gap just below t.  This
test restates that decision in numpy and compares it with the division on
random and tie-adjacent float16 inputs, so a wrong threshold fails here
without a GPU.  (For t = 1/2 the quotient of float16-derived operands never
falls within 2^-25 below t, so there h is pinned by its definition, checked
in the second test, rather than by the comparison.)
"""
import numpy as np
import pytest

H = {0.5: 2.0 ** -26, 1.5: 2.0 ** -24, 2.5: 2.0 ** -23}


def _division_codes(x, z, s, bits):
    d = x.astype(np.float32) - z.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = d / s.astype(np.float32)
    code = np.floor(q.astype(np.float64) + 0.5)
    code = np.where(s == 0, 0, np.clip(np.nan_to_num(code), 0, (1 << bits) - 1))
    return code.astype(np.int64)


def _threshold_codes(x, z, s, bits):
    sf = s.astype(np.float32)
    d = x.astype(np.float32) - z.astype(np.float32)
    code = np.zeros(x.shape, dtype=np.int64)
    for t in ([0.5] if bits == 1 else [0.5, 1.5, 2.5]):
        # one rounding of the exact d - t s (t s is exact; near the threshold so is the difference)
        a = (d.astype(np.float64) - t * sf.astype(np.float64)).astype(np.float32)
        code += (a >= -sf * np.float32(H[t])).astype(np.int64)
    return np.where(sf == 0, 0, code)


@pytest.mark.parametrize("bits", [1, 2])
def test_threshold_decision_equals_division(bits):
    rng = np.random.default_rng(5 + bits)
    n = 200_000
    s = (np.abs(rng.standard_normal(n)) * 10.0 ** rng.uniform(-6, 4, n)).astype(np.float16)
    z = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n)).astype(np.float16)
    t = rng.choice([0.5, 1.5, 2.5, 1.0, 3.0, -0.5], n) + rng.uniform(-1e-3, 1e-3, n) * rng.choice([1, 1e-3, 0], n)
    with np.errstate(over="ignore", invalid="ignore"):
        x = (z.astype(np.float64) + s.astype(np.float64) * t).astype(np.float16)
    ok = np.isfinite(x) & np.isfinite(s) & np.isfinite(z)
    x, z, s = x[ok], z[ok], s[ok]
    s[::97] = 0  # constant groups
    assert np.array_equal(_threshold_codes(x, z, s, bits), _division_codes(x, z, s, bits))


def test_threshold_h_is_half_the_gap_below_t():
    for t, h in H.items():
        below = np.nextafter(np.float32(t), np.float32(0))
        assert np.float64(t) - np.float64(below) == 2 * h
        # the midpoint rounds to t (ties to even): t's last mantissa bit is 0
        assert np.float32(np.float64(t) - h) == np.float32(t)
