"""The bound behind the quantizer's division-free codes, checked in binary32
arithmetic on the CPU (numpy float32 operations are IEEE-rounded).

The GPU quantizer computes t = fl(x * fl(1/s)) and keeps rint(t) whenever t is
farther than 2^-15 from every half-integer; only the other elements take the
correctly rounded quotient fl(x / s).  The claim checked here: whenever that
margin test passes, clamp(rint(t)) equals clamp(rint(fl(x / s))), the code the
quantizer's definition asks for (README "Quick start": int8 activations;
rounding half to even of the correctly rounded quotient is the reading taken).
"""
import numpy as np

MARGIN = np.float32(0.5) - np.float32(2.0 ** -15)


def _codes(x, s):
    r = np.float32(1.0) / s
    t = x * r
    n = np.rint(t)
    fast = np.abs(t - n) < MARGIN
    exact = np.rint(x / s)
    return fast, np.clip(n, -127, 127), np.clip(exact, -127, 127)


def test_margin_test_implies_the_exact_code_random():
    rng = np.random.default_rng(5)
    total_fast = 0
    for _ in range(40):
        s = np.float32(rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-120, 120)))
        # |x / s| up to 130: the quantizer's own range plus a little saturation
        x = (rng.uniform(-130.0, 130.0, 200000) * np.float64(s)).astype(np.float32)
        fast, n, exact = _codes(x, s)
        assert np.array_equal(n[fast], exact[fast])
        total_fast += int(fast.sum())
    assert total_fast > 0.99 * 40 * 200000


def test_margin_test_implies_the_exact_code_near_ties():
    """Values on and a few ulps around (k + 1/2) s, where t and fl(x / s) can round apart."""
    rng = np.random.default_rng(6)
    caught = 0
    for _ in range(200):
        s = np.float32(rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-100, 100)))
        k = rng.integers(-128, 128, 4000)
        base = ((k + 0.5) * np.float64(s)).astype(np.float32)
        xs = [base]
        up, down = base.copy(), base.copy()
        for _ in range(6):
            up = np.nextafter(up, np.float32(np.inf))
            down = np.nextafter(down, np.float32(-np.inf))
            xs += [up.copy(), down.copy()]
        x = np.concatenate(xs)
        fast, n, exact = _codes(x, s)
        assert np.array_equal(n[fast], exact[fast])
        caught += int((~fast).sum())
    assert caught > 0   # the margin does send elements to the exact quotient


def test_saturating_and_extreme_values():
    for s in (np.float32(2.0 ** -126), np.float32(2.0 ** 126), np.float32(0.0170001), np.float32(3.0e-3)):
        x = np.array([np.float32(3.0e38), np.float32(-3.0e38), np.float32(1e-45), np.float32(-1e-45),
                      np.float32(0.0), np.float32(-0.0)] + [np.float32(v) * s for v in (127.4, 127.6, -127.6, 128.0,
                                                                                       129.5, -4096.0)],
                     np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            fast, n, exact = _codes(x, s)
        assert np.array_equal(n[fast], exact[fast])
