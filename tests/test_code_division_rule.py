"""CPU check of the rule the GPU row quantizer uses for its codes: the code
rint(fl32(x / s)) (fl32 = the correctly rounded fp32 quotient) equals
rint(q) for q = fl32(x * r), r = an approximate reciprocal of s within 1 ulp,
whenever q lies farther than 2^-20 * max(|q|, 1) from every half-integer
(elsewhere the kernel takes the correctly rounded division itself).  Checked
here on seeded fp32 operands of the quantizer's ranges, with r = the
correctly rounded reciprocal and its two fp32 neighbours (the worst a 1-ulp
reciprocal can be), including quotients next to ties."""
import numpy as np


def _rule_holds(x, s):
    x = x.astype(np.float32)
    s = s.astype(np.float32)
    exact = np.rint((x / s).astype(np.float32))  # numpy fp32 division is correctly rounded
    r0 = (np.float32(1.0) / s).astype(np.float32)
    for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
        q = (x * r).astype(np.float32)
        fr = q - np.floor(q)
        tol = np.maximum(np.abs(q), np.float32(1.0)) * np.float32(2.0 ** -20)
        fast = np.abs(fr - np.float32(0.5)) > tol
        assert np.array_equal(np.rint(q)[fast], exact[fast]), "fast path disagrees"
        assert fast.mean() > 0.99  # the division is the rare case


def test_rule_on_quantizer_ranges():
    rng = np.random.default_rng(20260)
    for levels in (3, 7, 15, 31, 63, 255):
        s = (rng.uniform(1e-3, 4.0, 200000) / levels).astype(np.float32)
        x = (rng.uniform(-0.01, 1.01, s.size) * levels * s).astype(np.float32)
        _rule_holds(x, s)


def test_rule_next_to_ties():
    rng = np.random.default_rng(20261)
    s = rng.uniform(1e-3, 1.0, 100000).astype(np.float32)
    k = rng.integers(0, 255, s.size).astype(np.float32)
    # quotients a few ulp either side of k + 0.5
    x = ((k + np.float32(0.5)) * s).astype(np.float32)
    for steps in range(-6, 7):
        xs = x.copy()
        for _ in range(abs(steps)):
            xs = np.nextafter(xs, np.float32(np.inf) if steps > 0 else np.float32(-np.inf))
        _rule_holds_near(xs, s)


def _rule_holds_near(x, s):
    exact = np.rint((x / s).astype(np.float32))
    r0 = (np.float32(1.0) / s).astype(np.float32)
    for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
        q = (x * r).astype(np.float32)
        fr = q - np.floor(q)
        tol = np.maximum(np.abs(q), np.float32(1.0)) * np.float32(2.0 ** -20)
        fast = np.abs(fr - np.float32(0.5)) > tol
        assert np.array_equal(np.rint(q)[fast], exact[fast])


def test_rule_with_subnormal_scales():
    # scales in the fp32 subnormal range (groups whose range is about 1e-38):
    # the reciprocal overflows, q = x * r is inf or NaN, and the exponent-bit
    # test sends the code to the correctly rounded division; where q stays
    # finite the rule above still holds
    rng = np.random.default_rng(20262)
    s = (rng.uniform(1e-45, 1.2e-38, 100000)).astype(np.float32)
    s = s[s > 0]
    x = (rng.uniform(0.0, 1.0, s.size) * 15 * s).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        exact = np.rint((x / s).astype(np.float32))
        r = (np.float32(1.0) / s).astype(np.float32)
        q = (x * r).astype(np.float32)
        nonfinite = (q.view(np.uint32) & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
        assert nonfinite.any() and np.array_equal(nonfinite, ~np.isfinite(q))
        fr = q - np.floor(q)
        tol = np.maximum(np.abs(q), np.float32(1.0)) * np.float32(2.0 ** -20)
        fast = ~nonfinite & (np.abs(fr - np.float32(0.5)) > tol)
    assert np.array_equal(np.rint(q)[fast], exact[fast])
