"""The flush kernel forms each code's quotient (x - min) / s as a multiply by
the correctly rounded reciprocal 1 / s and takes the correctly rounded
division only where the product lies within 2^-12 of a half-integer.  This
checks, in IEEE binary32 on the CPU (numpy's float32 operations round
correctly), that the rule gives rne(fl(n / s)) for every n, s the quantizer
can meet: random groups of fp16 data, and quotients planted next to
half-integers, where the two roundings are most likely to part."""
import numpy as np

GUARD = np.float32(0.5) - np.float32(2.0 ** -12)


def _rule(n, s):
    r = np.float32(1.0) / s
    f = n * r
    t = np.rint(f)
    near = np.abs(f - t) > GUARD
    return np.where(near, np.rint(n / s), t), near


def _check(n, s):
    n = n.astype(np.float32)
    s = s.astype(np.float32)
    got, near = _rule(n, s)
    ref = np.rint(n / s)
    assert np.array_equal(got, ref)
    return near


def test_random_groups_of_fp16_data():
    rng = np.random.default_rng(7)
    for bits in (2, 4):
        levels = np.float32((1 << bits) - 1)
        for scale in (1e-3, 1.0, 40.0, 3000.0):
            x = (rng.standard_normal((4096, 64)) * scale).astype(np.float16).astype(np.float32)
            mn, mx = x.min(axis=1, keepdims=True), x.max(axis=1, keepdims=True)
            s = (mx - mn) / levels
            ok = (s > 0)[:, 0]
            _check((x - mn)[ok], np.broadcast_to(s, x.shape)[ok])


def test_quotients_next_to_half_integers():
    rng = np.random.default_rng(11)
    s = rng.uniform(1e-4, 1e3, 200000).astype(np.float32)
    k = rng.integers(0, 15, s.size).astype(np.float32)
    # n / s within a few ulps of k + 1/2, on both sides, and exactly on it
    base = ((k + np.float32(0.5)) * s).astype(np.float32)
    near_total = 0
    for d in range(-8, 9):
        n = base.copy()
        for _ in range(abs(d)):
            n = np.nextafter(n, np.float32(np.inf) if d > 0 else np.float32(0.0)).astype(np.float32)
        near_total += int(_check(n, s).sum())
    assert near_total > 0  # the division path is taken there


def test_symmetric_quotients():
    rng = np.random.default_rng(3)
    for c0 in (1.0, 7.0):
        x = (rng.standard_normal((4096, 32)) * 5.0).astype(np.float16).astype(np.float32)
        M = np.abs(x).max(axis=1, keepdims=True)
        s = M / np.float32(c0)
        _check(x, np.broadcast_to(s, x.shape))


def test_quotients_around_the_guard_band():
    """Quotients planted 2^-19 .. 2^-14 from half-integers, inside and outside
    the band where the division decides: everywhere the rule must give the
    correctly rounded quotient's integer (the bound behind the band is
    2^-18)."""
    rng = np.random.default_rng(5)
    s = rng.uniform(1e-4, 1e3, 100000).astype(np.float32)
    k = rng.integers(0, 15, s.size).astype(np.float32)
    for e in (-19, -18, -17, -16, -15, -14):
        for sign in (-1.0, 1.0):
            q = (k + np.float32(0.5) + np.float32(sign * 2.0 ** e)).astype(np.float32)
            _check((q * s).astype(np.float32), s)
