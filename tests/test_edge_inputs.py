"""CPU check that the flush kernel's edge-case inputs (tests/edge_inputs.py)
contain what they claim: exact half-integer quotients, quotients within 2^-12
of one, constant and signed-zero groups, fp16 subnormals and the largest
finite values -- so the device test does exercise those paths."""
import numpy as np

import oracle
from edge_inputs import NPAT, edge_kv, group


def _quotients(g, bits):
    g = g.astype(np.float32)
    mn, mx = np.float32(g.min() + np.float32(0.0)), g.max()
    s = np.float32((mx - mn) / np.float32((1 << bits) - 1))
    return (g - mn) / s if s > 0 else None


def test_patterns_plant_their_cases():
    rng = np.random.default_rng(0)
    for bits in (2, 4):
        ties = near = 0
        for _ in range(20):
            q = _quotients(group(0, rng, 32, bits, "f32"), bits)
            ties += int(np.sum(q - np.floor(q) == np.float32(0.5)))
            q = _quotients(group(1, rng, 32, bits, "f16"), bits)
            d = np.abs(q - (np.floor(q) + np.float32(0.5)))
            near += int(np.sum((d > 0) & (d < 2.0 ** -12)))
        assert ties > 100 and near > 50, (bits, ties, near)
    c = group(2, rng, 32, 2, "f32")
    assert np.all(c == c[0])
    z = group(3, rng, 64, 2, "f32")
    assert np.all(z == 0) and np.any(np.signbit(z)) and not np.all(np.signbit(z))
    m = group(4, rng, 64, 2, "f32")
    assert m.min() == 0 and np.any(np.signbit(m[m == 0]))
    sub = group(5, rng, 64, 2, "f16")
    assert np.all(np.abs(sub) < 2.0 ** -14) and np.any(sub != 0)
    ext = group(6, rng, 64, 4, "f16")
    assert ext.max() == 65504 and ext.min() == -65504
    assert group(6, rng, 64, 4, "bf16").max() == 65280


def test_oracle_codes_round_ties_to_even():
    """On a planted-tie group the oracle's codes are the round-half-even ones
    of the exact quotients (closed form), so a device match means the kernel
    took the ties the same way."""
    rng = np.random.default_rng(1)
    for bits in (2, 4):
        for _ in range(10):
            g = group(0, rng, 64, bits, "f32")
            codes, s, mn, _, _ = oracle.quantize_group(g, bits)
            q = (g - mn) / s
            assert np.array_equal(codes, np.rint(q).astype(np.uint16))  # numpy rint: half to even
            assert np.any(q - np.floor(q) == 0.5)


def test_edge_tensors_are_finite_and_in_range():
    K, V = edge_kv(1, 2, 32 * 3 + 5, 64, 32, 2, 4, "f32", 3)
    for X in (K, V):
        assert np.all(np.isfinite(X)) and np.abs(X).max() <= 65504
    assert NPAT == 8
