"""Pins for the CPU oracle: checks against things other than the oracle itself
(library routines, closed forms printed on the pages, invariants, brute force
in exact arithmetic).  CPU only."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- conversions
def test_f16_to_f32_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_probe_values():
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(200000).astype(np.float32) * np.float32(s) for s in (1e-6, 1e-4, 1e-2, 1, 100, 3e4)]
    # every binary16 value and every midpoint between neighbours (exact ties), nudged both ways
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    vals += [h.astype(np.float32), mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))]
    special = np.array([65504, 65519.996, 65520, 65536, 1e9, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -26,
                        2.0 ** -14, 2.0 ** -24, 0.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, np.inf], dtype=np.float32)
    vals.append(special)
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def test_f32_to_f16_matches_numpy_rne(orc):
    x = _f32_probe_values()
    got = orc.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_bf16_matches_torch_rne(orc):
    x = _f32_probe_values()
    got = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    back = orc.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128])
def test_fwht_matches_sylvester_matrix(orc, n):
    rng = np.random.default_rng(n)
    H = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    for _ in range(20):
        x = (rng.standard_normal(n) * np.exp(rng.standard_normal(n))).astype(np.float32)
        y = orc.fwht_f32(x).astype(np.float64)
        ref = H @ x.astype(np.float64)
        assert np.max(np.abs(y - ref)) <= 1e-6 * np.linalg.norm(x.astype(np.float64))
        assert np.allclose(orc.rotate_f64(x.astype(np.float64)), ref, rtol=0, atol=1e-12 * np.linalg.norm(x))


def test_fwht_basis_vector_and_constant(orc):
    # H e0 = (1/sqrt(128)) * ones, with the binary32 constant nearest 1/sqrt(128)
    e0 = np.zeros(128, np.float32)
    e0[0] = 1.0
    y = orc.fwht_f32(e0)
    assert set(y.view(np.uint32).tolist()) == {0x3DB504F3}
    # the row pattern of H e_i is the Sylvester sign pattern
    H = scipy.linalg.hadamard(128)
    for i in (1, 5, 77, 127):
        e = np.zeros(128, np.float32)
        e[i] = 1.0
        y = orc.fwht_f32(e)
        assert np.array_equal(np.sign(y), H[:, i].astype(np.float32))


def test_fwht_is_involution_and_preserves_dot(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128).astype(np.float32)
    z = rng.standard_normal(128).astype(np.float32)
    xx = orc.fwht_f32(orc.fwht_f32(x))
    assert np.max(np.abs(xx - x)) < 1e-5
    qx, qz = orc.rotate_f64(x.astype(np.float64)), orc.rotate_f64(z.astype(np.float64))
    assert abs(qx @ qz - x.astype(np.float64) @ z.astype(np.float64)) < 1e-12 * np.linalg.norm(x) * np.linalg.norm(z)


# ----------------------------------------------------------------- quantizer
def _fp16_values(rng, n, scale=1.0):
    return (rng.standard_normal(n) * scale).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("bits", list(range(1, 17)))
def test_quantizer_range_and_error_bound(orc, bits):
    rng = np.random.default_rng(100 + bits)
    L = 2 ** bits - 1
    for trial in range(300):
        scale = float(np.exp(rng.uniform(-6, 6)))
        x = _fp16_values(rng, int(rng.integers(2, 129)), scale)
        if trial % 7 == 0:
            x[int(rng.integers(0, x.size))] *= 50  # an outlier
            x = x.astype(np.float16).astype(np.float32)
        codes, s, mn, sc16, zr16 = orc.quantize_group(x, bits)
        assert codes.max() <= L
        xs = x.astype(np.float64)
        assert float(mn) == xs.min()
        s64 = float(s)
        err = np.abs(xs - (float(mn) + codes.astype(np.float64) * s64))
        assert err.max() <= s64 * (0.5 + 2.0 ** (bits - 23)) + 1e-300
        # fp16 storage: zero16 is exact, scale16 within half an fp16 ulp
        assert orc.f16_bits_to_f32(np.array([zr16], np.uint16))[0] == mn
        s16 = float(orc.f16_bits_to_f32(np.array([sc16], np.uint16))[0])
        if s64 >= 2.0 ** -14 and bits <= 8:
            err16 = np.abs(xs - (float(mn) + codes.astype(np.float64) * s16))
            assert err16.max() <= s64 * (0.5 + 2.0 ** (bits - 23) + L * 2.0 ** -11)


def _brute_codes(x, mn, s, bits):
    """Nearest level mn + c*s by exact rational search, ties to even c.
    Returns per element the set of acceptable codes: one code unless the
    exact quotient is within 2^-20 of a half-integer without being one."""
    out = []
    mnf, sf = Fraction(float(mn)), Fraction(float(s))
    for xi in x:
        xf = Fraction(float(xi))
        d = [abs(xf - mnf - c * sf) for c in range(2 ** bits)]
        best = min(d)
        cands = [c for c in range(2 ** bits) if d[c] == best]
        exact = [c for c in cands if c % 2 == 0] if len(cands) > 1 else cands
        q = (xf - mnf) / sf
        frac = q - math.floor(q)
        if frac != Fraction(1, 2) and abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20):
            out.append({math.floor(q), math.floor(q) + 1})
        else:
            out.append(set(exact))
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantizer_brute_force_small(orc, bits):
    rng = np.random.default_rng(bits)
    for _ in range(400):
        g = int(rng.integers(2, 9))
        x = _fp16_values(rng, g, float(np.exp(rng.uniform(-3, 3))))
        codes, s, mn, _, _ = orc.quantize_group(x, bits)
        if s == 0:
            assert not codes.any()
            continue
        ok = _brute_codes(x, mn, s, bits)
        assert all(int(c) in o for c, o in zip(codes, ok)), (x, codes, ok)


def test_quantizer_ties_go_to_even(orc):
    x = np.array([0.0, 3.0, 0.5, 1.5, 2.5], np.float32)  # b=2: s = 1 exactly
    codes, s, mn, _, _ = orc.quantize_group(x, 2)
    assert s == 1.0 and mn == 0.0
    assert codes.tolist() == [0, 3, 0, 2, 2]


def test_quantizer_one_bit_limit(orc):
    codes, s, mn, _, _ = orc.quantize_group(np.array([0, 1, 0.5, 0.5], np.float32), 1)
    assert codes.tolist() == [0, 1, 0, 0]  # midpoint to the even code
    a, b = -1.5, 2.25
    x = np.array([a, b, a, b, b], np.float32)
    codes, s, mn, sc16, zr16 = orc.quantize_group(x, 1)
    rec = orc.f16_bits_to_f32(np.array([zr16], np.uint16))[0] + codes * orc.f16_bits_to_f32(np.array([sc16], np.uint16))[0]
    assert np.array_equal(rec, x)  # a two-valued group reconstructs exactly


def test_quantizer_sixteen_bit_limit(orc):
    rng = np.random.default_rng(16)
    for _ in range(50):
        x = _fp16_values(rng, 64, 3.0)
        codes, s, mn, _, _ = orc.quantize_group(x, 16)
        err = np.abs(x.astype(np.float64) - (float(mn) + codes * float(s)))
        assert err.max() <= float(s) * (0.5 + 2.0 ** -7)


def test_quantizer_constant_group_and_signed_zero(orc):
    for val in (0.0, -0.0, 1.25, -7.5):
        codes, s, mn, sc16, zr16 = orc.quantize_group(np.full(32, val, np.float32), 2)
        assert not codes.any() and s == 0 and sc16 == 0
        assert zr16 == (0 if val == 0 else int(np.float16(val).view(np.uint16)))
    codes, s, mn, sc16, zr16 = orc.quantize_group(np.array([-0.0, 0.0, -0.0], np.float32), 4)
    assert (sc16, zr16) == (0, 0)


# ----------------------------------------------------------------- window bookkeeping
@pytest.mark.parametrize("G,R", [(32, 32), (64, 128), (32, 128), (32, 0), (64, 64)])
def test_window_bookkeeping(orc, G, R):
    prev = 0
    flushes = 0
    for n in range(0, 700):
        nq = orc.num_quantized(n, G, R)
        assert nq % G == 0 and 0 <= nq <= n
        nr = n - nq
        assert min(n, R) <= nr <= R + G - 1
        if nq != prev:
            assert nq - prev == G and nr == R  # a flush leaves exactly R recent tokens
            flushes += 1
        prev = nq
    assert flushes == max(0, (699 - R) // G)


# ----------------------------------------------------------------- slice encoding
def test_encode_axes_and_window(orc):
    D, G, R, n = 64, 32, 32, 100
    alpha = np.linspace(-3, 3, D).astype(np.float16).astype(np.float32)
    beta = np.linspace(-2, 5, n).astype(np.float16).astype(np.float32)
    k = np.tile(alpha, (n, 1))           # constant along tokens in each channel
    v = np.tile(beta[:, None], (1, D))   # constant along channels in each token
    enc = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False)
    nq = enc["nq"]
    assert nq == 64 and enc["k_resid"].shape == (36, D)
    assert not enc["k_codes"].any() and not enc["k_scale"].any()
    assert np.array_equal(enc["k_zero"], np.tile(alpha.astype(np.float16).view(np.uint16), (nq // G, 1)))
    assert not enc["v_codes"].any() and not enc["v_scale"].any()
    assert np.array_equal(enc["v_zero"], np.tile(beta[:nq, None].astype(np.float16).view(np.uint16), (1, D // G)))
    assert np.array_equal(enc["v_resid"], v[nq:].astype(np.float16).view(np.uint16))


def test_encode_prefix_consistency(orc):
    rng = np.random.default_rng(11)
    D, G, R = 64, 32, 32
    k = rng.standard_normal((300, D)).astype(np.float32)
    v = rng.standard_normal((300, D)).astype(np.float32)
    full = orc.encode_slice(k, v, "f32", D, 2, 4, G, R, False)
    for n in (1, 31, 32, 63, 64, 65, 95, 96, 97, 200, 299):
        part = orc.encode_slice(k[:n], v[:n], "f32", D, 2, 4, G, R, False)
        nq = part["nq"]
        for key in ("k_codes", "v_codes", "v_scale", "v_zero"):
            assert np.array_equal(part[key], full[key][:nq])
        for key in ("k_scale", "k_zero"):
            assert np.array_equal(part[key], full[key][: nq // G])
        assert np.array_equal(part["k_resid"], k[nq:n].astype(np.float16).view(np.uint16))


def test_encode_entry_rounding_bf16(orc):
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((40, 64)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    enc = orc.encode_slice(bits, bits, "bf16", 64, 2, 2, 32, 32, False)
    assert enc["nq"] == 0
    assert np.array_equal(enc["k_resid"], x.float().numpy().astype(np.float16).view(np.uint16))


def test_encode_rotation_sign_pattern(orc):
    D = 128
    H = scipy.linalg.hadamard(D)
    k = np.zeros((3, D), np.float32)
    for t, i in enumerate((0, 9, 100)):
        k[t, i] = 2.0
    enc = orc.encode_slice(k, k, "f32", D, 2, 2, 32, 32, True)
    c16 = np.float16(2.0 * np.float32(1 / math.sqrt(128)))
    for t, i in enumerate((0, 9, 100)):
        ref = (H[:, i] * c16).astype(np.float16).view(np.uint16)
        assert np.array_equal(enc["k_resid"][t], ref)
    assert np.array_equal(enc["v_resid"], k.astype(np.float16).view(np.uint16))  # values are not rotated


# ----------------------------------------------------------------- packing
def test_pack_worked_examples(orc):
    assert orc.pack_codes(np.array([[1, 2, 3, 0]]), 2).tolist() == [[0x39]]
    assert orc.pack_codes(np.array([[0xA, 0x5]]), 4).tolist() == [[0x5A]]
    assert orc.pack_codes(np.array([[1, 0, 1, 1, 0, 0, 0, 1]]), 1).tolist() == [[0x8D]]
    assert orc.pack_codes(np.array([[0x1234, 0xBEEF]]), 16).tolist() == [[0x34, 0x12, 0xEF, 0xBE]]
    assert orc.pack_codes(np.array([[7, 1, 6]]), 3).tolist() == [[0x8F, 0x01]]  # 111 | 001<<3 | 110<<6


@pytest.mark.parametrize("bits", list(range(1, 17)))
def test_pack_unpack_roundtrip(orc, bits):
    rng = np.random.default_rng(bits)
    D = 64
    codes = rng.integers(0, 2 ** bits, size=(37, D)).astype(np.uint16)
    packed = orc.pack_codes(codes, bits)
    assert packed.shape == (37, (D * bits + 7) // 8)
    assert np.array_equal(orc.unpack_codes(packed, D, bits), codes)


# ----------------------------------------------------------------- attention
def _decode(cache, D, G):
    """Dequantized keys/values (fp64) of a canonical slice, for closed-form checks."""
    f = lambda a: np.asarray(a, np.uint16).view(np.float16).astype(np.float64)
    nq = cache["nq"]
    kq = f(cache["k_zero"]).repeat(G, 0)[:nq] + cache["k_codes"] * f(cache["k_scale"]).repeat(G, 0)[:nq]
    vq = f(cache["v_zero"]).repeat(G, 1) + cache["v_codes"] * f(cache["v_scale"]).repeat(G, 1)
    return np.concatenate([kq, f(cache["k_resid"])]), np.concatenate([vq, f(cache["v_resid"])])


def _decimal_attention(q, K, V):
    getcontext().prec = 50
    D = q.shape[1]
    out = []
    for qh in q:
        sig = [sum(Decimal(float(qh[c])) * Decimal(float(K[t, c])) for c in range(D)) / Decimal(D).sqrt()
               for t in range(len(K))]
        m = max(sig)
        w = [(s - m).exp() for s in sig]
        L = sum(w)
        out.append([float(sum(w[t] * Decimal(float(V[t, c])) for t in range(len(K))) / L) for c in range(D)])
    return np.array(out)


@pytest.mark.parametrize("n,G,R", [(8, 2, 2), (7, 2, 0), (5, 4, 8), (8, 4, 0)])
def test_attention_brute_force_decimal(orc, n, G, R):
    rng = np.random.default_rng(n * 10 + G)
    D = 4
    k = rng.standard_normal((n, D)).astype(np.float32) * 2
    v = rng.standard_normal((n, D)).astype(np.float32)
    cache = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False)
    q = rng.standard_normal((3, D))
    got = orc.attend_slice(q, cache, D, G, R)
    K, V = _decode(cache, D, G)
    ref = _decimal_attention(q, K, V)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(21)
    D, G, R, n = 64, 32, 32, 200
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    cache = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False)
    K, V = _decode(cache, D, G)
    # q = 0: uniform weights, the mean of the decoded values
    out = orc.attend_slice(np.zeros((1, D)), cache, D, G, R)
    assert np.max(np.abs(out[0] - V.mean(0))) < 1e-12
    # constant values: weights sum to one
    ones = orc.encode_slice(k, np.ones((n, D), np.float32), "f32", D, 2, 2, G, R, False)
    out = orc.attend_slice(rng.standard_normal((4, D)) * 3, ones, D, G, R)
    assert np.max(np.abs(out - 1.0)) < 1e-14
    # one dominant key: output is that token's decoded value
    t_star = 17
    qq = K[t_star][None, :] * 1e4 / np.linalg.norm(K[t_star]) ** 2 * math.sqrt(D)
    out = orc.attend_slice(qq, cache, D, G, R)
    assert np.max(np.abs(out[0] - V[t_star])) < 1e-9


def test_attention_identical_keys_give_mean(orc):
    rng = np.random.default_rng(22)
    D, G, R, n = 64, 32, 32, 160
    krow = rng.standard_normal(D).astype(np.float32)
    k = np.tile(krow, (n, 1))
    v = rng.standard_normal((n, D)).astype(np.float32)
    cache = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False)
    _, V = _decode(cache, D, G)
    out = orc.attend_slice(rng.standard_normal((2, D)) * 5, cache, D, G, R)
    assert np.max(np.abs(out - V.mean(0)[None])) < 1e-12


def test_attention_permutation_invariance(orc):
    rng = np.random.default_rng(23)
    D, n = 64, 40
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    perm = rng.permutation(n)
    a = orc.encode_slice(k, v, "f32", D, 2, 2, 32, 64, False)  # all tokens in the window
    b = orc.encode_slice(k[perm], v[perm], "f32", D, 2, 2, 32, 64, False)
    q = rng.standard_normal((3, D))
    assert np.max(np.abs(orc.attend_slice(q, a, D, 32, 64) - orc.attend_slice(q, b, D, 32, 64))) < 1e-12


@pytest.mark.parametrize("S", [1, 2, 3, 7, 0])
def test_split_merge_matches_full(orc, S):
    rng = np.random.default_rng(24)
    D, G, R, n = 64, 32, 32, 237
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    cache = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False)
    q = rng.standard_normal((4, D)) * 2
    full = orc.attend_slice(q, cache, D, G, R)
    S = n if S == 0 else S
    cuts = sorted(set([0, n] + rng.choice(np.arange(1, n), size=S - 1, replace=False).tolist())) if S > 1 else [0, n]
    parts = [orc.attend_partial(q, cache, D, G, R, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    # an empty split contributes nothing
    parts.append(orc.attend_partial(q, cache, D, G, R, 5, 5))
    m = np.stack([p[0] for p in parts])
    l = np.stack([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])
    assert np.isneginf(m[-1]).all() and not l[-1].any()
    assert np.max(np.abs(orc.merge_partials(m, l, o) - full)) < 1e-12


# ----------------------------------------------------------------- accounting
def test_compression_table_from_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "akvq_compression_table.json")))
    for row in g["rows"]:
        assert round(g["fp16_bits"] / row["avg_bits"], 1) == row["compression"]
        if row["key_bits"] is not None:
            bpe = orc.bits_per_element(4096, row["key_bits"], row["value_bits"], 64, 0, overhead_bits=0.0)
            assert bpe == row["avg_bits"]


def test_memory_numbers_from_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "akvq_memory_7b_262k.json")))
    fp16_printed = g["rows"][0]["gb"]
    for row in g["rows"]:
        gb = orc.kv_cache_bytes(g["layers"], g["hidden"], g["tokens"], row["bits"]) / 1e9
        assert abs(gb - row["gb"]) <= 0.06, (row, gb)
        # the page's quantized rows scale its rounded fp16 figure by bits/16
        assert round(fp16_printed * row["bits"] / 16, 1) == row["gb"]
    assert round(orc.kv_cache_bytes(g["layers"], g["hidden"], g["tokens"], 16) / 1e9, 1) == fp16_printed


@pytest.mark.parametrize("kb,vb,G,R,n", [(2, 2, 32, 128, 8192), (4, 2, 64, 128, 32768 // 8), (2, 2, 32, 32, 1000), (2, 2, 32, 64, 777)])
def test_bits_per_element_counts_encoded_bytes(orc, kb, vb, G, R, n):
    rng = np.random.default_rng(n)
    D = 128
    k = rng.standard_normal((n, D)).astype(np.float32)
    cache = orc.encode_slice(k, k, "f32", D, kb, vb, G, R, False)
    bits = (orc.pack_codes(cache["k_codes"], kb).size + orc.pack_codes(cache["v_codes"], vb).size) * 8
    bits += 16 * sum(cache[x].size for x in ("k_scale", "k_zero", "v_scale", "v_zero", "k_resid", "v_resid"))
    assert bits / (2 * n * D) == pytest.approx(orc.bits_per_element(n, kb, vb, G, R), rel=1e-12)


def test_window_default_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "kivi_window_defaults.json")))
    from synth import WORKLOADS

    assert WORKLOADS[0].R == g["window_tokens"] and WORKLOADS[0].kbits == g["bits"] == WORKLOADS[0].vbits


# ------------------------------------------------- hybrid quantizer, sink window
def _fp16_vals(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _max_err_f64(orc, x, codes, sc, zr):
    s = float(orc.f16_bits_to_f32(np.array([sc], np.uint16))[0])
    z = float(orc.f16_bits_to_f32(np.array([zr], np.uint16))[0])
    return float(np.max(np.abs(np.asarray(x, np.float64) - (z + codes.astype(np.float64) * s))))


@pytest.mark.parametrize("bits", [2, 4])
def test_symmetric_quantizer_reproduces_its_grid(orc, bits):
    """Values on the grid s * k, |k| <= c0 (with 0 and both ends present), come
    back exactly from the symmetric quantizer, codes k + c0; the asymmetric
    quantizer cannot (2^b levels over 2 c0 + 1 grid points), so the hybrid
    keeps the symmetric one."""
    c0 = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(bits)
    ks = np.concatenate([[-c0, 0, c0], rng.integers(-c0, c0 + 1, 29)])
    x = _fp16_vals(0.5 * ks)
    codes, s, sc, zr = orc.quantize_group_sym(x, bits)
    assert s == np.float32(0.5 * c0 / c0)
    assert np.array_equal(codes, (ks + c0).astype(np.uint16))
    assert orc.f16_bits_to_f32(np.array([zr], np.uint16))[0] == np.float32(-0.5 * c0)
    assert orc.group_max_error(x, codes, sc, zr) == 0.0
    ca, _, _, sa, za = orc.quantize_group(x, bits)
    assert orc.group_max_error(x, ca, sa, za) > 0.0
    hc, hs, hz, sym = orc.quantize_group_hybrid(x, bits)
    assert sym and np.array_equal(hc, codes) and (hs, hz) == (sc, zr)


@pytest.mark.parametrize("bits", [2, 4])
def test_hybrid_keeps_asymmetric_for_one_sided_data(orc, bits):
    """Data in [10, 11]: the asymmetric error is at most half a step of 1/(2^b-1)
    (plus fp16 rounding of the scale), the symmetric one about 10 / c0 or more."""
    rng = np.random.default_rng(7 + bits)
    x = _fp16_vals(10.0 + rng.random(64))
    ca, _, _, sa, za = orc.quantize_group(x, bits)
    hc, hs, hz, sym = orc.quantize_group_hybrid(x, bits)
    assert not sym
    assert np.array_equal(hc, ca) and (hs, hz) == (sa, za)
    assert _max_err_f64(orc, x, hc, hs, hz) <= 0.5 / (2 ** bits - 1) + 0.01


@pytest.mark.parametrize("bits", [2, 4])
def test_hybrid_never_worse_and_well_formed(orc, bits):
    """On groups drawn from several shapes (centred, skewed, sparse, constant,
    with signed zeros) the kept quantizer's largest error, evaluated
    independently in fp64 from the stored fp16 parameters, is never above the
    asymmetric one's (up to fp32 rounding of the error itself), and a kept
    symmetric group has zero = fp16(-c0 * scale) and codes in [0, 2 c0]."""
    c0 = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(100 + bits)
    shapes = [
        lambda: rng.standard_normal(32),
        lambda: rng.standard_normal(32) + 3.0,
        lambda: np.where(rng.random(32) < 0.8, 0.0, rng.standard_normal(32) * 5),
        lambda: np.full(32, rng.standard_normal()),
        lambda: np.concatenate([[-0.0, 0.0], rng.laplace(size=30)]),
        lambda: rng.uniform(-1, 1, 32) ** 3,
    ]
    n_sym = 0
    for it in range(600):
        x = _fp16_vals(shapes[it % len(shapes)]())
        ca, _, _, sa, za = orc.quantize_group(x, bits)
        hc, hs, hz, sym = orc.quantize_group_hybrid(x, bits)
        ea = _max_err_f64(orc, x, ca, sa, za)
        eh = _max_err_f64(orc, x, hc, hs, hz)
        assert eh <= ea + 1e-6 * max(1.0, float(np.max(np.abs(x))))
        if sym:
            n_sym += 1
            s = orc.f16_bits_to_f32(np.array([hs], np.uint16))[0]
            assert hz == int(orc.f32_to_f16_bits(np.array([-(s * np.float32(c0))], np.float32))[0])
            assert hc.max() <= 2 * c0
        else:
            assert np.array_equal(hc, ca) and (hs, hz) == (sa, za)
    assert 0 < n_sym < 600  # both quantizers occur


def test_hybrid_constant_and_zero_groups_stay_asymmetric(orc):
    for x in (np.zeros(32, np.float32), np.full(32, 1.5, np.float32), np.full(32, -3.25, np.float32)):
        ca, s, mn, sa, za = orc.quantize_group(x, 2)
        assert s == 0.0 and not ca.any()
        hc, hs, hz, sym = orc.quantize_group_hybrid(x, 2)
        assert not sym and (hs, hz) == (sa, za) and not hc.any()


@pytest.mark.parametrize("G,R,S0", [(32, 64, 64), (64, 128, 64), (32, 0, 32), (32, 32, 128)])
def test_sink_window_bookkeeping(orc, G, R, S0):
    """Tokens [0, min(n, S0)) stay fp16, then whole groups aligned to S0 with
    at least R recent tokens left in fp16."""
    for n in range(0, S0 + R + 3 * G + 5):
        expect = 0 if n <= S0 else max(0, (n - S0 - R) // G) * G
        assert orc.num_quantized(n, G, R, S0) == expect


def test_sink_encoding_is_the_tail_encoding_plus_fp16_prefix(orc):
    """With a sink of S0 tokens the quantized groups are exactly those of the
    sequence without its first S0 tokens, and the fp16 tokens are the first
    S0 tokens (fp16 of the input) followed by that sequence's window."""
    rng = np.random.default_rng(31)
    D, G, R, S0, n = 64, 32, 32, 64, 64 + 5 * 32 + 17
    k = rng.standard_normal((n, D)).astype(np.float32) * 3
    v = rng.standard_normal((n, D)).astype(np.float32)
    for hybrid in (False, True):
        a = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False, sink=S0, hybrid=hybrid)
        b = orc.encode_slice(k[S0:], v[S0:], "f32", D, 4, 2, G, R, False, hybrid=hybrid)
        assert a["nq"] == b["nq"] == 4 * 32
        for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_sym", "v_sym"):
            assert np.array_equal(a[key], b[key]), key
        assert np.array_equal(a["k_resid"][:S0], orc.f32_to_f16_bits(k[:S0]))
        assert np.array_equal(a["v_resid"][:S0], orc.f32_to_f16_bits(v[:S0]))
        assert np.array_equal(a["k_resid"][S0:], b["k_resid"]) and np.array_equal(a["v_resid"][S0:], b["v_resid"])


def test_sink_attention_without_quantized_tokens_is_exact_softmax(orc):
    """n <= S0 + R + G - 1: nothing is quantized, so attention is exact softmax
    attention over the fp16-rounded inputs (computed here with numpy)."""
    rng = np.random.default_rng(5)
    D, G, R, S0, n = 64, 32, 32, 64, 64 + 32 + 31
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    c = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False, sink=S0)
    assert c["nq"] == 0
    q = rng.standard_normal((2, D))
    kh = k.astype(np.float16).astype(np.float64)
    vh = v.astype(np.float16).astype(np.float64)
    sc = q @ kh.T / np.sqrt(D)
    w = np.exp(sc - sc.max(1, keepdims=True))
    ref = w @ vh / w.sum(1, keepdims=True)
    assert np.max(np.abs(orc.attend_slice(q, c, D, G, R) - ref)) < 1e-12


def test_bits_per_element_with_sink_closed_form(orc):
    # n = 8192, G = 32, R = 128, S0 = 64, K2/V2: nq = 32 * floor(8000 / 32) = 8000
    # fp16 tokens 192; bpe = (8000 * (2 + 1) * 2 + 32 * 192) / (2 * 8192)
    assert orc.num_quantized(8192, 32, 128, 64) == 8000
    assert orc.bits_per_element(8192, 2, 2, 32, 128, sink=64) == pytest.approx((48000 + 6144) / 16384, abs=1e-12)


# --------------------------------------------------------- token-norm scaling
def test_row_norm_closed_forms_and_summation_tree(orc):
    x = np.zeros(128, np.float32)
    x[0], x[1] = 3.0, 4.0
    assert orc.row_norm_f32(x) == 5.0
    assert orc.row_norm_f32(np.ones(128, np.float32)) == np.float32(np.sqrt(128.0))
    assert orc.row_norm_f32(np.zeros(64, np.float32)) == 0.0
    # squares [2^24, 1, 1, 1]: the pairwise tree gives (2^24 + 1) + (1 + 1) =
    # 2^24 + 2 (the first sum rounds to 2^24), a left-to-right sum 2^24
    assert orc.row_norm_f32(np.array([4096.0, 1.0, 1.0, 1.0], np.float32)) == np.float32(np.sqrt(2.0 ** 24 + 2))


def test_token_norm_power_of_two_scaling(orc):
    """Scaling a key token by 2^k (exact in fp16) leaves every code, scale and
    zero unchanged and multiplies that token's stored norm by 2^k."""
    rng = np.random.default_rng(11)
    D, G, R, n = 64, 32, 32, 32 * 4 + 40
    k = orc.f16_bits_to_f32(orc.f32_to_f16_bits(rng.standard_normal((n, D)).astype(np.float32)))
    v = rng.standard_normal((n, D)).astype(np.float32)
    a = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False, token_norm=True)
    k2 = k.copy()
    scale = np.ones(n, np.float32)
    scale[[3, 40, 77, 100]] = [4.0, 0.5, 2.0, 0.25]
    k2 *= scale[:, None]
    b = orc.encode_slice(k2, v, "f32", D, 4, 2, G, R, False, token_norm=True)
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(a[key], b[key]), key
    na = orc.f16_bits_to_f32(a["k_norm"])
    nb = orc.f16_bits_to_f32(b["k_norm"])
    assert np.array_equal(nb, na * scale[:a["nq"]])


def test_token_norm_attention_on_one_direction(orc):
    """Keys 2^e_t * u along one direction u: every normalized row is the same,
    so each channel group is constant (codes 0, zero = the normalized value)
    and the decoded key is the stored norm times it; attention then equals
    softmax over sigma_t = |2^e_t u|_norm * (q . u_hat) / sqrt(D) (numpy)."""
    rng = np.random.default_rng(12)
    D, G, R, n = 64, 32, 32, 32 * 3 + 32
    u = orc.f16_bits_to_f32(orc.f32_to_f16_bits(rng.standard_normal(D).astype(np.float32)))
    e = rng.integers(-3, 4, n)
    k = (u[None, :] * (2.0 ** e)[:, None]).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    c = orc.encode_slice(k, v, "f32", D, 2, 2, G, R, False, token_norm=True)
    nq = c["nq"]
    assert nq == 96 and not c["k_codes"].any()
    nrm = orc.row_norm_f32(u)
    uh = orc.f16_bits_to_f32(orc.f32_to_f16_bits(u / np.float32(nrm))).astype(np.float64)
    assert np.array_equal(orc.f16_bits_to_f32(c["k_zero"][0]).astype(np.float64), uh)
    norms = orc.f16_bits_to_f32(c["k_norm"]).astype(np.float64)
    kd = np.concatenate([norms[:, None] * uh[None, :], k[nq:].astype(np.float16).astype(np.float64)])
    vd = np.concatenate([orc.f16_bits_to_f32(c["v_zero"]).repeat(G, 1) + c["v_codes"] *
                         orc.f16_bits_to_f32(c["v_scale"]).repeat(G, 1), v[nq:].astype(np.float16)]).astype(np.float64)
    q = rng.standard_normal((3, D))
    sc = q @ kd.T / np.sqrt(D)
    w = np.exp(sc - sc.max(1, keepdims=True))
    ref = w @ vd / w.sum(1, keepdims=True)
    assert np.max(np.abs(orc.attend_slice(q, c, D, G) - ref)) < 1e-12


def test_token_norm_zero_rows_and_reconstruction(orc):
    rng = np.random.default_rng(13)
    D, G, R, n = 64, 32, 0, 64
    k = rng.standard_normal((n, D)).astype(np.float32) * rng.uniform(0.1, 10, (n, 1)).astype(np.float32)
    k[5] = 0.0
    v = rng.standard_normal((n, D)).astype(np.float32)
    c = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False, token_norm=True)
    nrm = orc.f16_bits_to_f32(c["k_norm"]).astype(np.float64)
    assert nrm[5] == 0.0
    s = orc.f16_bits_to_f32(c["k_scale"]).astype(np.float64).repeat(G, 0)
    z = orc.f16_bits_to_f32(c["k_zero"]).astype(np.float64).repeat(G, 0)
    kd = nrm[:, None] * (z + c["k_codes"] * s)
    assert not kd[5].any()
    # per element: |k - khat| <= norm * (s / 2 + fp16 rounding of the normalized value) + fp16 rounding of the norm
    kh = k.astype(np.float16).astype(np.float64)
    bound = nrm[:, None] * (s / 2 + 2.0 ** -11) + np.abs(kh) * 2.0 ** -10 + 1e-6
    assert np.all(np.abs(kd - kh) <= bound)


# ------------------------------------------------- position-adaptive bit widths
LOW, MID, HIGH = (2, 2), (4, 2), (4, 4)


def test_adaptive_regions_of_a_prefill_closed_form(orc):
    """Prefill of 8192 tokens, delta 1024, G 64, R 128: 126 groups; group g ends
    at 1-based position 64 g + 64.  Early (<= 1024): g < 16; recent (> 8192 -
    1024 = 7168): g >= 112; middle in between."""
    kb, vb = orc.adaptive_group_bits(64, 128, 0, 1024, [8192], LOW, MID, HIGH)
    assert kb.size == 126
    g = np.arange(126)
    expect = np.where(g >= 112, 2, np.where(g < 16, 0, 1))
    bits = np.array([LOW, MID, HIGH])
    assert np.array_equal(kb, bits[expect, 0]) and np.array_equal(vb, bits[expect, 1])


def test_adaptive_regions_short_prefill_and_sink(orc):
    # n = 1500 < 2 delta: a group both early and recent is recent (printed order);
    # 21 groups, recent when 64 g + 64 > 476, i.e. g >= 7
    kb, vb = orc.adaptive_group_bits(64, 128, 0, 1024, [1500], LOW, MID, HIGH)
    assert kb.size == 21
    assert np.array_equal(kb, np.where(np.arange(21) >= 7, 4, 2)) and np.array_equal(vb, kb)
    # with a 64-token sink the groups shift by 64 positions: group g ends at 64 g + 128
    kb, vb = orc.adaptive_group_bits(64, 128, 64, 1024, [8192], LOW, MID, HIGH)
    g = np.arange(kb.size)
    assert kb.size == 125
    assert np.array_equal(kb, np.where(64 * g + 128 > 7168, 4, np.where(64 * g + 128 <= 1024, 2, 4)))
    assert np.array_equal(vb, np.where(64 * g + 128 > 7168, 4, 2))


def test_adaptive_groups_quantized_while_decoding_are_recent(orc):
    """One token per append: each group is quantized when n = S0 + gG + G + R,
    its last token is at n - R > n - delta, so every group is recent."""
    kb, vb = orc.adaptive_group_bits(32, 64, 0, 1024, [1] * 3000, LOW, MID, HIGH)
    assert kb.size == (3000 - 64) // 32 and (kb == 4).all() and (vb == 4).all()
    # a prefill, then steps: the prefill's regions stay, later groups are recent
    kb2, _ = orc.adaptive_group_bits(32, 64, 0, 1024, [5000] + [1] * 500, LOW, MID, HIGH)
    kb1, _ = orc.adaptive_group_bits(32, 64, 0, 1024, [5000], LOW, MID, HIGH)
    assert np.array_equal(kb2[:kb1.size], kb1) and (kb2[kb1.size:] == 4).all()
    assert (kb1 == 2).any() and (kb1 == 4).any()


def test_adaptive_encoding_is_per_group_fixed_bit_encoding(orc):
    """Each group's codes and parameters are those of the fixed-width encoder
    at that group's bits; equal bits everywhere is the plain encoder."""
    rng = np.random.default_rng(21)
    D, G, R, n = 64, 32, 32, 32 * 12 + 40
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    gk = np.array([2, 4, 4, 2, 2, 4, 2, 4, 4, 4, 2, 2], np.uint8)
    gv = np.array([2, 2, 4, 4, 2, 4, 2, 2, 4, 4, 4, 2], np.uint8)
    a = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False, group_bits=(gk, gv))
    ref = {(kb, vb): orc.encode_slice(k, v, "f32", D, kb, vb, G, R, False) for kb in (2, 4) for vb in (2, 4)}
    for g in range(12):
        r = ref[(int(gk[g]), int(gv[g]))]
        sl = slice(g * G, g * G + G)
        assert np.array_equal(a["k_codes"][sl], r["k_codes"][sl])
        assert np.array_equal(a["k_scale"][g], r["k_scale"][g]) and np.array_equal(a["k_zero"][g], r["k_zero"][g])
        assert np.array_equal(a["v_codes"][sl], r["v_codes"][sl]) and np.array_equal(a["v_scale"][sl], r["v_scale"][sl])
    same = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False, group_bits=(np.full(12, 4, np.uint8), np.full(12, 2, np.uint8)))
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid"):
        assert np.array_equal(same[key], ref[(4, 2)][key]), key


# ------------------------------------------------- drift detection (KL of code histograms)
def test_kl_closed_forms(orc):
    ln = np.log
    assert orc.kl_divergence([0.25, 0.25, 0.5], [0.25, 0.25, 0.5]) == 0.0
    # one-hot p: D_KL = -ln q_i
    assert orc.kl_divergence([0, 0, 1], [0.25, 0.25, 0.5]) == pytest.approx(ln(2), rel=1e-15)
    assert orc.kl_divergence([1, 0, 0], [0.25, 0.25, 0.5]) == pytest.approx(ln(4), rel=1e-15)
    assert orc.kl_divergence([1, 0], [0.5, 0.5]) == pytest.approx(ln(2), rel=1e-15)
    # mass where the calibration has none: infinite; no mass where it has none: ignored
    assert orc.kl_divergence([0.5, 0.5], [1.0, 0.0]) == float("inf")
    assert orc.kl_divergence([1.0, 0.0], [1.0, 0.0]) == 0.0
    # two bins, p = (1/4, 3/4), q = (1/2, 1/2): (1/4) ln(1/2) + (3/4) ln(3/2) = (3/4) ln 3 - ln 2
    assert orc.kl_divergence([0.25, 0.75], [0.5, 0.5]) == pytest.approx(0.75 * ln(3) - ln(2), rel=1e-14)


def test_kl_matches_library_relative_entropy(orc):
    from scipy.stats import entropy

    rng = np.random.default_rng(5)
    for nb in (4, 16):
        for _ in range(50):
            p = rng.dirichlet(np.ones(nb) * 0.7)
            q = rng.dirichlet(np.ones(nb) * 2.0)
            got = orc.kl_divergence(p, q)
            assert got == pytest.approx(entropy(p, q), rel=1e-12, abs=1e-15)
            assert got > 0.0  # Gibbs: zero only at p = q


def test_code_histogram_counts(orc):
    ramp = np.arange(16 * 37) % 16
    h = orc.code_histogram(ramp, 4)
    assert np.array_equal(h, np.full(16, 37))
    rng = np.random.default_rng(9)
    c = rng.integers(0, 4, 5000)
    h = orc.code_histogram(c, 2)
    assert h.sum() == 5000 and np.array_equal(h, np.bincount(c, minlength=4))
    assert np.array_equal(orc.code_histogram(rng.permutation(c), 2), h)
    with pytest.raises(ValueError):
        orc.code_histogram(np.array([4]), 2)


def test_drift_check_flags_closed_forms(orc):
    G, D = 32, 64
    per = G * D
    # calibration: key codes uniform over 16 values, value codes (1, 1, 1, 5) / 8
    cal_k = np.full(16, 1000, np.int64)
    cal_v = np.array([1, 1, 1, 5], np.int64) * 100
    kc = np.zeros((3, per), np.uint16)
    vc = np.zeros((3, per), np.uint16)
    kc[0] = np.arange(per) % 16                       # matches the calibration exactly
    vc[0] = np.repeat([0, 1, 2, 3, 3, 3, 3, 3], per // 8)
    kc[1] = 7                                         # one value: KL = ln 16
    vc[1] = 3                                         # one value: KL = ln (8 / 5)
    kc[2] = np.arange(per) % 8                        # half the values, evenly: KL = ln 2
    vc[2] = np.arange(per) % 4                        # uniform vs (1,1,1,5)/8: sum 1/4 ln(2) * 3 + 1/4 ln(2/5)
    kl_k, kl_v, flags = orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, cal_k, cal_v, 0.1)
    ln = np.log
    assert kl_k[0] == 0.0 and kl_v[0] == 0.0 and flags[0] == 0
    assert kl_k[1] == pytest.approx(ln(16), rel=1e-14) and kl_v[1] == pytest.approx(ln(8 / 5), rel=1e-14)
    assert flags[1] == 3
    assert kl_k[2] == pytest.approx(ln(2), rel=1e-14)
    assert kl_v[2] == pytest.approx(0.75 * ln(2) + 0.25 * ln(2 / 5), rel=1e-13)
    assert flags[2] == (1 | (2 if kl_v[2] > 0.1 else 0))
    # the threshold is strict
    _, _, f = orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, cal_k, cal_v, float(kl_k[2]))
    assert (f[2] & 1) == 0


def test_drift_check_empty_calibration_closed_form(orc):
    """A calibration without counts has no mass in any bin, so every group
    (which always has G * D codes) has KL = +inf against it and its flag set;
    an empty key calibration leaves the value side as it is, and the reverse.
    A negative count is rejected."""
    G, D = 32, 64
    per = G * D
    kc = np.zeros((2, per), np.uint16)
    vc = np.zeros((2, per), np.uint16)
    kc[0] = np.arange(per) % 16
    vc[0] = np.arange(per) % 4
    kc[1] = 5
    vc[1] = 2
    zk, zv = np.zeros(16, np.int64), np.zeros(4, np.int64)
    uk, uv = np.full(16, 10, np.int64), np.full(4, 10, np.int64)
    kl_k, kl_v, flags = orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, zk, zv, 0.1)
    assert np.isposinf(kl_k).all() and np.isposinf(kl_v).all()
    assert (flags == 3).all()
    # empty keys only: key KL +inf, value KL = closed form against the uniform value calibration
    kl_k, kl_v, flags = orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, zk, uv, 0.1)
    assert np.isposinf(kl_k).all()
    assert kl_v[0] == 0.0 and kl_v[1] == pytest.approx(np.log(4), rel=1e-14)
    assert list(flags) == [1, 3]
    # empty values only
    kl_k, kl_v, flags = orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, uk, zv, 0.1)
    assert np.isposinf(kl_v).all()
    assert kl_k[0] == 0.0 and kl_k[1] == pytest.approx(np.log(16), rel=1e-14)
    assert list(flags) == [2, 3]
    with pytest.raises(ValueError):
        orc.drift_check(kc.reshape(-1, D), vc.reshape(-1, D), G, D, 4, 2, np.array([-1] + [1] * 15), uv, 0.1)


def test_drift_check_on_encoded_caches(orc):
    """Stationary Gaussian tokens stay far below the 0.1 threshold against a
    calibration taken from the first groups; tokens whose values turn heavy
    tailed (most near zero, a few large) concentrate their codes and cross it."""
    rng = np.random.default_rng(13)
    D, G, R, n = 64, 32, 32, 32 * 40 + 32
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    # groups 30..39: heavy tails (a scale of 0.05 with 5% of entries times 40)
    sl = slice(30 * G, 40 * G)
    for x in (k, v):
        x[sl] *= 0.05
        mask = rng.random(x[sl].shape) < 0.05
        x[sl][mask] *= 40
    enc = orc.encode_slice(k, v, "f32", D, 4, 2, G, R, False)
    ng = enc["nq"] // G
    assert ng == 40
    cal_k = orc.code_histogram(enc["k_codes"][:10 * G], 4)
    cal_v = orc.code_histogram(enc["v_codes"][:10 * G], 2)
    kl_k, kl_v, flags = orc.drift_check(enc["k_codes"], enc["v_codes"], G, D, 4, 2, cal_k, cal_v, 0.1)
    assert (kl_k[:30] < 0.05).all() and (kl_v[:30] < 0.05).all() and (flags[:30] == 0).all()
    assert (kl_k[30:] > 0.1).all() and (kl_v[30:] > 0.1).all() and (flags[30:] == 3).all()


def test_input_widening_matches_torch(orc):
    """input_to_f64 widens stored f32 values and f16 / bf16 bit patterns exactly
    (checked against torch's own conversions of the same bits)."""
    import torch

    rng = np.random.default_rng(5)
    x = (rng.standard_normal(4096) * 30).astype(np.float32)
    assert np.array_equal(orc.input_to_f64(x, "f32"), x.astype(np.float64))
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        t = torch.from_numpy(x).to(tdt)
        bits = t.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(orc.input_to_f64(bits, dt), t.to(torch.float64).numpy()), dt
