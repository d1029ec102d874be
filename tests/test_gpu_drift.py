"""GPU parity of drift detection (code histograms, KL per group, flags) and of
requantization, through the C ABI, against the oracle on the same seeded
inputs.  Histograms and requantized codes must match exactly; the KL values
(fp64 on both sides, summed in another order) to 1e-12 relative."""
import numpy as np
import pytest
import torch

from _parity import assert_export_matches, log, oracle_encode_slices
from synth import WORKLOADS, Synth

pytestmark = pytest.mark.gpu

THR = 0.1


def _lib():
    import decode_attention_asym_amd as kvq

    return kvq


def _heavy_tail(X, t0, t1, seed):
    """Tokens [t0, t1) of X scaled by 0.05 with 5% of entries times 40 (a
    drifted, heavy-tailed stretch), in place, seeded."""
    g = torch.Generator(device=X.device)
    g.manual_seed(seed)
    sl = X[:, :, t0:t1].float()
    mask = torch.rand(sl.shape, generator=g, device=X.device) < 0.05
    sl = sl * 0.05 * torch.where(mask, 40.0, 1.0)
    X[:, :, t0:t1] = sl.to(X.dtype)


DRIFT = [
    WORKLOADS[2].replace(name="drift-k4v2-g64", B=2, Hq=8, Hkv=2, N=4096 + 77),
    WORKLOADS[1].replace(name="drift-k2v2-g32-sink-hybrid", B=2, Hq=8, Hkv=2, N=3000 + 5, sink=64, hybrid=True),
    WORKLOADS[0].replace(name="drift-d64-k4v4-rot-tokennorm", B=2, Hq=4, Hkv=2, N=1500 + 3, kbits=4, vbits=4,
                         rotate=True, token_norm=True),
    WORKLOADS[1].replace(name="drift-d64-k2v4-g32", B=3, Hq=6, Hkv=3, D=64, N=1200, kbits=2, vbits=4, G=32, R=32),
]


@pytest.mark.parametrize("w", DRIFT, ids=lambda w: w.name)
def test_drift_check_and_requantize_match_oracle(w):
    kvq = _lib()
    import oracle

    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    n = w.N
    G = w.G
    ng = oracle.num_quantized(n, G, w.R, w.sink) // G
    # the last third of the quantized groups drift
    d0 = w.sink + (2 * ng // 3) * G
    d1 = w.sink + ng * G
    _heavy_tail(K, d0, d1, 11)
    _heavy_tail(V, d0, d1, 12)
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    assert c.num_groups() == ng
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    encs = oracle_encode_slices(w, K, V, pairs)
    ncal = ng // 3
    log(f"[drift] {w.name}: {ng} groups, calibration groups [0, {ncal}), drift from group {(d0 - w.sink) // G}")

    # calibration histograms: exact counts per kv head over every sequence
    kh, vh = c.code_histograms(0, ncal)
    ref_k = np.zeros((w.Hkv, 1 << w.kbits), np.int64)
    ref_v = np.zeros((w.Hkv, 1 << w.vbits), np.int64)
    for (b, h), e in encs.items():
        ref_k[h] += oracle.code_histogram(e["k_codes"][:ncal * G], w.kbits)
        ref_v[h] += oracle.code_histogram(e["v_codes"][:ncal * G], w.vbits)
    assert np.array_equal(kh.cpu().numpy(), ref_k)
    assert np.array_equal(vh.cpu().numpy(), ref_v)

    # per-group KL and flags over all groups
    kl_k, kl_v, flags = c.drift_check(kh, vh, 0, ng, THR)
    torch.cuda.synchronize()
    kl_k, kl_v, flags = kl_k.cpu().numpy(), kl_v.cpu().numpy(), flags.cpu().numpy()
    nflag = 0
    ref_flags = np.zeros_like(flags)
    for (b, h), e in encs.items():
        s = b * w.Hkv + h
        rk, rv, rf = oracle.drift_check(e["k_codes"], e["v_codes"], G, w.D, w.kbits, w.vbits, ref_k[h], ref_v[h], THR)
        for got, ref in ((kl_k[s], rk), (kl_v[s], rv)):
            fin = np.isfinite(ref)
            assert np.array_equal(np.isfinite(got), fin)
            np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-15)
        # flags: identical wherever the KL is not within rounding of the threshold
        clear = (np.abs(rk - THR) > 1e-9) & (np.abs(rv - THR) > 1e-9)
        assert np.array_equal(flags[s][clear], rf[clear])
        ref_flags[s] = rf
        nflag += int((rf != 0).sum())
    log(f"[drift] {w.name}: {nflag} of {len(pairs) * ng} groups flagged; "
        f"key KL median {np.median(kl_k):.4f} max finite {np.max(kl_k[np.isfinite(kl_k)]):.3f}")
    assert nflag > 0

    # requantize the groups the oracle flags from replacement tokens (fresh,
    # stationary): the cache must equal the oracle encoding of the sequence
    # with exactly those groups' tokens replaced
    g0, g1 = 0, ng
    t0, t1 = w.sink + g0 * G, w.sink + g1 * G
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    Kn = (torch.randn((w.B, w.Hkv, t1 - t0, w.D), generator=gen, device="cuda")).to(K.dtype)
    Vn = (torch.randn((w.B, w.Hkv, t1 - t0, w.D), generator=gen, device="cuda")).to(V.dtype)
    flags_dev = torch.from_numpy(ref_flags).cuda()
    c.requantize(Kn, Vn, g0, g1, flags_dev)
    K2, V2 = K.clone(), V.clone()
    for (b, h) in pairs:
        s = b * w.Hkv + h
        for g in np.flatnonzero(ref_flags[s]):
            a0, a1 = t0 + g * G, t0 + g * G + G
            K2[b, h, a0:a1] = Kn[b, h, g * G:g * G + G]
            V2[b, h, a0:a1] = Vn[b, h, g * G:g * G + G]
    exp = c.export()
    assert_export_matches(w, exp, 0, oracle_encode_slices(w, K2, V2, pairs))

    # requantizing every group from its own tokens changes nothing
    c.requantize(K2[:, :, t0:t1].contiguous(), V2[:, :, t0:t1].contiguous(), g0, g1, None)
    exp2 = c.export()
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid"):
        assert np.array_equal(exp[key], exp2[key]), key


def test_requantize_partial_range_and_adaptive_cache():
    """A group range in the middle, on a position-adaptive cache (each group
    keeps its widths): the named groups are re-encoded from the given tokens,
    the others are untouched."""
    kvq = _lib()
    from _parity import oracle_group_bits

    w = WORKLOADS[2].replace(name="requant-adaptive", B=1, Hq=8, Hkv=2, N=3000, adapt_delta=512, bits_low=(2, 2),
                             bits_high=(4, 4))
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    G, ng = w.G, c.num_groups()
    g0, g1 = 3, ng - 4
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    Kn = torch.randn((w.B, w.Hkv, (g1 - g0) * G, w.D), generator=gen, device="cuda").to(K.dtype)
    Vn = torch.randn((w.B, w.Hkv, (g1 - g0) * G, w.D), generator=gen, device="cuda").to(V.dtype)
    c.requantize(Kn, Vn, g0, g1)
    K2, V2 = K.clone(), V.clone()
    K2[:, :, g0 * G:g1 * G] = Kn
    V2[:, :, g0 * G:g1 * G] = Vn
    pairs = [(0, h) for h in range(w.Hkv)]
    assert oracle_group_bits(w, [w.N]) is not None
    assert_export_matches(w, c.export(), 0, oracle_encode_slices(w, K2, V2, pairs, calls=[w.N]))
    # a range past the quantized groups is refused by the library (tensors of
    # the range's size), a tensor not of the range's size by the binding
    Kx = torch.zeros((w.B, w.Hkv, (ng + 1 - g0) * G, w.D), dtype=K.dtype, device="cuda")
    with pytest.raises(kvq.KVQError):
        c.requantize(Kx, Kx, g0, ng + 1)
    with pytest.raises(ValueError):
        c.requantize(Kn, Vn, g0, ng + 1)
    with pytest.raises(kvq.KVQError):
        c.code_histograms(0, 4)  # no drift detection on adaptive caches


@pytest.mark.parametrize("g0,g1", [(5, 6), (3, 10), (7, 20), (1, 40)])
def test_drift_subranges_equal_full_range(g0, g1):
    """Histograms and KL over a middle group range (odd starts and lengths, so
    the kernel's groups per wave and its pairs end mid-way) equal the oracle's
    and the same groups' values from the full-range call."""
    kvq = _lib()
    import oracle

    w = DRIFT[0].replace(name="drift-subrange", B=1, Hq=8, Hkv=2, N=3000)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    _heavy_tail(K, 1500, 2400, 21)
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    ng = c.num_groups()
    assert g1 <= ng
    pairs = [(0, h) for h in range(w.Hkv)]
    encs = oracle_encode_slices(w, K, V, pairs)
    kh, vh = c.code_histograms(g0, g1)
    ref_k = np.zeros((w.Hkv, 1 << w.kbits), np.int64)
    ref_v = np.zeros((w.Hkv, 1 << w.vbits), np.int64)
    for (b, h), e in encs.items():
        ref_k[h] += oracle.code_histogram(e["k_codes"][g0 * w.G:g1 * w.G], w.kbits)
        ref_v[h] += oracle.code_histogram(e["v_codes"][g0 * w.G:g1 * w.G], w.vbits)
    assert np.array_equal(kh.cpu().numpy(), ref_k)
    assert np.array_equal(vh.cpu().numpy(), ref_v)
    full = [x.cpu().numpy() for x in c.drift_check(kh, vh, 0, ng, THR)]
    part = [x.cpu().numpy() for x in c.drift_check(kh, vh, g0, g1, THR)]
    for f, p in zip(full, part):
        assert np.array_equal(f[:, g0:g1], p)
    for (b, h), e in encs.items():
        rk, rv, rf = oracle.drift_check(e["k_codes"][g0 * w.G:g1 * w.G], e["v_codes"][g0 * w.G:g1 * w.G], w.G, w.D,
                                        w.kbits, w.vbits, ref_k[h], ref_v[h], THR)
        np.testing.assert_allclose(part[0][h], rk, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(part[1][h], rv, rtol=1e-12, atol=1e-15)


def test_drift_check_with_empty_calibration_matches_oracle():
    """A calibration histogram with no counts (on both sides, then on the key
    side only): KL and flags equal the oracle's -- +inf against an empty
    calibration, with the flag set -- and the non-empty side its KL."""
    kvq = _lib()
    import oracle

    w = DRIFT[0].replace(name="drift-empty-cal", B=1, Hq=4, Hkv=2, N=1500)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    ng = c.num_groups()
    encs = oracle_encode_slices(w, K, V, [(0, h) for h in range(w.Hkv)])
    _, vh_full = c.code_histograms(0, ng)
    kh = torch.zeros((w.Hkv, 1 << w.kbits), dtype=torch.int64, device="cuda")
    for vh in (torch.zeros((w.Hkv, 1 << w.vbits), dtype=torch.int64, device="cuda"), vh_full):
        kl_k, kl_v, flags = (x.cpu().numpy() for x in c.drift_check(kh, vh, 0, ng, THR))
        vh_host = vh.cpu().numpy()
        for (b, h), e in encs.items():
            rk, rv, rf = oracle.drift_check(e["k_codes"], e["v_codes"], w.G, w.D, w.kbits, w.vbits,
                                            np.zeros(1 << w.kbits, np.int64), vh_host[h], THR)
            assert np.isposinf(rk).all()
            assert np.array_equal(kl_k[h], rk)
            np.testing.assert_allclose(kl_v[h], rv, rtol=1e-12, atol=1e-15)
            assert np.array_equal(flags[h], rf)