"""Shared helpers of the GPU parity tests: run the oracle on host copies of the
same seeded inputs and compare with what the HIP library produced."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from synth import to_oracle_input

TOL_REL_L2 = 2e-3  # attention output vs the oracle on the same dequantized cache
THREADS = 16


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def oracle_group_bits(w, calls):
    """Per-group (key, value) bits of a position-adaptive workload appended in
    `calls` (token counts per append), or None without adaptive bits."""
    if not w.adapt_delta:
        return None
    return oracle.adaptive_group_bits(w.G, w.R, w.sink, w.adapt_delta, calls, w.bits_low, (w.kbits, w.vbits),
                                      w.bits_high)


def oracle_encode_slices(w, K, V, pairs, calls=None):
    """Oracle encoding of (b, hkv) slices.  K, V: torch [B, Hkv, n, D] (any
    device); calls: the append sizes that built the cache (adaptive bits)."""
    gb = oracle_group_bits(w, [K.shape[2]] if calls is None else calls)

    def enc(bh):
        b, h = bh
        k = to_oracle_input(K[b, h], w.dtype)
        v = to_oracle_input(V[b, h], w.dtype)
        e = oracle.encode_slice(k, v, w.dtype, w.D, w.kbits, w.vbits, w.G, w.R, w.rotate, sink=w.sink,
                                hybrid=w.hybrid, token_norm=w.token_norm, group_bits=gb)
        if gb is not None:
            e["gbits"] = gb
        return e

    with ThreadPoolExecutor(THREADS) as ex:
        return dict(zip(pairs, ex.map(enc, pairs)))


def assert_export_matches(w, exp, b0, encs):
    """exp: KVQCache.export(b0, ...) arrays; encs: {(b, h): oracle encoding}."""
    for (b, h), enc in encs.items():
        bi = b - b0
        assert exp["nq"] == enc["nq"], (exp["nq"], enc["nq"])
        if "gbits" in enc:
            ng = enc["nq"] // w.G
            assert np.array_equal(exp["k_gbits"], enc["gbits"][0][:ng]), "key group bits"
            assert np.array_equal(exp["v_gbits"], enc["gbits"][1][:ng]), "value group bits"
        code_keys = (("k_codes", w.kbits), ("v_codes", w.vbits))
        if "k_codes_u8" in exp:  # mixed widths: one code per byte
            code_keys = ()
            for key in ("k_codes", "v_codes"):
                got = exp[key + "_u8"][bi, h]
                if not np.array_equal(got, enc[key]):
                    bad = np.argwhere(got != enc[key])
                    raise AssertionError(f"{key} mismatch at slice ({b},{h}): {len(bad)} codes, first {bad[:5].tolist()}")
        for key, bits in code_keys:
            ref = oracle.pack_codes(enc[key], bits) if enc["nq"] else np.zeros((0, w.D * bits // 8), np.uint8)
            got = exp[key][bi, h]
            if not np.array_equal(got, ref):
                bad = np.argwhere(got != ref)
                raise AssertionError(f"{key} mismatch at slice ({b},{h}): {len(bad)} bytes, first {bad[:5].tolist()}")
        keys = ("k_scale", "k_zero", "v_scale", "v_zero", "k_resid", "v_resid") + (("k_norm",) if "k_norm" in enc else ())
        for key in keys:
            got = exp[key][bi, h]
            if not np.array_equal(got, enc[key]):
                bad = np.argwhere(got != enc[key])
                raise AssertionError(f"{key} mismatch at slice ({b},{h}): {len(bad)} elements, first {bad[:5].tolist()}")


def canonical_slice(exp, bi, h, D, kbits, vbits):
    """One slice of an export as an oracle cache dict (codes unpacked)."""
    if "k_codes_u8" in exp:
        kc = exp["k_codes_u8"][bi, h].astype(np.uint16)
        vc = exp["v_codes_u8"][bi, h].astype(np.uint16)
    else:
        kc = oracle.unpack_codes(exp["k_codes"][bi, h], D, kbits)
        vc = oracle.unpack_codes(exp["v_codes"][bi, h], D, vbits)
    return {
        "k_codes": kc,
        "v_codes": vc,
        "k_scale": exp["k_scale"][bi, h], "k_zero": exp["k_zero"][bi, h],
        "v_scale": exp["v_scale"][bi, h], "v_zero": exp["v_zero"][bi, h],
        "k_resid": exp["k_resid"][bi, h], "v_resid": exp["v_resid"][bi, h],
        "nq": exp["nq"], "n": exp["n"],
        "k_norm": exp["k_norm"][bi, h] if "k_norm" in exp else None,
    }


def oracle_queries(w, q_host_b):
    """[Hq, D] fp64 queries of one batch row (rotated when the keys are)."""
    q = oracle.input_to_f64(q_host_b, w.dtype).reshape(w.Hq, w.D)
    if w.rotate:
        q = np.stack([oracle.rotate_f64(x) for x in q])
    return q


def oracle_rows(w, exp, b0, q_host, batches):
    """Oracle attention for every query head of the given batch rows, on the
    exported (dequantized) cache.  Returns {b: [Hq, D] fp64}."""
    jobs, keys = [], []
    for b in batches:
        qb = oracle_queries(w, q_host[b])
        for h in range(w.Hkv):
            cache = canonical_slice(exp, b - b0, h, w.D, w.kbits, w.vbits)
            jobs.append((qb[h * w.gqa:(h + 1) * w.gqa], cache, w.D, w.G, w.R))
            keys.append((b, h))
    outs = oracle.attend_slices_parallel(jobs, THREADS)
    res = {b: np.zeros((w.Hq, w.D)) for b in batches}
    for (b, h), o in zip(keys, outs):
        res[b][h * w.gqa:(h + 1) * w.gqa] = o
    return res


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rows = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=1) / np.maximum(
        np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1), 1e-300)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), float(rows.max())
