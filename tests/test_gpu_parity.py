"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.  Codes, fp16 scales/zeros and the fp16 window must match
bit for bit; attention must be within relative L2 2e-3 of the oracle's fp64
attention on the exported (dequantized) cache, over the whole output and for
every (sequence, query head) row."""
import numpy as np
import pytest
import torch

from _parity import (TOL_REL_L2, assert_export_matches, log, oracle_encode_slices, oracle_rows, rel_l2)
from synth import WORKLOADS, Synth, to_oracle_input

pytestmark = pytest.mark.gpu


def _lib():
    import decode_attention_asym_amd as kvq

    return kvq


def _run_prefill(w, max_tokens=None, seed_positions=None):
    kvq = _lib()
    syn = Synth(w, "cuda", positions=seed_positions)
    K, V = syn.kv_all()
    cache = kvq.KVQCache(kvq.config_for(w, max_tokens))
    cache.append(K, V)
    q = syn.q()
    return syn, K, V, q, cache


def _check_full(w, splits=None, check_codes=True, batches=None):
    log(f"[parity] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} N={w.N} K{w.kbits}V{w.vbits} G={w.G} R={w.R} "
        f"rot={w.rotate} {w.dtype} splits={splits}")
    syn, K, V, q, cache = _run_prefill(w)
    out = cache.decode(q, splits=splits)
    torch.cuda.synchronize()
    batches = list(range(w.B)) if batches is None else batches
    q_host = to_oracle_input(q, w.dtype)
    res = []
    for b in batches:
        exp = cache.export(b, 1)
        if check_codes:
            encs = oracle_encode_slices(w, K, V, [(b, h) for h in range(w.Hkv)])
            assert_export_matches(w, exp, b, encs)
        ref = oracle_rows(w, exp, b, q_host, [b])[b]
        res.append((out[b].double().cpu().numpy(), ref))
    got = np.stack([r[0] for r in res])
    ref = np.stack([r[1] for r in res])
    err, worst = rel_l2(got, ref)
    log(f"[parity] {w.name}: rel L2 {err:.3e} (worst row {worst:.3e}) over batches {batches[:4]}...")
    assert err <= TOL_REL_L2 and worst <= TOL_REL_L2
    return cache, K, V, q, out


SMALL = [
    WORKLOADS[0],
    WORKLOADS[2].replace(name="k4v2-g64-drift-ragged", B=2, N=4096 + 77),
    WORKLOADS[3].replace(name="gqa8-r32-ragged", B=1, N=8192 + 45),
    WORKLOADS[4].replace(name="mha-fwht-ragged", B=2, Hq=8, Hkv=8, N=2048 + 13),
    WORKLOADS[1].replace(name="d64-k4v4-g64-gqa2-f16", B=3, Hq=4, Hkv=2, D=64, N=1000, kbits=4, vbits=4, G=64, R=64, dtype="f16"),
    WORKLOADS[1].replace(name="k2v4-g32-gqa16-r0", B=1, Hq=32, Hkv=2, N=700, kbits=2, vbits=4, G=32, R=0),
    WORKLOADS[1].replace(name="d64-k2v4-g32-gqa8", B=2, Hq=16, Hkv=2, D=64, N=1500 + 3, kbits=2, vbits=4, G=32, R=32),
    WORKLOADS[1].replace(name="d64-k4v2-g64-gqa1", B=2, Hq=3, Hkv=3, D=64, N=900 + 9, kbits=4, vbits=2, G=64, R=64),
    WORKLOADS[0].replace(name="d64-rot-k4v2-g32", B=2, Hq=4, Hkv=4, N=333, kbits=4, vbits=2, rotate=True),
    WORKLOADS[1].replace(name="window-only", B=2, N=100, R=128),
    WORKLOADS[1].replace(name="single-token", B=2, N=1, R=32),
    WORKLOADS[1].replace(name="window-full", B=2, N=128 + 31, R=128),
    WORKLOADS[1].replace(name="first-flush", B=2, N=128 + 32, R=128),
    # attention-sink fp16 window and the per-group symmetric/asymmetric choice
    WORKLOADS[2].replace(name="sink64-hybrid-k4v2-g64", B=2, N=4096 + 77, sink=64, hybrid=True),
    WORKLOADS[3].replace(name="sink32-gqa8-r32", B=1, N=2000 + 5, sink=32),
    WORKLOADS[1].replace(name="hybrid-k2v4-g32", B=2, N=1500 + 9, vbits=4, hybrid=True),
    WORKLOADS[0].replace(name="d64-rot-sink-hybrid", B=2, Hq=4, Hkv=2, N=600 + 3, kbits=4, vbits=2, rotate=True,
                         sink=64, hybrid=True),
    WORKLOADS[1].replace(name="sink-only", B=2, N=100, R=32, G=64, sink=128),
    WORKLOADS[1].replace(name="sink-no-flush-yet", B=2, N=64 + 128 + 31, R=128, sink=64),
    WORKLOADS[1].replace(name="sink-first-flush", B=2, N=64 + 128 + 32, R=128, sink=64),
    WORKLOADS[4].replace(name="mha-fwht-sink-hybrid", B=1, Hq=8, Hkv=8, N=1024 + 13, sink=32, hybrid=True),
    # key token norms after the rotation (rotate-then-scale keys), with and without rotation
    WORKLOADS[4].replace(name="mha-fwht-tokennorm", B=2, Hq=8, Hkv=8, N=2048 + 13, token_norm=True),
    WORKLOADS[2].replace(name="k4v2-g64-rot-tokennorm", B=2, N=3000 + 21, rotate=True, token_norm=True),
    WORKLOADS[3].replace(name="gqa8-tokennorm-sink-hybrid", B=1, N=1500 + 7, token_norm=True, sink=64, hybrid=True),
    WORKLOADS[0].replace(name="d64-tokennorm-k4v4", B=2, Hq=4, Hkv=2, N=700 + 1, kbits=4, vbits=4, token_norm=True),
    # position-adaptive bit widths (early / middle / recent groups), one prefill
    WORKLOADS[2].replace(name="adapt-k4v2-lo22-hi44", B=2, N=3000 + 21, adapt_delta=512, bits_low=(2, 2),
                         bits_high=(4, 4)),
    WORKLOADS[1].replace(name="adapt-k2v2-lo24-hi42-sink", B=2, N=2000 + 3, sink=64, adapt_delta=256,
                         bits_low=(2, 4), bits_high=(4, 2)),
    WORKLOADS[0].replace(name="d64-adapt-tokennorm-gqa2", B=2, Hq=4, Hkv=2, N=900 + 5, token_norm=True,
                         adapt_delta=128, bits_low=(4, 4), bits_high=(4, 4)),
    WORKLOADS[3].replace(name="gqa8-adapt-hybrid", B=1, N=2500 + 9, hybrid=True, adapt_delta=640,
                         bits_low=(4, 2), bits_high=(4, 4)),
    WORKLOADS[1].replace(name="adapt-delta-covers-all", B=2, N=700 + 3, adapt_delta=4096, bits_low=(2, 2),
                         bits_high=(4, 4)),
    # gqa 1 (the head in every slot, a value group per slot) on the mixed-width kernel
    WORKLOADS[4].replace(name="mha-fwht-adapt-lo22-hi44", B=1, Hq=6, Hkv=6, N=2000 + 11, adapt_delta=512,
                         bits_low=(2, 2), bits_high=(4, 4)),
    WORKLOADS[0].replace(name="d64-mha-adapt-g64-tokennorm", B=2, Hq=3, Hkv=3, N=1200 + 5, G=64, R=64,
                         token_norm=True, adapt_delta=256, bits_low=(4, 2), bits_high=(2, 4)),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_prefill_bitexact_and_decode(w):
    _check_full(w)


def test_llama8b_8k_full():
    """The 8B-shaped 8k workload at full size: every slice bit-exact, every row checked."""
    _check_full(WORKLOADS[1])


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 16])
def test_split_counts_agree(splits):
    w = WORKLOADS[1].replace(name="splits", B=2, N=3000 + 17)
    _check_full(w, splits=splits, check_codes=(splits == 1))


def _split_ranges(n, ng, G, S_req, sink=0):
    """Canonical token ranges (quantized tokens first, then the fp16 tokens:
    sink, then window) of each split: a contiguous, group-aligned run of
    ceil(ng / S) groups, plus the fp16 chunks f (the sink's 32-token chunks,
    then the window's) with f mod S = S - 1 - s."""
    S = min(S_req, max(1, ng))
    gps = -(-ng // S) if ng else 0
    if gps:
        S = -(-ng // gps)
    nq = ng * G
    ns = min(n, sink)
    nsc = -(-ns // 32)
    nwin = n - sink - nq if n > sink else 0
    chunks = [(nq + 32 * c, nq + min(ns, 32 * c + 32)) for c in range(nsc)]
    chunks += [(nq + ns + 32 * w, nq + ns + min(nwin, 32 * w + 32)) for w in range(-(-nwin // 32))]
    ranges = []
    for s in range(S):
        r = [(min(ng, s * gps) * G, min(ng, (s + 1) * gps) * G)]
        r += [chunks[f] for f in range(S - 1 - s, len(chunks), S)]
        ranges.append([x for x in r if x[1] > x[0]])
    return S, ranges


@pytest.mark.parametrize("base,sink,tn,S_req,gqa", [(2, 0, False, 4, 4), (2, 64, False, 4, 4), (2, 0, True, 4, 4),
                                                    (1, 0, False, 8, 4), (1, 0, True, 8, 4), (1, 64, False, 8, 4),
                                                    (1, 0, False, 8, 1), (1, 64, True, 6, 1), (2, 0, True, 4, 1)])
def test_decode_partials_per_split_match_oracle(base, sink, tn, S_req, gqa):
    """kvq_decode_partials: every split's (m, l, o) against the oracle's partial
    attention over the same tokens; kvq_merge_partials of them equals
    kvq_decode_attn_splits with the same split count (64- and 32-token groups,
    with and without sink chunks and key token norms; gqa 4, and gqa 1, whose
    records are written by the head slots of their value groups)."""
    kvq = _lib()
    import oracle
    from _parity import canonical_slice, oracle_queries

    w = WORKLOADS[base].replace(name=f"partials-g{WORKLOADS[base].G}-sink{sink}-tn{int(tn)}-gqa{gqa}", B=2,
                                Hq=2 * gqa, Hkv=2, N=sink + 64 * 9 + 128 + 21, sink=sink, token_norm=tn)
    syn, K, V, q, cache = _run_prefill(w)
    partials, S = cache.decode_partials(q, splits=S_req)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    kvq.merge_partials(partials, out, w.B * w.Hq, S, w.D)
    full = cache.decode(q, splits=S_req)  # the same splits through kvq_decode_attn_splits
    torch.cuda.synchronize()
    err, _ = rel_l2(full.double().cpu().numpy(), out.double().cpu().numpy())
    assert err <= 1e-6, err
    exp = cache.export()
    ng = exp["nq"] // w.G
    S_exp, ranges = _split_ranges(w.N, ng, w.G, S_req, sink)
    assert S == S_exp
    P = partials.reshape(-1)[:w.B * w.Hq * S * (w.D + 4)].double().cpu().numpy().reshape(w.B, w.Hq, S, w.D + 4)
    q_host = to_oracle_input(q, w.dtype)
    log2e = 1.0 / np.log(2.0)
    for b in range(w.B):
        qb = oracle_queries(w, q_host[b])
        for h in range(w.Hkv):
            sl = canonical_slice(exp, b, h, w.D, w.kbits, w.vbits)
            hq = slice(h * w.gqa, (h + 1) * w.gqa)
            for s, rs in enumerate(ranges):
                # the oracle's partial over the split's token ranges, merged (O9)
                parts = [oracle.attend_partial(qb[hq], sl, w.D, w.G, w.R, t0, t1) for t0, t1 in rs]
                m = np.max([pp[0] for pp in parts], axis=0)
                l = sum(pp[1] * np.exp(pp[0] - m) for pp in parts)
                o = sum(pp[2] * np.exp(pp[0] - m)[:, None] for pp in parts)
                got = P[b, hq, s]
                # m is the kernel's lazily moved reference point: at most 0.5 below the max
                mx = m * log2e
                assert np.all(got[:, w.D] <= mx + 1e-3) and np.all(got[:, w.D] >= mx - 0.5 - 1e-3), (b, h, s)
                l_at_max = got[:, w.D + 1] * np.exp2(got[:, w.D] - mx)
                assert np.all(np.abs(l_at_max / l - 1.0) <= 2e-3), (b, h, s)
                err, worst = rel_l2(got[:, :w.D] / got[:, w.D + 1:w.D + 2], o / l[:, None])
                assert err <= TOL_REL_L2 and worst <= TOL_REL_L2, (b, h, s, err, worst)


@pytest.mark.parametrize("D,S", [(128, 1), (128, 6), (128, 8), (64, 13), (128, 17), (128, 24), (128, 33), (64, 37),
                                 (64, 64), (128, 64), (128, 65), (128, 100), (64, 256), (128, 256)])
def test_merge_partials_against_oracle(D, S):
    """kvq_merge_partials on seeded partials (wide score ranges, empty splits
    whose o and l hold NaN) against the oracle's split merge; up to 64
    records per row the merge runs one wave per row (37 rows: a partial
    block of four rows at the end), above that one block per row."""
    kvq = _lib()
    import oracle

    rows = 37
    rng = np.random.default_rng(1000 + 7 * D + S)
    m2 = rng.standard_normal((rows, S)) * 20.0
    empty = rng.random((rows, S)) < 0.2
    empty[:, 0] = False
    m2[empty] = -np.inf
    l = rng.uniform(0.5, 50.0, (rows, S))
    o = rng.standard_normal((rows, S, D)) * l[..., None]
    rec = np.zeros((rows, S, D + 4), np.float32)
    rec[..., :D] = o
    rec[..., D] = m2
    rec[..., D + 1] = l
    rec[..., D + 2:] = np.nan
    rec[empty, :D] = np.nan
    rec[empty, D + 1] = np.nan
    part = torch.from_numpy(rec).cuda()
    out = torch.empty((rows, D), dtype=torch.float32, device="cuda")
    kvq.merge_partials(part, out, rows, S, D)
    torch.cuda.synchronize()
    r32 = rec.astype(np.float64)
    ln2 = np.log(2.0)
    o_ref = np.where(empty[..., None], 0.0, r32[..., :D])
    l_ref = np.where(empty, 0.0, r32[..., D + 1])
    ref = oracle.merge_partials((r32[..., D] * ln2).T, l_ref.T, o_ref.transpose(1, 0, 2))
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err, worst = rel_l2(got, ref)
    assert worst <= 1e-5, (err, worst)


def test_repeated_decodes_with_changing_split_counts():
    """Decodes on one cache with the split count changing from call to call
    (and one single-split call, which writes the output directly): every
    result matches the oracle."""
    w = WORKLOADS[2].replace(name="resplit", B=2, Hq=8, Hkv=2, N=64 * 23 + 128 + 5)
    syn, K, V, q, cache = _run_prefill(w)
    exp = cache.export()
    ref = oracle_rows(w, exp, 0, to_oracle_input(q, w.dtype), range(w.B))
    ref = np.stack([ref[b] for b in range(w.B)])
    for S in (5, 8, 3, 8, 1, 16, 23, 2):
        out = cache.decode(q, splits=S)
        torch.cuda.synchronize()
        err, worst = rel_l2(out.double().cpu().numpy(), ref)
        log(f"[parity] resplit splits={S}: rel L2 {err:.3e} (worst row {worst:.3e})")
        assert err <= TOL_REL_L2 and worst <= TOL_REL_L2, (S, err, worst)


@pytest.mark.parametrize("sink,hybrid,tn", [(0, False, False), (64, True, False), (64, True, True)])
def test_stepwise_append_equals_prefill(sink, hybrid, tn):
    kvq = _lib()
    w = WORKLOADS[2].replace(name="stepwise", B=2, Hkv=2, Hq=8, N=700, sink=sink, hybrid=hybrid, token_norm=tn)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    a = kvq.KVQCache(kvq.config_for(w))
    a.append(K, V)
    b = kvq.KVQCache(kvq.config_for(w))
    sizes = [1, 1, 7, 64, 1, 100, 3, 128, 65, 1, 1, 200]
    sizes.append(w.N - sum(sizes))
    t = 0
    for s in sizes:
        b.append(K[:, :, t:t + s].contiguous(), V[:, :, t:t + s].contiguous())
        t += s
    assert a.num_tokens == b.num_tokens == w.N
    ea, eb = a.export(), b.export()
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid") + (
            ("k_norm",) if tn else ()):
        assert np.array_equal(ea[key], eb[key]), key
    encs = oracle_encode_slices(w, K, V, [(bb, h) for bb in range(w.B) for h in range(w.Hkv)])
    assert_export_matches(w, ea, 0, encs)


@pytest.mark.parametrize("sink,tn", [(0, False), (64, True)])
def test_adaptive_stepwise_matches_oracle(sink, tn):
    """Position-adaptive bits built by a prefill and then appends: the groups'
    bits follow the lengths after each append, codes and parameters are
    bit-exact, and decode over the mixed-width runs (several split counts, so
    runs get one or more splits) matches the oracle."""
    kvq = _lib()
    w = WORKLOADS[2].replace(name="adaptive-stepwise", B=2, Hkv=2, Hq=8, N=2600, sink=sink, token_norm=tn,
                             adapt_delta=384, bits_low=(2, 2), bits_high=(4, 4))
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    sizes = [1500, 1, 64, 1, 200, 3, 130, 1]
    sizes.append(w.N - sum(sizes))
    t = 0
    q = syn.q()
    q_host = to_oracle_input(q, w.dtype)
    for i, sz in enumerate(sizes):
        c.append(K[:, :, t:t + sz].contiguous(), V[:, :, t:t + sz].contiguous())
        t += sz
        if i in (0, 4, len(sizes) - 1):
            exp = c.export()
            encs = oracle_encode_slices(w, K[:, :, :t], V[:, :, :t], [(b, h) for b in range(w.B) for h in range(w.Hkv)],
                                        calls=sizes[:i + 1])
            assert_export_matches(w, exp, 0, encs)
            kb, _ = c.group_bits()
            log(f"[adaptive] n={t}: group bits runs {np.flatnonzero(np.diff(kb.astype(int))).tolist()}")
            ref = oracle_rows(w, exp, 0, q_host, list(range(w.B)))
            refs = np.stack([ref[b] for b in range(w.B)])
            for splits in (1, 2, 7, None):
                out = c.decode(q, splits=splits)
                torch.cuda.synchronize()
                err, worst = rel_l2(out.double().cpu().numpy(), refs)
                log(f"[adaptive] n={t} splits={splits}: rel L2 {err:.3e} (worst row {worst:.3e})")
                assert err <= TOL_REL_L2 and worst <= TOL_REL_L2, (t, splits, err, worst)


def test_adaptive_many_runs_matches_oracle():
    """Appends of 512 tokens with Delta = 256 > R leave, per append, middle
    groups then two groups quantized while recent: more runs of equal widths
    than one mixed launch takes (8), so the decode falls back to one launch
    per run; before that, with fewer runs, it uses the mixed launch."""
    kvq = _lib()
    w = WORKLOADS[2].replace(name="adaptive-many-runs", B=1, Hkv=2, Hq=8, N=600 + 5 * 512, adapt_delta=256,
                             bits_low=(2, 2), bits_high=(4, 4))
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    sizes = [600] + [512] * 5
    q = syn.q()
    q_host = to_oracle_input(q, w.dtype)
    t = 0
    for i, sz in enumerate(sizes):
        c.append(K[:, :, t:t + sz].contiguous(), V[:, :, t:t + sz].contiguous())
        t += sz
        if i not in (2, len(sizes) - 1):
            continue
        kb, vb = c.group_bits()
        pair = kb.astype(int) * 16 + vb
        runs = 1 + int(np.count_nonzero(np.diff(pair)))
        log(f"[adaptive] n={t}: {runs} runs of equal widths")
        assert (runs <= 8) if i == 2 else (runs > 8)
        exp = c.export()
        encs = oracle_encode_slices(w, K[:, :, :t], V[:, :, :t], [(0, h) for h in range(w.Hkv)], calls=sizes[:i + 1])
        assert_export_matches(w, exp, 0, encs)
        ref = oracle_rows(w, exp, 0, q_host, [0])[0]
        for splits in (1, 5, None):
            out = c.decode(q, splits=splits)
            torch.cuda.synchronize()
            err, worst = rel_l2(out[0].double().cpu().numpy(), ref)
            log(f"[adaptive] n={t} splits={splits}: rel L2 {err:.3e} (worst row {worst:.3e})")
            assert err <= TOL_REL_L2 and worst <= TOL_REL_L2, (t, splits, err, worst)


def test_adaptive_rejects_import_and_packed_export():
    kvq = _lib()
    w = WORKLOADS[1].replace(name="adaptive-api", B=1, N=600, adapt_delta=128, bits_low=(2, 2), bits_high=(4, 4))
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    exp = c.export()
    assert exp["k_codes"] is None and exp["k_codes_u8"].shape == (1, w.Hkv, c.num_quantized, w.D)
    z = np.zeros(16, np.uint8)
    st = kvq.lib.kvq_export(c.h, 0, 1, z.ctypes.data, *([None] * 7), 0)
    assert st == kvq.KVQ_E_UNSUPPORTED
    arrs = [np.zeros(1 << 20, np.uint8) for _ in range(8)]
    st = kvq.lib.kvq_import(c.h, 600, 0, 1, *(a.ctypes.data for a in arrs), 0)
    assert st == kvq.KVQ_E_UNSUPPORTED


@pytest.mark.parametrize("tn", [False, True])
def test_import_then_decode_matches_oracle(tn):
    """Decode on a cache the oracle encoded (imported), independent of the GPU quantizer."""
    kvq = _lib()
    w = WORKLOADS[1].replace(name=f"import-tn{int(tn)}", B=2, N=2000 + 5, token_norm=tn, rotate=tn)
    syn = Synth(w, "cpu")
    K, V = syn.kv_all()
    encs = oracle_encode_slices(w, K, V, [(b, h) for b in range(w.B) for h in range(w.Hkv)])
    import oracle

    arrays = {}
    for key, bits in (("k_codes", w.kbits), ("v_codes", w.vbits)):
        arrays[key] = np.stack([np.stack([oracle.pack_codes(encs[(b, h)][key], bits) for h in range(w.Hkv)])
                                for b in range(w.B)])
    for key in ("k_scale", "k_zero", "v_scale", "v_zero", "k_resid", "v_resid") + (("k_norm",) if tn else ()):
        arrays[key] = np.stack([np.stack([encs[(b, h)][key] for h in range(w.Hkv)]) for b in range(w.B)])
    cache = kvq.KVQCache(kvq.config_for(w))
    cache.import_(arrays, w.N)
    exp = cache.export()
    for key in arrays:
        assert np.array_equal(exp[key], arrays[key]), key
    q = syn.q().cuda()
    out = cache.decode(q)
    ref = oracle_rows(w, exp, 0, to_oracle_input(q, w.dtype), range(w.B))
    err, worst = rel_l2(out.double().cpu().numpy(), np.stack([ref[b] for b in range(w.B)]))
    log(f"[parity] import: rel L2 {err:.3e} worst row {worst:.3e}")
    assert err <= TOL_REL_L2 and worst <= TOL_REL_L2


def test_identical_keys_give_mean_of_values():
    kvq = _lib()
    w = WORKLOADS[1].replace(name="identical-keys", B=1, Hq=4, Hkv=1, N=900)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    K = K[:, :, :1, :].expand(-1, -1, w.N, -1).contiguous()
    cache = kvq.KVQCache(kvq.config_for(w))
    cache.append(K, V)
    out = cache.decode(syn.q() * 4)
    exp = cache.export()
    # dequantized values: per token zero + code * scale
    import oracle

    codes = oracle.unpack_codes(exp["v_codes"][0, 0], w.D, w.vbits).astype(np.float64)
    f = lambda a: a.view(np.float16).astype(np.float64)
    vq = f(exp["v_zero"][0, 0]).repeat(w.G, 1) + codes * f(exp["v_scale"][0, 0]).repeat(w.G, 1)
    mean = np.concatenate([vq, f(exp["v_resid"][0, 0])]).mean(0)
    err = np.abs(out[0].double().cpu().numpy() - mean[None]).max()
    assert err < 1e-3 * np.abs(mean).max() + 1e-4


def test_capacity_and_empty_errors():
    kvq = _lib()
    w = WORKLOADS[0].replace(name="cap", N=64)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    cache = kvq.KVQCache(kvq.config_for(w, max_tokens=100))
    with pytest.raises(kvq.KVQError) as ei:
        cache.decode(syn.q())
    assert ei.value.status == kvq.KVQ_E_STATE
    cache.append(K, V)
    with pytest.raises(kvq.KVQError) as ei:
        cache.append(K, V)  # 128 > 100
    assert ei.value.status == kvq.KVQ_E_CAPACITY
    assert cache.num_tokens == 64
    out = cache.decode(syn.q())
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("kb,vb,G,hq", [(kb, vb, G, hq) for kb in (2, 4) for vb in (2, 4) for G in (32, 64)
                                        for hq in (1, 4, 8, 16)],
                         ids=lambda v: str(v))
def test_bits_group_gqa_matrix(kb, vb, G, hq):
    """Every decode kernel instantiation at D=128 (bit widths x group size x
    head-slot modes: gqa 1 with the head in every slot and a value group per
    slot, gqa 4, 8, 16), one kv head, ragged length."""
    w = WORKLOADS[1].replace(name=f"k{kb}v{vb}g{G}h{hq}", B=1, Hq=hq, Hkv=1, N=1000 + 7, kbits=kb, vbits=vb, G=G, R=64)
    _check_full(w, splits=1)


STEP = [
    WORKLOADS[2].replace(name="step-k4v2-g64", B=2, Hq=8, Hkv=2, N=1000 + 7),
    WORKLOADS[4].replace(name="step-mha-fwht", B=1, Hq=4, Hkv=4, N=500 + 60),
    WORKLOADS[0].replace(name="step-d64-gqa16-rot", B=2, Hq=32, Hkv=2, N=300 + 17, rotate=True),
    WORKLOADS[1].replace(name="step-sink-start", B=2, Hq=8, Hkv=2, N=20, sink=64, R=32),
    WORKLOADS[1].replace(name="step-r0", B=2, Hq=8, Hkv=2, N=640 + 30, R=0),
    WORKLOADS[2].replace(name="step-adapt-tokennorm", B=1, Hq=8, Hkv=2, N=1500, adapt_delta=256, bits_low=(2, 2),
                         bits_high=(4, 4), token_norm=True, rotate=True),
]


@pytest.mark.parametrize("w", STEP, ids=lambda w: w.name)
def test_step_entry_equals_separate_calls(w):
    """kvq_append_decode_attn gives bit-identical outputs and cache contents to
    kvq_append + kvq_decode_attn, step by step across group flushes (sink,
    R = 0, rotation, gqa 16, adaptive widths); the final state also matches
    the oracle."""
    kvq = _lib()
    steps = 70
    syn = Synth(w, "cuda", positions=w.N + steps + 1)
    K, V = syn.kv_all()
    a = kvq.KVQCache(kvq.config_for(w, w.N + steps))
    b = kvq.KVQCache(kvq.config_for(w, w.N + steps))
    a.append(K, V)
    b.append(K, V)
    ks, vs = [K], [V]
    for i in range(steps):
        k, v = syn.step_kv(i)
        q = syn.q(i + 1)
        a.append(k, v)
        oa = a.decode(q)
        ob = b.append_decode(k, v, q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {i}: outputs differ"
        ks.append(k)
        vs.append(v)
    ea, eb = a.export(), b.export()
    for key in ("k_scale", "k_zero", "v_scale", "v_zero", "k_resid", "v_resid") + (
            ("k_codes", "v_codes") if not w.adapt_delta else ("k_codes_u8", "v_codes_u8")):
        assert np.array_equal(ea[key], eb[key]), key
    # the stepped cache against the oracle
    Kall, Vall = torch.cat(ks, dim=2), torch.cat(vs, dim=2)
    calls = [w.N] + [1] * steps
    encs = oracle_encode_slices(w, Kall, Vall, [(bb, h) for bb in range(w.B) for h in range(w.Hkv)], calls=calls)
    assert_export_matches(w, eb, 0, encs)
    q = syn.q(steps)
    out = b.decode(q)
    torch.cuda.synchronize()
    ref = oracle_rows(w, eb, 0, to_oracle_input(q, w.dtype), list(range(w.B)))
    err, worst = rel_l2(out.double().cpu().numpy(), np.stack([ref[bb] for bb in range(w.B)]))
    log(f"[step] {w.name}: rel L2 {err:.3e} (worst row {worst:.3e}) after {steps} steps")
    assert err <= TOL_REL_L2 and worst <= TOL_REL_L2


def test_step_partials_and_argument_checks():
    kvq = _lib()
    w = WORKLOADS[2].replace(name="step-partials", B=2, Hq=8, Hkv=2, N=900)
    syn = Synth(w, "cuda", positions=w.N + 4)
    K, V = syn.kv_all()
    a = kvq.KVQCache(kvq.config_for(w, w.N + 3))
    b = kvq.KVQCache(kvq.config_for(w, w.N + 3))
    a.append(K, V)
    b.append(K, V)
    k, v = syn.step_kv(0)
    q = syn.q(1)
    a.append(k, v)
    pa, Sa = a.decode_partials(q, splits=3)
    pb, Sb = b.append_decode_partials(k, v, q, splits=3)
    torch.cuda.synchronize()
    # o, m, l of every split (the last two floats of a record are padding)
    assert Sa == Sb and torch.equal(pa[:, :, :w.D + 2], pb[:, :, :w.D + 2])
    # checked before anything is enqueued: the token count does not move
    n = b.num_tokens
    small = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KVQError):
        b.append_decode_partials(k, v, q, small, splits=3)
    with pytest.raises(kvq.KVQError):
        b.append_decode_partials(k, v, q, splits=10 ** 6)
    assert b.num_tokens == n
    b.append_decode(k, v, q)
    b.append_decode(k, v, q)
    with pytest.raises(kvq.KVQError):  # capacity
        b.append_decode(k, v, q)
    assert b.num_tokens == w.N + 3


def test_adaptive_pieces_at_many_split_counts():
    """The piece plan of a position-adaptive cache (big runs cut into partner
    pieces and pieces of T bytes, small runs last; per-run splits when that
    does not apply) gives the oracle's attention at every split count, and
    the partials of every plan merge to the same output."""
    kvq = _lib()
    w = WORKLOADS[2].replace(name="adaptive-pieces", B=2, Hkv=2, Hq=8, N=6000 + 37, adapt_delta=640,
                             bits_low=(2, 2), bits_high=(4, 4), sink=64)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    q = syn.q()
    exp = c.export()
    encs = oracle_encode_slices(w, K, V, [(b, h) for b in range(w.B) for h in range(w.Hkv)])
    assert_export_matches(w, exp, 0, encs)
    ref = oracle_rows(w, exp, 0, to_oracle_input(q, w.dtype), list(range(w.B)))
    refs = np.stack([ref[b] for b in range(w.B)])
    for splits in (1, 2, 3, 4, 5, 6, 9, 16, 40, None):
        out = c.decode(q, splits=splits)
        parts, S = c.decode_partials(q, splits=splits if splits else c.default_splits())
        merged = torch.empty_like(out)
        kvq.merge_partials(parts, merged, w.B * w.Hq, S, w.D)
        torch.cuda.synchronize()
        err, worst = rel_l2(out.double().cpu().numpy(), refs)
        log(f"[pieces] splits={splits}: {S} slots, rel L2 {err:.3e} (worst row {worst:.3e})")
        assert err <= TOL_REL_L2 and worst <= TOL_REL_L2, (splits, err, worst)
        assert torch.allclose(merged, out, rtol=1e-6, atol=1e-7), splits
