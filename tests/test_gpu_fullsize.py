"""Parity at the full workload sizes, in the launch configuration bench.py
times (default split count): the oracle checks sampled (batch) rows one by
one -- every kv head of those rows bit-exact, every query head's attention
within relative L2 2e-3."""
import numpy as np
import pytest
import torch

from _parity import (TOL_REL_L2, assert_export_matches, log, oracle_encode_slices, oracle_rows, rel_l2)
from synth import WORKLOADS, Synth, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [2, 3, 4], ids=["llama3-8b-32k-k4v2-drift", "70b-128k", "175b-mha-fwht"])
def test_full_size_sampled_rows(idx):
    import decode_attention_asym_amd as kvq

    w = WORKLOADS[idx]
    log(f"[full] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N}")
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    cache = kvq.KVQCache(kvq.config_for(w))
    cache.append(K, V)
    q = syn.q()
    out = cache.decode(q)  # default split count, as timed by bench.py
    torch.cuda.synchronize()
    log(f"[full] {w.name}: splits {cache.default_splits()}")
    q_host = to_oracle_input(q, w.dtype)
    got, ref = [], []
    for b in (0, w.B - 1):
        exp = cache.export(b, 1)
        encs = oracle_encode_slices(w, K, V, [(b, h) for h in range(w.Hkv)])
        assert_export_matches(w, exp, b, encs)
        ref.append(oracle_rows(w, exp, b, q_host, [b])[b])
        got.append(out[b].double().cpu().numpy())
    err, worst = rel_l2(np.stack(got), np.stack(ref))
    log(f"[full] {w.name}: codes bit-exact on sampled rows; rel L2 {err:.3e} (worst row {worst:.3e})")
    assert err <= TOL_REL_L2


def test_70b_append_decode_steps_cross_flushes():
    """The 70B-shaped 128k workload's step loop: 64 steps of append(1) +
    decode, two group flushes (G = 32) on the way; decode checked at steps
    that straddle a flush, cache contents bit-exact at the end."""
    import decode_attention_asym_amd as kvq

    w = WORKLOADS[3]
    steps = 64
    syn = Synth(w, "cuda", positions=w.N + steps + 1)
    K, V = syn.kv_all()
    cache = kvq.KVQCache(kvq.config_for(w, max_tokens=w.N + steps))
    cache.append(K, V)
    ks, vs = [], []
    errs = []
    for i in range(steps):
        k, v = syn.step_kv(i)
        ks.append(k)
        vs.append(v)
        cache.append(k, v)
        q = syn.q(i)
        out = cache.decode(q)
        if i in (0, 30, 31, 32, 63):
            torch.cuda.synchronize()
            exp = cache.export(0, 1)
            ref = oracle_rows(w, exp, 0, to_oracle_input(q, w.dtype), [0])[0]
            err, worst = rel_l2(out[0].double().cpu().numpy(), ref)
            log(f"[steps] step {i}: n={cache.num_tokens} nq={cache.num_quantized} rel L2 {err:.3e}")
            errs.append(err)
    assert max(errs) <= TOL_REL_L2
    Kall = torch.cat([K[:1]] + [k[:1] for k in ks], dim=2)
    Vall = torch.cat([V[:1]] + [v[:1] for v in vs], dim=2)
    encs = oracle_encode_slices(w, Kall, Vall, [(0, h) for h in range(w.Hkv)])
    assert_export_matches(w, cache.export(0, 1), 0, encs)
