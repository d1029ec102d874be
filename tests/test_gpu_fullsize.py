"""Parity at the full workload sizes, in the launch configuration bench.py
times (default split count), on every (batch, kv head) slice: every code,
scale, zero and window value bit-exact against the oracle's encoding, and the
attention output of every query head of every sequence against the oracle's
fp64 attention on the same (exported) cache -- relative L2 over the whole
output within 2e-3, and each head's row within the same bound, so that an
error confined to one head or split cannot hide in the norm of the rest."""
import numpy as np
import pytest
import torch

from _parity import (TOL_REL_L2, assert_export_matches, log, oracle_encode_slices, oracle_rows)
from synth import WORKLOADS, Synth, to_oracle_input

pytestmark = pytest.mark.gpu

ROW_TOL = 2e-3  # relative L2 of any one (sequence, query head) output row
SLICES_PER_PASS = 16


class _Err:
    """Accumulates the squared errors of output rows against the oracle."""

    def __init__(self):
        self.num = self.den = 0.0
        self.rows = []

    def add(self, got, ref):
        d = got - ref
        self.num += float((d ** 2).sum())
        self.den += float((ref ** 2).sum())
        self.rows.extend((np.linalg.norm(d, axis=-1) / np.linalg.norm(ref, axis=-1)).ravel().tolist())

    def report(self, tag):
        whole = (self.num / self.den) ** 0.5
        r = np.asarray(self.rows)
        log(f"[full] {tag}: rel L2 {whole:.3e} over {r.size} rows; per row median {np.median(r):.2e}, "
            f"p99 {np.percentile(r, 99):.2e}, max {r.max():.2e}")
        return whole, float(r.max())


def check_every_slice(w, cache, K, V, q, out, calls=None, tag=""):
    """Every slice's export against the oracle encoding of K, V, and every
    output row against the oracle's attention on the export."""
    q_host = to_oracle_input(q, w.dtype)
    rows_per_pass = max(1, SLICES_PER_PASS // w.Hkv)
    err = _Err()
    for b0 in range(0, w.B, rows_per_pass):
        bc = min(rows_per_pass, w.B - b0)
        exp = cache.export(b0, bc)
        batches = list(range(b0, b0 + bc))
        encs = oracle_encode_slices(w, K, V, [(b, h) for b in batches for h in range(w.Hkv)], calls)
        assert_export_matches(w, exp, b0, encs)
        del encs
        ref = oracle_rows(w, exp, b0, q_host, batches)
        for b in batches:
            err.add(out[b].double().cpu().numpy(), ref[b])
    whole, worst = err.report(tag or w.name)
    assert whole <= TOL_REL_L2, whole
    assert worst <= ROW_TOL, worst


# the oracle's encoding and fp64 attention of every slice take one to two
# minutes of host time per workload on a 16-core share
@pytest.mark.timeout(480)
@pytest.mark.parametrize("idx", [2, 3, 4], ids=["llama3-8b-32k-k4v2-drift", "70b-128k", "175b-mha-fwht"])
def test_full_size_every_slice(idx):
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
    check_every_slice(w, cache, K, V, q, out)


@pytest.mark.timeout(480)
def test_70b_append_decode_steps_cross_flushes():
    """The 70B-shaped 128k workload's step loop: 64 one-call steps
    (kvq_append_decode_attn: append one token, whose window write the decode
    does, then decode), two group flushes (G = 32) on the way; the decode of
    every sequence checked at steps that straddle a flush, every slice's cache
    contents bit-exact at those steps."""
    import decode_attention_asym_amd as kvq

    w = WORKLOADS[3]
    steps = 64
    syn = Synth(w, "cuda", positions=w.N + steps + 1)
    K, V = syn.kv_all()
    cache = kvq.KVQCache(kvq.config_for(w, max_tokens=w.N + steps))
    cache.append(K, V)
    ks, vs = [], []
    for i in range(steps):
        k, v = syn.step_kv(i)
        ks.append(k)
        vs.append(v)
        q = syn.q(i)
        out = cache.append_decode(k, v, q)
        if i in (0, 30, 31, 32, 63):
            torch.cuda.synchronize()
            log(f"[steps] step {i}: n={cache.num_tokens} nq={cache.num_quantized}")
            Kall = torch.cat([K] + ks, dim=2)
            Vall = torch.cat([V] + vs, dim=2)
            check_every_slice(w, cache, Kall, Vall, q, out, tag=f"{w.name} step {i}")
            del Kall, Vall
