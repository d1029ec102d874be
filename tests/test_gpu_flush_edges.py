"""The flush kernel on the quantizer's edge cases (tests/edge_inputs.py):
planted exact half-integer quotients (the kernel's division fallback and
round-half-even), quotients within 2^-12 of a half-integer, constant and
signed-zero groups, fp16 subnormals and the largest finite inputs -- codes,
scales, zeros and window bit-exact against the oracle, for a prefill and for
one-token appends that flush group by group, in f32, f16 and bf16 inputs."""
import numpy as np
import pytest
import torch

from _parity import assert_export_matches, log, oracle_encode_slices
from edge_inputs import edge_kv
from synth import WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [
    # (name, D, kbits, vbits, G, R, dtype, hybrid)
    ("d128-k2v2-g32-f32", 128, 2, 2, 32, 32, "f32", False),
    ("d64-k4v4-g64-f16-r0", 64, 4, 4, 64, 0, "f16", False),
    ("d128-k4v2-g64-bf16-hybrid", 128, 4, 2, 64, 128, "bf16", True),
    ("d64-k2v4-g32-f16-hybrid", 64, 2, 4, 32, 32, "f16", True),
]
_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_flush_edge_cases_bit_exact(case):
    import decode_attention_asym_amd as kvq

    name, D, kb, vb, G, R, dtype, hybrid = case
    N = R + 6 * G + 5
    steps = 2 * G + 3  # one-token appends crossing two flushes
    w = WORKLOADS[0].replace(name=name, B=1, Hq=2, Hkv=2, D=D, N=N, kbits=kb, vbits=vb, G=G, R=R, dtype=dtype,
                             hybrid=hybrid)
    Kn, Vn = edge_kv(w.B, w.Hkv, N, D, G, kb, vb, dtype, seed=D + kb * 10 + vb)
    K = torch.from_numpy(Kn).to(_TORCH[dtype]).cuda()
    V = torch.from_numpy(Vn).to(_TORCH[dtype]).cuda()
    # the conversion to the input dtype is exact for every planted value
    assert torch.equal(K.float().cpu(), torch.from_numpy(Kn)) or dtype == "bf16"
    pairs = [(0, h) for h in range(w.Hkv)]
    encs = oracle_encode_slices(w, K, V, pairs)
    # one prefill
    a = kvq.KVQCache(kvq.config_for(w))
    a.append(K, V)
    assert_export_matches(w, a.export(), 0, encs)
    # a shorter prefill, then one token at a time (groups flushed from the window ring)
    b = kvq.KVQCache(kvq.config_for(w))
    b.append(K[:, :, :N - steps].contiguous(), V[:, :, :N - steps].contiguous())
    for t in range(N - steps, N):
        b.append(K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous())
    assert_export_matches(w, b.export(), 0, encs)
    enc = encs[(0, 0)]
    log(f"[edges] {name}: {enc['nq'] // G} groups bit-exact (prefill and one-token appends); "
        f"constant-group key scales: {int(np.sum(enc['k_scale'] == 0))}")
