"""kvq_decode_attn_noalloc (split partials in the library's per-device scratch
array) against kvq_decode_attn (caller workspace), through the C ABI: the
same kernels at the same split count, so the outputs must be identical, on
two calls in a row, the second with a smaller cache; a decode whose partials
exceed the scratch is refused before anything is enqueued."""
import ctypes

import pytest
import torch

from _parity import log
from synth import WORKLOADS, Synth

pytestmark = pytest.mark.gpu


def _run(kvq, w):
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    q = syn.q()
    ref = c.decode(q)
    out = torch.full_like(ref, float("nan"))
    c.decode_noalloc(q, out)
    torch.cuda.synchronize()
    log(f"[noalloc] {w.name}: splits {c.default_splits()}, max |diff| {(out - ref).abs().max().item():.3e}")
    assert torch.isfinite(ref).all()
    assert torch.equal(out, ref)
    return c


def test_noalloc_equals_workspace_decode_twice():
    import decode_attention_asym_amd as kvq

    big = WORKLOADS[1].replace(name="noalloc-8k", B=4, N=8192 + 77)
    small = WORKLOADS[2].replace(name="noalloc-small", B=1, Hq=8, Hkv=2, N=900)
    for w in (big, small):
        _run(kvq, w)


def test_noalloc_equals_workspace_decode_merged_in_kernel():
    """A decode whose splits merge inside the kernel (the 32k layer's slice
    count) uses no partials: the no-allocation entry point gives the same
    output, and does not need the scratch array."""
    import decode_attention_asym_amd as kvq

    w = WORKLOADS[2].replace(name="noalloc-merged", N=64 * 16 + 128 + 5)
    c = _run(kvq, w)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert c.decode_plan() == (4, True, 0)


def test_noalloc_refuses_partials_beyond_the_scratch():
    import decode_attention_asym_amd as kvq

    # 8192 slices at the minimum of two splits: 32768 rows x 2 x 132 floats > 32 MiB
    w = WORKLOADS[1].replace(name="noalloc-too-big", B=1024, Hq=32, Hkv=8, N=200, R=32)
    syn = Synth(w, "cuda")
    K, V = syn.kv_all()
    c = kvq.KVQCache(kvq.config_for(w))
    c.append(K, V)
    assert c.default_splits() == 2
    need = w.B * w.Hq * 2 * (w.D + 4) * 4
    assert need > 32 << 20
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KVQError, match="no-allocation scratch"):
        c.decode_noalloc(syn.q(), out)
    torch.cuda.synchronize()
    assert not out.any()  # nothing was enqueued
    # the cache still decodes through the workspace entry point
    assert torch.isfinite(c.decode(syn.q())).all()
