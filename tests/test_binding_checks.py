"""The binding's argument checks (CPU): a tensor on the wrong device, of the
wrong dtype, strided, or of the wrong shape raises ValueError before any call
into the library -- the C ABI takes bare pointers and could not tell."""
import pytest
import torch

import decode_attention_asym_amd as kvq
from decode_attention_asym_amd.kvq import KVQCache, merge_partials

B, HQ, HKV, D, G = 2, 8, 2, 128, 32


def _cache(dtype="bf16"):
    """A handle-less cache object that believes it lives on cuda:0: every
    check runs as on the GPU, and a call that got past the checks would fail
    in the library on the NULL handle (KVQError), not with ValueError."""
    c = KVQCache.__new__(KVQCache)
    c.cfg = kvq.Config(batch=B, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, max_tokens=4096, k_bits=2, v_bits=2,
                       group_size=G, residual=32, in_dtype=dtype)
    c.device = torch.device("cuda", 0)
    c.h = None
    c.ws = torch.empty(16, dtype=torch.uint8, device="meta")
    return c


def _meta(shape, dtype=torch.bfloat16):
    # tensors that claim to be on the cache's device without a GPU: only
    # metadata is inspected by the checks
    return torch.empty(shape, dtype=dtype, device="meta")


def test_cpu_tensor_rejected():
    c = _cache()
    k = torch.zeros((B, HKV, 4, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on cpu"):
        c.append(k, k)
    with pytest.raises(ValueError, match="on cpu"):
        c.decode(torch.zeros((B, HQ, D), dtype=torch.bfloat16))


def test_checks_on_meta_tensors():
    c = _cache()
    c.device = torch.device("meta")
    good_kv = _meta((B, HKV, 4, D))
    # wrong dtype (fp16 into a bf16 config)
    with pytest.raises(ValueError, match="dtype"):
        c.append(_meta((B, HKV, 4, D), torch.float16), good_kv)
    # a transposed [B, T, H, D] view
    t = _meta((B, 4, HKV, D)).transpose(1, 2)
    with pytest.raises(ValueError, match="not contiguous"):
        c.append(t, good_kv)
    # wrong shapes
    with pytest.raises(ValueError, match="shape"):
        c.append(_meta((B, HKV + 1, 4, D)), _meta((B, HKV + 1, 4, D)))
    with pytest.raises(ValueError, match="shape"):
        c.append(good_kv, _meta((B, HKV, 5, D)))
    with pytest.raises(ValueError, match="shape"):
        c.decode(_meta((B, HQ - 1, D)))
    # out of the wrong dtype or shape
    q = _meta((B, HQ, D))
    with pytest.raises(ValueError, match="dtype"):
        c.decode(q, out=_meta((B, HQ, D), torch.float16))
    with pytest.raises(ValueError, match="shape"):
        c.decode(q, out=_meta((B * HQ * D,), torch.float32))
    # one-token steps take exactly one token
    with pytest.raises(ValueError, match="shape"):
        c.append_decode(good_kv, good_kv, q)
    # partials must be float32
    with pytest.raises(ValueError, match="dtype"):
        c.decode_partials(q, partials=_meta((B * HQ, 4, D + 4), torch.float16))
    # drift: calibration counts are int64 [H_kv, 2^bits]
    with pytest.raises(ValueError, match="dtype"):
        c.drift_check(_meta((HKV, 4), torch.int32), _meta((HKV, 4), torch.int64), 0, 1)
    with pytest.raises(ValueError, match="shape"):
        c.drift_check(_meta((HKV, 16), torch.int64), _meta((HKV, 4), torch.int64), 0, 1)
    # requantize: tokens of exactly the group range, flags uint8 [B * H_kv, groups]
    kv2 = _meta((B, HKV, 2 * G, D))
    with pytest.raises(ValueError, match="shape"):
        c.requantize(good_kv, good_kv, 0, 2)
    with pytest.raises(ValueError, match="shape"):
        c.requantize(kv2, kv2, 0, 2, flags=_meta((B * HKV, 3), torch.uint8))


def test_checks_pass_through_to_the_library():
    """Well-formed arguments reach the library, which then rejects the NULL
    handle: the checks do not stand in for the C side's own validation."""
    c = _cache()
    c.device = torch.device("meta")
    q = _meta((B, HQ, D))
    with pytest.raises(kvq.KVQError):
        c.decode(q, out=_meta((B, HQ, D), torch.float32), stream=0)


def test_merge_partials_checks():
    with pytest.raises(ValueError, match="GPU"):
        merge_partials(torch.zeros(100), torch.zeros(10), 1, 1, 64)
    with pytest.raises(ValueError):
        merge_partials(_meta((10,), torch.float32), _meta((10,), torch.float32), 0, 1, 64)


def test_cache_refuses_host_memory():
    cfg = _cache().cfg
    with pytest.raises(ValueError, match="not a GPU"):
        KVQCache(cfg, device="cpu")
