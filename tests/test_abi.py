"""CPU-only checks of the C ABI: the library loads, exports every entry point
include/kvq.h declares, and validates arguments on the host (no device work,
no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("kvq_create", "kvq_append", "kvq_decode_attn"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from decode_attention_asym_amd import kvq

    raw = ctypes.CDLL(kvq.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(kvq.SIGNATURES), "binding and header disagree"


def _cfg(**kw):
    from decode_attention_asym_amd import Config

    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=1000, k_bits=4, v_bits=2,
                group_size=64, residual=128, rotate=False, in_dtype="bf16")
    base.update(kw)
    return Config(**base)


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(k_bits=3), dict(v_bits=8), dict(group_size=16), dict(residual=48),
    dict(num_q_heads=6, num_kv_heads=2), dict(num_q_heads=64, num_kv_heads=2),
    dict(batch=0), dict(max_tokens=0), dict(head_dim=64, group_size=128),
    dict(sink_tokens=32), dict(sink_tokens=-64), dict(sink_tokens=1088),
])
def test_invalid_configs_rejected(bad):
    import decode_attention_asym_amd as kvq

    assert kvq.cache_bytes(_cfg(**bad)) == 0
    assert kvq.lib.kvq_last_error()


def test_cache_bytes_matches_bit_accounting():
    """Quantized pages hold exactly codes + fp16 scale/zero (the oracle's bits
    per element), plus a fp16 window ring of R + G tokens and the fp16
    attention-sink tokens per slice."""
    import decode_attention_asym_amd as kvq
    import oracle

    for kb, vb, G, R, D, S0 in ((4, 2, 64, 128, 128, 0), (2, 2, 32, 32, 128, 0), (2, 4, 32, 64, 64, 0),
                                (4, 2, 64, 128, 128, 64), (2, 2, 32, 32, 64, 96)):
        n = 10000
        c = _cfg(k_bits=kb, v_bits=vb, group_size=G, residual=R, head_dim=D, max_tokens=n,
                 num_q_heads=2, num_kv_heads=2, sink_tokens=S0)
        nq = oracle.num_quantized(n, G, R, S0)
        quant_bits = oracle.bits_per_element(n, kb, vb, G, R, sink=S0) * 2 * n * D - 2 * 16 * (n - nq) * D
        ring = (R + G) * D * 2 * 2
        sink = S0 * D * 2 * 2
        total = kvq.cache_bytes(c)
        slices = c.batch * c.num_kv_heads
        assert total >= slices * (quant_bits / 8 + ring + sink)
        assert total <= slices * (quant_bits / 8 + ring + sink) + 768


def test_host_validation_without_device_work():
    import decode_attention_asym_amd as kvq
    from decode_attention_asym_amd.kvq import lib

    c = _cfg()
    cc = c.c()
    need = kvq.cache_bytes(c)
    fake = 1 << 40  # never dereferenced: every call below fails or returns before device work
    h = ctypes.c_void_p()
    assert lib.kvq_create(ctypes.byref(cc), None, need, ctypes.byref(h)) == kvq.KVQ_E_ARG
    assert lib.kvq_create(ctypes.byref(cc), fake + 16, need, ctypes.byref(h)) == kvq.KVQ_E_ARG  # misaligned
    assert lib.kvq_create(ctypes.byref(cc), fake, need - 1, ctypes.byref(h)) == kvq.KVQ_E_ARG   # too small
    assert lib.kvq_create(ctypes.byref(cc), fake, need, ctypes.byref(h)) == kvq.KVQ_OK
    try:
        assert lib.kvq_num_tokens(h) == 0
        assert lib.kvq_append(h, fake, fake, 0, None) == kvq.KVQ_OK  # no-op
        assert lib.kvq_append(h, fake, fake, -1, None) == kvq.KVQ_E_ARG
        assert lib.kvq_append(h, None, fake, 5, None) == kvq.KVQ_E_ARG
        assert lib.kvq_append(h, fake, fake, 1001, None) == kvq.KVQ_E_CAPACITY
        assert lib.kvq_num_tokens(h) == 0
        assert lib.kvq_decode_attn(h, fake, fake, fake, 1 << 30, None) == kvq.KVQ_E_STATE  # empty cache
        assert b"empty" in lib.kvq_last_error()
        assert lib.kvq_reset(h) == kvq.KVQ_OK
    finally:
        assert lib.kvq_destroy(h) == kvq.KVQ_OK
    assert lib.kvq_destroy(None) == kvq.KVQ_OK
    # key norms exist only with token_norm
    h2 = ctypes.c_void_p()
    assert lib.kvq_create(ctypes.byref(cc), fake, need, ctypes.byref(h2)) == kvq.KVQ_OK
    assert lib.kvq_export_key_norms(h2, 0, 1, fake, None) == kvq.KVQ_E_STATE
    assert lib.kvq_import_key_norms(h2, 0, 1, fake, None) == kvq.KVQ_E_STATE
    assert lib.kvq_export_key_norms(h2, 0, 1, None, None) == kvq.KVQ_E_ARG
    assert lib.kvq_destroy(h2) == kvq.KVQ_OK
    # merge: argument checks before any launch
    assert lib.kvq_merge_partials(fake, fake, 4, 257, 128, None) == kvq.KVQ_E_ARG
    assert lib.kvq_merge_partials(fake, fake, 4, 0, 128, None) == kvq.KVQ_E_ARG
    assert lib.kvq_merge_partials(fake + 4, fake, 4, 8, 128, None) == kvq.KVQ_E_ARG
    assert lib.kvq_merge_partials(fake, fake, 4, 8, 96, None) == kvq.KVQ_E_UNSUPPORTED
    cc.struct_size = 4
    assert lib.kvq_create(ctypes.byref(cc), fake, need, ctypes.byref(h)) == kvq.KVQ_E_ARG


def test_workspace_bounds_split_request():
    import decode_attention_asym_amd as kvq

    for w in ("tiny", "big"):
        c = _cfg(batch=1 if w == "tiny" else 64, num_kv_heads=8, num_q_heads=32)
        ws = kvq.workspace_bytes(c)
        assert ws > 0 and ws % 16 == 0


def test_token_norm_adds_two_bytes_per_quantized_token():
    import decode_attention_asym_amd as kvq

    for G, R, D in ((64, 128, 128), (32, 32, 64)):
        a = kvq.cache_bytes(_cfg(group_size=G, residual=R, head_dim=D, max_tokens=10000))
        b = kvq.cache_bytes(_cfg(group_size=G, residual=R, head_dim=D, max_tokens=10000, token_norm=True))
        slices = 2 * 2
        pages = (10000 - R) // G
        assert abs((b - a) - slices * pages * G * 2) <= 256


@pytest.mark.parametrize("bad", [
    dict(adapt_delta=32),  # not a multiple of G = 64
    dict(adapt_delta=-64),
    dict(adapt_delta=128, bits_low=(3, 2), bits_high=(4, 4)),
    dict(adapt_delta=128, bits_low=(2, 2), bits_high=(4, 8)),
    dict(adapt_delta=128),  # widths left at 0
])
def test_invalid_adaptive_configs_rejected(bad):
    import decode_attention_asym_amd as kvq

    assert kvq.cache_bytes(_cfg(**bad)) == 0
    assert kvq.lib.kvq_last_error()


def test_adaptive_group_slots_hold_the_widest_page():
    """Every group slot of a position-adaptive cache is as large as the widest
    of the three (key, value) bit pairs' pages; the fp16 parts do not change."""
    import decode_attention_asym_amd as kvq

    n, G, R = 10000, 64, 128
    base = dict(max_tokens=n, group_size=G, residual=R, k_bits=2, v_bits=2)
    pages = (n - R) // G
    slices = 2 * 2
    plain = {(kb, vb): kvq.cache_bytes(_cfg(**{**base, "k_bits": kb, "v_bits": vb})) for kb in (2, 4) for vb in (2, 4)}
    a = kvq.cache_bytes(_cfg(**base, adapt_delta=512, bits_low=(2, 2), bits_high=(4, 4)))
    assert a == plain[(4, 4)]
    b = kvq.cache_bytes(_cfg(**base, adapt_delta=512, bits_low=(2, 4), bits_high=(2, 2)))
    assert b == plain[(2, 4)]
    # the widest page per slot: K4V4 pages are (4 + 4) * D / 8 * G bytes of codes larger than K2V2 by 2x
    assert (plain[(4, 4)] - plain[(2, 2)]) == pytest.approx(slices * pages * G * 128 * 4 / 8, abs=512)


def test_group_bits_on_a_fresh_handle():
    import decode_attention_asym_amd as kvq
    from decode_attention_asym_amd.kvq import lib

    c = _cfg(adapt_delta=128, bits_low=(2, 2), bits_high=(4, 4))
    cc = c.c()
    h = ctypes.c_void_p()
    assert lib.kvq_create(ctypes.byref(cc), 1 << 40, kvq.cache_bytes(c), ctypes.byref(h)) == kvq.KVQ_OK
    try:
        assert lib.kvq_group_bits(h, None, None, 0) == 0
        assert lib.kvq_export_codes_u8(h, 0, 1, None, None, None) == kvq.KVQ_E_ARG
        assert lib.kvq_export_codes_u8(h, 0, 3, 1 << 40, None, None) == kvq.KVQ_E_ARG  # batch range
    finally:
        lib.kvq_destroy(h)
    assert lib.kvq_group_bits(None, None, None, 0) == -1


def test_drift_entry_points_validate_on_the_host():
    import decode_attention_asym_amd as kvq
    from decode_attention_asym_amd.kvq import lib

    c = _cfg()
    cc = c.c()
    fake = 1 << 40
    h = ctypes.c_void_p()
    assert lib.kvq_create(ctypes.byref(cc), fake, kvq.cache_bytes(c), ctypes.byref(h)) == kvq.KVQ_OK
    try:
        # an empty cache has no quantized groups: any non-empty range is out of bounds
        assert lib.kvq_code_histograms(h, 0, 1, fake, fake, None) == kvq.KVQ_E_ARG
        assert lib.kvq_drift_check(h, 0, 1, fake, fake, 0.1, fake, fake, fake, None) == kvq.KVQ_E_ARG
        assert lib.kvq_requantize(h, 0, 1, fake, fake, None, None) == kvq.KVQ_E_ARG
        assert lib.kvq_requantize(h, 0, 0, None, None, None, None) == kvq.KVQ_OK  # empty range: no-op
        assert lib.kvq_drift_check(h, 0, 0, None, fake, 0.1, fake, fake, fake, None) == kvq.KVQ_E_ARG
        assert lib.kvq_drift_check(h, 0, 0, fake, fake, -1.0, fake, fake, fake, None) == kvq.KVQ_E_ARG
    finally:
        lib.kvq_destroy(h)
    ca = _cfg(adapt_delta=128, bits_low=(2, 2), bits_high=(4, 4)).c()
    assert lib.kvq_create(ctypes.byref(ca), fake, kvq.cache_bytes(_cfg(adapt_delta=128, bits_low=(2, 2),
                                                                        bits_high=(4, 4))), ctypes.byref(h)) == 0
    try:
        assert lib.kvq_code_histograms(h, 0, 0, fake, fake, None) == kvq.KVQ_E_UNSUPPORTED
    finally:
        lib.kvq_destroy(h)
