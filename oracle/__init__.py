"""Python wrapper around the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the oracle is the slow, obviously-correct CPU
reference that the HIP library is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg import this package.  It imports
nothing from the product package and shares no code with it.

Every function here is argument marshalling around one C routine; the
arithmetic lives in oracle.c, whose header cites the page passages each step
follows.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b

            _b.build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(L):
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f16_to_f32.restype = ctypes.c_float
    L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    for name in ("orc_f32_to_f16_n", "orc_f16_to_f32_n", "orc_bf16_to_f32_n", "orc_f32_to_bf16_n"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [P, P, i64]
    L.orc_fwht_f32.restype = None
    L.orc_fwht_f32.argtypes = [P, i32]
    L.orc_rotate_f64.restype = None
    L.orc_rotate_f64.argtypes = [P, P, i32]
    L.orc_quantize_group.restype = None
    L.orc_quantize_group.argtypes = [P, i32, i32, P, P, P, P, P]
    L.orc_quantize_group_sym.restype = None
    L.orc_quantize_group_sym.argtypes = [P, i32, i32, P, P, P, P]
    L.orc_group_max_error.restype = ctypes.c_float
    L.orc_group_max_error.argtypes = [P, P, i32, ctypes.c_uint16, ctypes.c_uint16]
    L.orc_quantize_group_hybrid.restype = i32
    L.orc_quantize_group_hybrid.argtypes = [P, i32, i32, P, P, P]
    L.orc_num_quantized.restype = i64
    L.orc_num_quantized.argtypes = [i64, i32, i32]
    L.orc_num_quantized_sink.restype = i64
    L.orc_num_quantized_sink.argtypes = [i64, i32, i32, i32]
    L.orc_encode_slice.restype = i64
    L.orc_encode_slice.argtypes = [P, P, i32, i64, i32, i32, i32, i32, i32, i32] + [P] * 8
    L.orc_encode_slice_ext.restype = i64
    L.orc_encode_slice_ext.argtypes = [P, P, i32, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32] + [P] * 13
    L.orc_adaptive_group_bits.restype = i64
    L.orc_adaptive_group_bits.argtypes = [i32, i32, i32, i32, i32, P] + [i32] * 6 + [P, P]
    L.orc_row_norm_f32.restype = ctypes.c_float
    L.orc_row_norm_f32.argtypes = [P, i32]
    L.orc_pack_codes.restype = None
    L.orc_pack_codes.argtypes = [P, i64, i32, i32, P]
    L.orc_unpack_codes.restype = None
    L.orc_unpack_codes.argtypes = [P, i64, i32, i32, P]
    L.orc_attend_partial.restype = None
    L.orc_attend_partial.argtypes = [P, i32, i64, i64, i32, i32] + [P] * 9 + [i64, i64, P, P, P]
    L.orc_attend_slice.restype = None
    L.orc_attend_slice.argtypes = [P, i32, i64, i64, i32, i32] + [P] * 9 + [P]
    L.orc_merge_partials.restype = None
    L.orc_merge_partials.argtypes = [i32, i32, i32, P, P, P, P]
    L.orc_bits_per_element.restype = f64
    L.orc_bits_per_element.argtypes = [i64, i32, i32, i32, i32, f64]
    L.orc_bits_per_element_sink.restype = f64
    L.orc_bits_per_element_sink.argtypes = [i64, i32, i32, i32, i32, i32, f64]
    L.orc_code_histogram.restype = i32
    L.orc_code_histogram.argtypes = [P, i64, i32, P]
    L.orc_kl_divergence.restype = f64
    L.orc_kl_divergence.argtypes = [P, P, i32]
    L.orc_drift_check.restype = i32
    L.orc_drift_check.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, f64, P, P, P]
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- conversions
def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(out), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_n(_p(h), _p(out), h.size)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_f32_n(_p(b), _p(out), b.size)
    return out


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_p(x), _p(out), x.size)
    return out


def input_to_f64(a, dtype: str) -> np.ndarray:
    """Widen stored input elements (f32 values, or f16/bf16 bit patterns) to fp64 exactly."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return f16_bits_to_f32(a).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


# ---------------------------------------------------------------- rotation
def fwht_f32(y) -> np.ndarray:
    y = np.array(y, dtype=np.float32, copy=True, order="C")
    lib().orc_fwht_f32(_p(y), y.size)
    return y


def rotate_f64(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    out = np.empty_like(q)
    lib().orc_rotate_f64(_p(q), _p(out), q.size)
    return out


# ---------------------------------------------------------------- quantizer
def quantize_group(x, bits: int):
    """Quantize one group of fp16-valued binary32 numbers.

    Returns (codes uint16[count], s_f32, mn_f32, scale16_bits, zero16_bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, np.uint16)
    s = np.zeros(1, np.float32)
    mn = np.zeros(1, np.float32)
    sc = np.zeros(1, np.uint16)
    zr = np.zeros(1, np.uint16)
    lib().orc_quantize_group(_p(x), x.size, bits, _p(codes), _p(s), _p(mn), _p(sc), _p(zr))
    return codes, np.float32(s[0]), np.float32(mn[0]), int(sc[0]), int(zr[0])


def quantize_group_sym(x, bits: int):
    """Symmetric quantizer of one group: (codes, s_f32, scale16_bits, zero16_bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, np.uint16)
    s = np.zeros(1, np.float32)
    sc = np.zeros(1, np.uint16)
    zr = np.zeros(1, np.uint16)
    lib().orc_quantize_group_sym(_p(x), x.size, bits, _p(codes), _p(s), _p(sc), _p(zr))
    return codes, np.float32(s[0]), int(sc[0]), int(zr[0])


def group_max_error(x, codes, scale16: int, zero16: int) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    return float(lib().orc_group_max_error(_p(x), _p(codes), x.size, scale16, zero16))


def quantize_group_hybrid(x, bits: int):
    """Hybrid quantizer of one group: (codes, scale16_bits, zero16_bits, symmetric_kept)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, np.uint16)
    sc = np.zeros(1, np.uint16)
    zr = np.zeros(1, np.uint16)
    sym = lib().orc_quantize_group_hybrid(_p(x), x.size, bits, _p(codes), _p(sc), _p(zr))
    return codes, int(sc[0]), int(zr[0]), bool(sym)


def num_quantized(n: int, G: int, R: int, sink: int = 0) -> int:
    return int(lib().orc_num_quantized_sink(n, G, R, sink))


def row_norm_f32(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return float(lib().orc_row_norm_f32(_p(x), x.size))


def adaptive_group_bits(G: int, R: int, sink: int, delta: int, calls, low, mid, high):
    """Per-group (key bits, value bits) of a position-adaptive slice built by
    appends of `calls` tokens; low/mid/high are (key, value) bit pairs."""
    calls = np.ascontiguousarray(calls, dtype=np.int64)
    n = int(calls.sum())
    cap = max(1, n // G + 1)
    kb = np.zeros(cap, np.uint8)
    vb = np.zeros(cap, np.uint8)
    ng = lib().orc_adaptive_group_bits(G, R, sink, delta, calls.size, _p(calls), low[0], low[1], mid[0], mid[1],
                                       high[0], high[1], _p(kb), _p(vb))
    if ng < 0:
        raise ValueError("orc_adaptive_group_bits rejected its arguments")
    return kb[:ng].copy(), vb[:ng].copy()


def code_histogram(codes, bits: int) -> np.ndarray:
    """Counts of each code value in [0, 2^bits) (int64)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint16).reshape(-1)
    hist = np.zeros(1 << bits, np.int64)
    if lib().orc_code_histogram(_p(codes), codes.size, bits, _p(hist)) < 0:
        raise ValueError("code out of range")
    return hist


def kl_divergence(p, q) -> float:
    """D_KL(p || q), natural log, 0 log 0 = 0, +inf where q has no mass."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    assert p.shape == q.shape
    return float(lib().orc_kl_divergence(_p(p), _p(q), p.size))


def drift_check(k_codes, v_codes, G: int, D: int, kbits: int, vbits: int, cal_k, cal_v, thr: float = 0.1):
    """Per-group KL of the key and value code histograms of one slice's
    canonical codes against calibration counts; returns (kl_k, kl_v, flags)."""
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint16)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint16)
    ng = k_codes.size // (G * D)
    cal_k = np.ascontiguousarray(cal_k, dtype=np.int64)
    cal_v = np.ascontiguousarray(cal_v, dtype=np.int64)
    kl_k, kl_v = np.zeros(max(ng, 1)), np.zeros(max(ng, 1))
    flags = np.zeros(max(ng, 1), np.uint8)
    if lib().orc_drift_check(_p(k_codes), _p(v_codes), ng, G, D, kbits, vbits, _p(cal_k), _p(cal_v), thr,
                             _p(kl_k), _p(kl_v), _p(flags)) < 0:
        raise ValueError("orc_drift_check rejected its arguments")
    return kl_k[:ng], kl_v[:ng], flags[:ng]


def encode_slice(k, v, dtype: str, D: int, kbits: int, vbits: int, G: int, R: int, rotate: bool,
                 sink: int = 0, hybrid: bool = False, token_norm: bool = False, group_bits=None):
    """Encode one (batch, kv-head) slice.  k, v: [n][D] in the input dtype
    (float32 values for "f32", uint16 bit patterns for "f16"/"bf16").

    Returns a dict of canonical arrays (codes unpacked, one per uint16); the
    fp16 tokens (an attention-sink window of `sink` tokens, then the recent
    window) are k_resid / v_resid; k_sym / v_sym mark symmetric groups;
    k_norm (fp16 bits, one per quantized token) is present with token_norm.
    group_bits = (key bits, value bits) arrays give per-group widths."""
    np_dt = np.float32 if dtype == "f32" else np.uint16
    k = np.ascontiguousarray(k, dtype=np_dt).reshape(-1, D)
    v = np.ascontiguousarray(v, dtype=np_dt).reshape(-1, D)
    n = k.shape[0]
    nq = num_quantized(n, G, R, sink)
    nr = n - nq
    out = {
        "k_codes": np.zeros((nq, D), np.uint16),
        "k_scale": np.zeros((nq // G, D), np.uint16),
        "k_zero": np.zeros((nq // G, D), np.uint16),
        "v_codes": np.zeros((nq, D), np.uint16),
        "v_scale": np.zeros((nq, D // G), np.uint16),
        "v_zero": np.zeros((nq, D // G), np.uint16),
        "k_resid": np.zeros((nr, D), np.uint16),
        "v_resid": np.zeros((nr, D), np.uint16),
        "k_sym": np.zeros((nq // G, D), np.uint8),
        "v_sym": np.zeros((nq, D // G), np.uint8),
    }
    k_norm = np.zeros(max(nq, 1), np.uint16)
    gkb = gvb = None
    if group_bits is not None:
        gkb = np.ascontiguousarray(group_bits[0], dtype=np.uint8)
        gvb = np.ascontiguousarray(group_bits[1], dtype=np.uint8)
        assert gkb.size >= nq // G and gvb.size >= nq // G
    r = lib().orc_encode_slice_ext(
        _p(k), _p(v), DTYPE_CODE[dtype], n, D, kbits, vbits, G, R, int(bool(rotate)), int(sink), int(bool(hybrid)),
        int(bool(token_norm)),
        *(_p(out[key]) for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid",
                                   "k_sym", "v_sym")),
        _p(k_norm), None if gkb is None else _p(gkb), None if gvb is None else _p(gvb),
    )
    if token_norm:
        out["k_norm"] = k_norm[:nq].copy()
    if r < 0:
        raise ValueError("orc_encode_slice rejected its arguments")
    out["nq"] = nq
    out["n"] = n
    return out


def pack_codes(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    rows, D = codes.shape
    out = np.zeros((rows, (D * bits + 7) // 8), np.uint8)
    lib().orc_pack_codes(_p(codes), rows, D, bits, _p(out))
    return out


def unpack_codes(packed, D: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.zeros((rows, D), np.uint16)
    lib().orc_unpack_codes(_p(packed), rows, D, bits, _p(out))
    return out


# ---------------------------------------------------------------- attention
_CACHE_KEYS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid")


def _cache_ptrs(cache):
    """Pointers to the canonical arrays, then to k_norm (NULL without token norms)."""
    arrs = [np.ascontiguousarray(cache[k], dtype=np.uint16) for k in _CACHE_KEYS]
    ptrs = [_p(a) for a in arrs]
    if cache.get("k_norm") is not None:
        kn = np.ascontiguousarray(cache["k_norm"], dtype=np.uint16)
        arrs.append(kn)
        ptrs.append(_p(kn))
    else:
        ptrs.append(None)
    return arrs, ptrs


def attend_slice(q, cache, D: int, G: int, R: int | None = None) -> np.ndarray:
    """fp64 attention of q[nh][D] (fp64, rotated already if keys were) over a
    canonical slice (its quantized token count is cache["nq"]; R is implied)."""
    q = np.ascontiguousarray(q, dtype=np.float64).reshape(-1, D)
    nh = q.shape[0]
    out = np.zeros((nh, D), np.float64)
    keep, ptrs = _cache_ptrs(cache)
    lib().orc_attend_slice(_p(q), nh, int(cache["n"]), int(cache["nq"]), D, G, *ptrs, _p(out))
    del keep
    return out


def attend_partial(q, cache, D: int, G: int, R: int | None, t0: int, t1: int):
    """Partial statistics over canonical token indices [t0, t1): the quantized
    tokens first (cache["nq"] of them), then the fp16 tokens."""
    q = np.ascontiguousarray(q, dtype=np.float64).reshape(-1, D)
    nh = q.shape[0]
    m = np.zeros(nh, np.float64)
    l = np.zeros(nh, np.float64)
    o = np.zeros((nh, D), np.float64)
    keep, ptrs = _cache_ptrs(cache)
    lib().orc_attend_partial(_p(q), nh, int(cache["n"]), int(cache["nq"]), D, G, *ptrs, t0, t1, _p(m), _p(l), _p(o))
    del keep
    return m, l, o


def merge_partials(m, l, o) -> np.ndarray:
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    S, nh, D = o.shape
    out = np.zeros((nh, D), np.float64)
    lib().orc_merge_partials(S, nh, D, _p(m), _p(l), _p(o), _p(out))
    return out


def attend_slices_parallel(jobs, threads: int):
    """Run attend_slice over many (q, cache, D, G, R) jobs on `threads` host
    threads (ctypes releases the GIL during each C call)."""
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda j: attend_slice(*j), jobs))


# ---------------------------------------------------------------- accounting
def bits_per_element(n: int, kbits: int, vbits: int, G: int, R: int, overhead_bits: float = 32.0,
                     sink: int = 0) -> float:
    return float(lib().orc_bits_per_element_sink(n, kbits, vbits, G, R, sink, overhead_bits))


def kv_cache_bytes(layers: int, hidden: int, tokens: int, bits_per_elem: float) -> float:
    """K and V of `layers` layers with `hidden` channels each, `tokens` tokens,
    at `bits_per_elem` bits per stored element (section 5.4 memory model of
    "Asymmetric Key-Value Quantization ...")."""
    return 2.0 * layers * hidden * tokens * bits_per_elem / 8.0
