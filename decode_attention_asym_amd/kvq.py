"""Thin ctypes binding of libkvq.so (include/kvq.h): argument marshalling only.

Every step of the quantize-append and decode-attention path runs in the HIP
kernels behind the C ABI; PyTorch provides device memory and streams.  If the
library is not built this module raises on import -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import NamedTuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK, KVQ_E_ARG, KVQ_E_UNSUPPORTED, KVQ_E_CAPACITY, KVQ_E_DEVICE, KVQ_E_STATE = range(6)
STATUS_NAMES = ["KVQ_OK", "KVQ_E_ARG", "KVQ_E_UNSUPPORTED", "KVQ_E_CAPACITY", "KVQ_E_DEVICE", "KVQ_E_STATE"]
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}

# entry points declared in include/kvq.h, with (restype, argtypes)
_P, _SZ, _I32, _I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64


class kvq_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("k_bits", ctypes.c_int32),
        ("v_bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32),
        ("hybrid", ctypes.c_int32),
        ("token_norm", ctypes.c_int32),
        ("adapt_delta", ctypes.c_int32),
        ("k_bits_low", ctypes.c_int32),
        ("v_bits_low", ctypes.c_int32),
        ("k_bits_high", ctypes.c_int32),
        ("v_bits_high", ctypes.c_int32),
    ]


_CFG_P = ctypes.POINTER(kvq_config)
SIGNATURES = {
    "kvq_cache_bytes": (_SZ, [_CFG_P]),
    "kvq_workspace_bytes": (_SZ, [_CFG_P]),
    "kvq_create": (ctypes.c_int, [_CFG_P, _P, _SZ, ctypes.POINTER(_P)]),
    "kvq_append": (ctypes.c_int, [_P, _P, _P, _I32, _P]),
    "kvq_decode_attn": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P]),
    "kvq_decode_attn_splits": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _I32, _P]),
    "kvq_decode_attn_noalloc": (ctypes.c_int, [_P, _P, _P, _P]),
    "kvq_default_splits": (_I32, [_P]),
    "kvq_decode_partials": (ctypes.c_int, [_P, _P, _P, _SZ, _I32, ctypes.POINTER(_I32), _P]),
    "kvq_decode_plan": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "kvq_merge_partials": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P]),
    "kvq_num_tokens": (_I64, [_P]),
    "kvq_num_quantized": (_I64, [_P]),
    "kvq_reset": (ctypes.c_int, [_P]),
    "kvq_destroy": (ctypes.c_int, [_P]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_export": (ctypes.c_int, [_P, _I32, _I32] + [_P] * 8 + [_P]),
    "kvq_import": (ctypes.c_int, [_P, _I64, _I32, _I32] + [_P] * 8 + [_P]),
    "kvq_export_key_norms": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "kvq_import_key_norms": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "kvq_export_codes_u8": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "kvq_group_bits": (_I64, [_P, _P, _P, _I64]),
    "kvq_append_decode_attn": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _SZ, _P]),
    "kvq_append_decode_partials": (ctypes.c_int, [_P, _P, _P, _P, _P, _SZ, _I32, ctypes.POINTER(_I32), _P]),
    "kvq_code_histograms": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "kvq_drift_check": (ctypes.c_int, [_P, _I64, _I64, _P, _P, ctypes.c_double, _P, _P, _P, _P]),
    "kvq_requantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python decode_attention_asym_amd/build.py). There is no CPU fallback."
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.kvq_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES[status] if 0 <= status < 6 else status}: {msg}")


def check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KVQError(status, where)


@dataclass
class Config:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_tokens: int
    k_bits: int
    v_bits: int
    group_size: int
    residual: int
    rotate: bool = False
    in_dtype: str = "bf16"
    sink_tokens: int = 0
    hybrid: bool = False
    token_norm: bool = False
    adapt_delta: int = 0
    bits_low: tuple = (0, 0)   # (key, value) bits of early groups when adapt_delta > 0
    bits_high: tuple = (0, 0)  # (key, value) bits of recent groups when adapt_delta > 0

    def c(self) -> kvq_config:
        return kvq_config(
            ctypes.sizeof(kvq_config), self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
            self.max_tokens, self.k_bits, self.v_bits, self.group_size, self.residual, int(bool(self.rotate)),
            DTYPES[self.in_dtype], self.sink_tokens, int(bool(self.hybrid)), int(bool(self.token_norm)),
            self.adapt_delta, self.bits_low[0], self.bits_low[1], self.bits_high[0], self.bits_high[1],
        )


def cache_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(lib.kvq_cache_bytes(ctypes.byref(c)))


def workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(lib.kvq_workspace_bytes(ctypes.byref(c)))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch

        return int(torch.cuda.current_stream().cuda_stream)
    return int(stream)


_TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def _require(t, name: str, device, dtype, shape=None, min_numel: int | None = None):
    """Raise ValueError unless t is a contiguous torch tensor on `device` with
    `dtype` and exactly `shape` (or at least `min_numel` elements).  The C ABI
    takes bare pointers, so a tensor on another device, of another dtype, a
    strided view or a short buffer would be read or written out of bounds."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")
    want = dtype if isinstance(dtype, torch.dtype) else getattr(torch, dtype)
    if t.dtype != want:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous (strides {tuple(t.stride())} for shape {tuple(t.shape)})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")


def merge_partials(partials, out, rows: int, splits: int, head_dim: int, stream=None):
    """out [rows, head_dim] float32 from split partials [rows, splits, head_dim + 4]
    float32 (both contiguous, on one device)."""
    if rows < 1 or splits < 1:
        raise ValueError("rows and splits must be positive")
    dev = getattr(partials, "device", None)
    if dev is None or dev.type != "cuda":
        raise ValueError(f"partials: expected a GPU tensor, got {dev}")
    _require(partials, "partials", dev, "float32", min_numel=rows * splits * (head_dim + 4))
    _require(out, "out", partials.device, "float32", min_numel=rows * head_dim)
    check(lib.kvq_merge_partials(_ptr(partials), _ptr(out), rows, splits, head_dim, _stream(stream)),
          "kvq_merge_partials")
    return out


class DecodePlan(NamedTuple):
    """How a decode runs (kvq_decode_plan)."""

    splits: int  # splits per slice
    merged: bool  # the decode kernel writes the output itself
    records: int  # partial records per row the merge kernel combines (0 when merged)


class KVQCache:
    """A quantized KV cache in a torch-allocated device buffer.

    append(k, v): k, v [B, H_kv, T, D] contiguous tensors of the config dtype.
    decode(q, out=None): q [B, H_q, D]; returns out [B, H_q, D] float32.
    """

    def __init__(self, cfg: Config, device="cuda"):
        import torch

        self.cfg = cfg
        if torch.device(device).type != "cuda":
            raise ValueError(f"the cache lives in GPU memory; device {device!r} is not a GPU")
        nbytes = cache_bytes(cfg)
        if nbytes == 0:
            raise KVQError(KVQ_E_UNSUPPORTED if lib.kvq_last_error() else KVQ_E_ARG, "kvq_cache_bytes")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(workspace_bytes(cfg), 16), dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        c = cfg.c()
        check(lib.kvq_create(ctypes.byref(c), self.buf.data_ptr(), nbytes, ctypes.byref(h)), "kvq_create")
        self.h = h
        self.device = self.buf.device

    # ---- argument checks (before any call into the library)
    def _in(self, t, name, shape):
        _require(t, name, self.device, _TORCH_DTYPES[self.cfg.in_dtype], shape)

    def _out(self, out, q):
        import torch

        c = self.cfg
        if out is None:
            return torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device=self.device)
        _require(out, "out", self.device, "float32", (c.batch, c.num_q_heads, c.head_dim))
        return out

    def _q(self, q):
        c = self.cfg
        self._in(q, "q", (c.batch, c.num_q_heads, c.head_dim))

    def _kv(self, k, v, T=None):
        c = self.cfg
        if T is None:
            T = k.shape[2] if hasattr(k, "shape") and len(k.shape) == 4 else -1
        shape = (c.batch, c.num_kv_heads, T, c.head_dim)
        self._in(k, "k", shape)
        self._in(v, "v", shape)
        return T

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            lib.kvq_destroy(h)
            self.h = None

    @property
    def num_tokens(self) -> int:
        return int(lib.kvq_num_tokens(self.h))

    @property
    def num_quantized(self) -> int:
        return int(lib.kvq_num_quantized(self.h))

    def default_splits(self) -> int:
        return int(lib.kvq_default_splits(self.h))

    def decode_plan(self, splits: int | None = None) -> DecodePlan:
        """(split count, merged inside the decode kernel, partial records per
        row the merge kernel combines) of decode(q, splits=splits) on the
        current tokens; nothing is launched."""
        S_req = self.default_splits() if splits is None else splits
        used, records = ctypes.c_int32(0), ctypes.c_int32(0)
        check(lib.kvq_decode_plan(self.h, S_req, ctypes.byref(used), ctypes.byref(records)), "kvq_decode_plan")
        return DecodePlan(int(used.value), records.value == 0, int(records.value))

    def append(self, k, v, stream=None) -> None:
        """k, v: [B, H_kv, T, D] contiguous, the config dtype, on the cache's device."""
        T = self._kv(k, v)
        check(lib.kvq_append(self.h, _ptr(k), _ptr(v), T, _stream(stream)), "kvq_append")

    def decode(self, q, out=None, splits: int | None = None, stream=None):
        self._q(q)
        out = self._out(out, q)
        if splits is None:
            st = lib.kvq_decode_attn(self.h, _ptr(q), _ptr(out), _ptr(self.ws), self.ws.numel(), _stream(stream))
        else:
            st = lib.kvq_decode_attn_splits(self.h, _ptr(q), _ptr(out), _ptr(self.ws), self.ws.numel(), splits,
                                            _stream(stream))
        check(st, "kvq_decode_attn")
        return out

    def decode_noalloc(self, q, out=None, stream=None):
        """decode(q) with the split partials in the library's per-device
        scratch array instead of this cache's workspace (no device memory is
        allocated by the call when `out` is given)."""
        self._q(q)
        out = self._out(out, q)
        check(lib.kvq_decode_attn_noalloc(self.h, _ptr(q), _ptr(out), _stream(stream)), "kvq_decode_attn_noalloc")
        return out

    def append_decode(self, k, v, q, out=None, stream=None):
        """One step: append one token (k, v [B, H_kv, 1, D]) and decode q,
        every argument checked before anything is enqueued.  The decode kernel
        may read k and v itself (it writes the token's window slots), so they
        must stay unchanged until the work enqueued on the stream is done."""
        self._kv(k, v, 1)
        self._q(q)
        out = self._out(out, q)
        check(lib.kvq_append_decode_attn(self.h, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(self.ws), self.ws.numel(),
                                         _stream(stream)), "kvq_append_decode_attn")
        return out

    def append_decode_partials(self, k, v, q, partials=None, splits: int | None = None, stream=None):
        """As append_decode, stopping at the split partials; returns (partials, S)."""
        import torch

        rows, W = self.cfg.batch * self.cfg.num_q_heads, self.cfg.head_dim + 4
        self._kv(k, v, 1)
        self._q(q)
        if partials is None:
            partials = torch.empty(self.ws.numel() // 4, dtype=torch.float32, device=self.device)
        else:
            _require(partials, "partials", self.device, "float32")
        S_req = splits if splits is not None else int(lib.kvq_default_splits(self.h))
        used = ctypes.c_int32(0)
        check(lib.kvq_append_decode_partials(self.h, _ptr(k), _ptr(v), _ptr(q), _ptr(partials), partials.numel() * 4,
                                             S_req, ctypes.byref(used), _stream(stream)), "kvq_append_decode_partials")
        S = int(used.value)
        return partials.reshape(-1)[: rows * S * W].view(rows, S, W), S

    def decode_partials(self, q, partials=None, splits: int | None = None, stream=None):
        """Split partials [B*H_q, S, D+4] (o unnormalized, m, l in base 2); returns (partials, S)."""
        import torch

        self._q(q)
        S_req = self.default_splits() if splits is None else splits
        rows, W = self.cfg.batch * self.cfg.num_q_heads, self.cfg.head_dim + 4
        if partials is not None:
            _require(partials, "partials", self.device, "float32")
        else:
            # a position-adaptive cache may use a few more splits than asked
            # (one per run of equal bit widths at least)
            cap = max(S_req, self.ws.numel() // (rows * W * 4))
            partials = torch.empty((rows, cap, W), dtype=torch.float32, device=self.device)
        used = ctypes.c_int32(0)
        check(lib.kvq_decode_partials(self.h, _ptr(q), _ptr(partials), partials.numel() * 4, S_req,
                                      ctypes.byref(used), _stream(stream)), "kvq_decode_partials")
        S = int(used.value)
        if partials.dim() == 3 and partials.shape[1] != S:
            partials = partials.reshape(-1)[: rows * S * W].view(rows, S, W)
        return partials, S

    def num_groups(self) -> int:
        return self.num_quantized // self.cfg.group_size

    def code_histograms(self, g0: int = 0, g1: int | None = None, stream=None):
        """Calibration code counts over groups [g0, g1): (k_hist [H_kv, 2^k_bits],
        v_hist [H_kv, 2^v_bits]) int64 device tensors."""
        import torch

        c = self.cfg
        g1 = self.num_groups() if g1 is None else g1
        dev = self.device
        kh = torch.empty((c.num_kv_heads, 1 << c.k_bits), dtype=torch.int64, device=dev)
        vh = torch.empty((c.num_kv_heads, 1 << c.v_bits), dtype=torch.int64, device=dev)
        check(lib.kvq_code_histograms(self.h, g0, g1, _ptr(kh), _ptr(vh), _stream(stream)), "kvq_code_histograms")
        return kh, vh

    def drift_check(self, cal_k, cal_v, g0: int = 0, g1: int | None = None, threshold: float = 0.1, stream=None):
        """Per (slice, group) KL of the code histograms against calibration
        counts: (kl_k, kl_v float64, flags uint8), each [B * H_kv, g1 - g0]."""
        import torch

        c = self.cfg
        g1 = self.num_groups() if g1 is None else g1
        dev = self.device
        _require(cal_k, "cal_k", dev, "int64", (c.num_kv_heads, 1 << c.k_bits))
        _require(cal_v, "cal_v", dev, "int64", (c.num_kv_heads, 1 << c.v_bits))
        if g1 < g0:
            raise ValueError(f"group range [{g0}, {g1}) is empty or reversed")
        shape = (c.batch * c.num_kv_heads, g1 - g0)
        kl_k = torch.empty(shape, dtype=torch.float64, device=dev)
        kl_v = torch.empty(shape, dtype=torch.float64, device=dev)
        flags = torch.empty(shape, dtype=torch.uint8, device=dev)
        check(lib.kvq_drift_check(self.h, g0, g1, _ptr(cal_k), _ptr(cal_v), threshold, _ptr(kl_k), _ptr(kl_v),
                                  _ptr(flags), _stream(stream)), "kvq_drift_check")
        return kl_k, kl_v, flags

    def requantize(self, k, v, g0: int, g1: int, flags=None, stream=None) -> None:
        """Quantize groups [g0, g1) again from k, v [B, H_kv, (g1 - g0) * G, D]
        where flags (uint8 [B * H_kv, g1 - g0]) is nonzero (all if None)."""
        c = self.cfg
        if g1 < g0:
            raise ValueError(f"group range [{g0}, {g1}) is reversed")
        self._kv(k, v, (g1 - g0) * c.group_size)
        if flags is not None:
            _require(flags, "flags", self.device, "uint8", (c.batch * c.num_kv_heads, g1 - g0))
        check(lib.kvq_requantize(self.h, g0, g1, _ptr(k), _ptr(v), _ptr(flags), _stream(stream)), "kvq_requantize")

    def group_bits(self):
        """(key bits, value bits) uint8 arrays, one entry per quantized group."""
        import numpy as np

        ng = int(lib.kvq_group_bits(self.h, None, None, 0))
        kb, vb = np.zeros(max(ng, 1), np.uint8), np.zeros(max(ng, 1), np.uint8)
        lib.kvq_group_bits(self.h, kb.ctypes.data, vb.ctypes.data, ng)
        return kb[:ng], vb[:ng]

    def reset(self) -> None:
        check(lib.kvq_reset(self.h), "kvq_reset")

    def export(self, batch_begin: int = 0, batch_count: int | None = None, stream=None):
        """Canonical host arrays (numpy) for sequences [batch_begin, batch_begin + batch_count)."""
        import numpy as np

        c = self.cfg
        bc = c.batch - batch_begin if batch_count is None else batch_count
        nq, n = self.num_quantized, self.num_tokens
        nr, D, G, H = n - nq, c.head_dim, c.group_size, c.num_kv_heads
        adaptive = c.adapt_delta > 0
        out = {
            "k_codes": None if adaptive else np.zeros((bc, H, nq, D * c.k_bits // 8), np.uint8),
            "k_scale": np.zeros((bc, H, nq // G, D), np.uint16),
            "k_zero": np.zeros((bc, H, nq // G, D), np.uint16),
            "v_codes": None if adaptive else np.zeros((bc, H, nq, D * c.v_bits // 8), np.uint8),
            "v_scale": np.zeros((bc, H, nq, D // G), np.uint16),
            "v_zero": np.zeros((bc, H, nq, D // G), np.uint16),
            "k_resid": np.zeros((bc, H, nr, D), np.uint16),
            "v_resid": np.zeros((bc, H, nr, D), np.uint16),
        }
        keys = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid")
        check(lib.kvq_export(self.h, batch_begin, bc, *(None if out[k] is None else out[k].ctypes.data for k in keys),
                             _stream(stream)), "kvq_export")
        if adaptive:
            # codes of mixed widths: one per byte, with the groups' bit widths
            out["k_codes_u8"] = np.zeros((bc, H, nq, D), np.uint8)
            out["v_codes_u8"] = np.zeros((bc, H, nq, D), np.uint8)
            check(lib.kvq_export_codes_u8(self.h, batch_begin, bc, out["k_codes_u8"].ctypes.data,
                                          out["v_codes_u8"].ctypes.data, _stream(stream)), "kvq_export_codes_u8")
            out["k_gbits"], out["v_gbits"] = self.group_bits()
        if c.token_norm:
            out["k_norm"] = np.zeros((bc, H, nq), np.uint16)
            check(lib.kvq_export_key_norms(self.h, batch_begin, bc, out["k_norm"].ctypes.data, _stream(stream)),
                  "kvq_export_key_norms")
        out["nq"], out["n"] = nq, n
        return out

    def import_(self, arrays, n_tokens: int, batch_begin: int = 0, stream=None) -> None:
        import numpy as np

        keys = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid")
        arrs = [np.ascontiguousarray(arrays[k]) for k in keys]
        bc = arrs[0].shape[0]
        check(lib.kvq_import(self.h, n_tokens, batch_begin, bc, *(a.ctypes.data for a in arrs), _stream(stream)),
              "kvq_import")
        if self.cfg.token_norm:
            kn = np.ascontiguousarray(arrays["k_norm"], dtype=np.uint16)
            check(lib.kvq_import_key_norms(self.h, batch_begin, bc, kn.ctypes.data, _stream(stream)),
                  "kvq_import_key_norms")
