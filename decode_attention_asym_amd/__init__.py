"""MI355X-native asymmetric low-bit KV-cache quantization fused into decode attention.

The compute path is libkvq.so (hand-written HIP kernels for gfx950 behind the
C ABI in include/kvq.h); this package is the ctypes binding over it.
"""
from .kvq import (  # noqa: F401
    Config,
    DecodePlan,
    KVQCache,
    KVQError,
    cache_bytes,
    check,
    lib,
    merge_partials,
    workspace_bytes,
    KVQ_OK,
    KVQ_E_ARG,
    KVQ_E_UNSUPPORTED,
    KVQ_E_CAPACITY,
    KVQ_E_DEVICE,
    KVQ_E_STATE,
)


def config_for(w, max_tokens: int | None = None) -> "Config":
    """Library config for a synthetic workload description (synth.Workload)."""
    return Config(
        batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
        max_tokens=max_tokens or w.N, k_bits=w.kbits, v_bits=w.vbits, group_size=w.G,
        residual=w.R, rotate=w.rotate, in_dtype=w.dtype, sink_tokens=getattr(w, "sink", 0),
        hybrid=getattr(w, "hybrid", False), token_norm=getattr(w, "token_norm", False),
        adapt_delta=getattr(w, "adapt_delta", 0), bits_low=tuple(getattr(w, "bits_low", (0, 0))),
        bits_high=tuple(getattr(w, "bits_high", (0, 0))),
    )
