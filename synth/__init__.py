"""Seeded synthetic inputs for the five decode workloads.

This module only draws random numbers and shapes them; it holds none of the
quantization or attention arithmetic.  Both the HIP library's tests/bench and
the CPU oracle take their inputs from here.

Shapes follow the head layouts of the models the pages name (an 8B
Llama-3-shaped layer, a 70B-shaped layer, a 175B-shaped MHA layer); the value
distributions stand in for real activations, which the pages measure on
datasets and trained weights that are not available:

  tiny      fp32 N(0,1); keys scaled per (kv head, channel) by lognormal(0, 1),
            with 4 outlier channels per kv head scaled by a further x10
  lognormal bf16 N(0,1); keys scaled per (kv head, channel) by lognormal(0, 0.7)
  drift     bf16; std grows linearly from 1.0 (first position) to 2.0 (last
            prefilled position); key means follow a per-(kv head, channel)
            random walk over positions with N(0, 0.01^2) steps; K = mu + sigma z,
            V = sigma z
  queries   N(0,1) in the workload dtype

Per-(kv head, channel) parameters are model properties: shared across the
batch and drawn on the host with numpy, so they are identical on every device.
Bulk tensors are drawn with torch on the requested device from per-batch
generators, so any batch row can be regenerated independently.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    N: int           # prefilled tokens per sequence
    kbits: int
    vbits: int
    G: int
    R: int
    rotate: bool
    dtype: str       # "f32" | "bf16"
    dist: str        # "tiny" | "lognormal" | "drift"
    append_per_step: bool = False
    idx: int = 0
    sink: int = 0            # attention-sink tokens kept in fp16
    hybrid: bool = False     # per-group symmetric/asymmetric quantizer choice
    token_norm: bool = False  # key tokens divided by their norm before quantization
    adapt_delta: int = 0      # position-adaptive bit widths: region size Delta (0: off)
    bits_low: tuple = (0, 0)  # (key, value) bits of early groups
    bits_high: tuple = (0, 0)  # (key, value) bits of recent groups

    @property
    def gqa(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    def replace(self, **kw) -> "Workload":
        d = {f: getattr(self, f) for f in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


WORKLOADS = [
    Workload("tiny-2h-d64-512", 1, 2, 2, 64, 512, 2, 2, 32, 32, False, "f32", "tiny", idx=0),
    Workload("llama3-8b-layer-8k", 16, 32, 8, 128, 8192, 2, 2, 32, 128, False, "bf16", "lognormal", idx=1),
    Workload("llama3-8b-layer-32k-k4v2-drift", 64, 32, 8, 128, 32768, 4, 2, 64, 128, False, "bf16", "drift", idx=2),
    Workload("70b-layer-128k-append", 4, 64, 8, 128, 131072, 2, 2, 32, 32, False, "bf16", "lognormal", True, idx=3),
    Workload("175b-mha-16k-fwht", 32, 96, 96, 128, 16384, 2, 2, 32, 64, True, "bf16", "lognormal", idx=4),
]

# tensor ids used in seeds
_K, _V, _Q, _KSCALE, _OUTLIER, _WALK, _STEP_K, _STEP_V, _STEP_Q = range(9)
_SHARED = 65535


def _seed(w: Workload, tensor: int, b: int, extra: int = 0) -> int:
    ss = np.random.SeedSequence([w.idx, tensor, b, extra, w.N, w.D])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def key_channel_scale(w: Workload) -> np.ndarray:
    """[Hkv, D] fp32 per-channel key scales (ones for the drift workload)."""
    if w.dist == "drift":
        return np.ones((w.Hkv, w.D), np.float32)
    rng = np.random.default_rng(_seed(w, _KSCALE, _SHARED))
    sigma = 1.0 if w.dist == "tiny" else 0.7
    s = np.exp(rng.standard_normal((w.Hkv, w.D)) * sigma)
    if w.dist == "tiny":
        prng = np.random.default_rng(_seed(w, _OUTLIER, _SHARED))
        for h in range(w.Hkv):
            s[h, prng.choice(w.D, size=4, replace=False)] *= 10.0
    return s.astype(np.float32)


def drift_mean(w: Workload, positions: int) -> np.ndarray:
    """[Hkv, positions, D] fp32 key means: per-(head, channel) random walk, mu(0) = 0."""
    rng = np.random.default_rng(_seed(w, _WALK, _SHARED))
    steps = rng.standard_normal((w.Hkv, positions, w.D)) * 0.01
    steps[:, 0, :] = 0.0
    return np.cumsum(steps, axis=1).astype(np.float32)


def drift_sigma(w: Workload, pos: np.ndarray) -> np.ndarray:
    """Std at absolute positions: 1.0 at 0 rising linearly to 2.0 at N-1 (continuing beyond)."""
    return (1.0 + pos.astype(np.float64) / max(w.N - 1, 1)).astype(np.float32)


class Synth:
    """Input source for one workload on one device.  `positions` bounds the
    absolute positions that appended tokens may take (N + steps)."""

    def __init__(self, w: Workload, device="cpu", positions: int | None = None):
        self.w = w
        self.device = torch.device(device)
        self.positions = positions or w.N
        self.kscale = torch.from_numpy(key_channel_scale(w)).to(self.device)  # [Hkv, D]
        self._mu = None

    def _mu_t(self):
        if self._mu is None:
            self._mu = torch.from_numpy(drift_mean(self.w, self.positions)).to(self.device)
        return self._mu

    def _shape_kv(self, zk, zv, pos0: int):
        """zk, zv: fp32 [Hkv, T, D] standard normals at positions pos0.. -> K, V fp32."""
        w = self.w
        T = zk.shape[1]
        if w.dist == "drift":
            sig = torch.from_numpy(drift_sigma(w, np.arange(pos0, pos0 + T))).to(self.device)[None, :, None]
            k = self._mu_t()[:, pos0:pos0 + T, :] + sig * zk
            v = sig * zv
        else:
            k = zk * self.kscale[:, None, :]
            v = zv
        return k, v

    def kv(self, b: int):
        """Prefill K, V for batch row b: [Hkv, N, D] in the workload dtype."""
        w = self.w
        zk = torch.randn((w.Hkv, w.N, w.D), generator=_gen(self.device, _seed(w, _K, b)), device=self.device)
        zv = torch.randn((w.Hkv, w.N, w.D), generator=_gen(self.device, _seed(w, _V, b)), device=self.device)
        k, v = self._shape_kv(zk, zv, 0)
        return k.to(w.torch_dtype), v.to(w.torch_dtype)

    def kv_all(self):
        """[B, Hkv, N, D] K and V in the workload dtype."""
        w = self.w
        K = torch.empty((w.B, w.Hkv, w.N, w.D), dtype=w.torch_dtype, device=self.device)
        V = torch.empty_like(K)
        for b in range(w.B):
            K[b], V[b] = self.kv(b)
        return K, V

    def step_kv(self, step: int):
        """K, V of the token appended at decode step `step` (absolute position N + step): [B, Hkv, 1, D]."""
        w = self.w
        g = _gen(self.device, _seed(w, _STEP_K, _SHARED, step))
        zk = torch.randn((w.B, w.Hkv, 1, w.D), generator=g, device=self.device)
        zv = torch.randn((w.B, w.Hkv, 1, w.D), generator=g, device=self.device)
        ks, vs = [], []
        for b in range(w.B):
            k, v = self._shape_kv(zk[b], zv[b], w.N + step)
            ks.append(k)
            vs.append(v)
        return torch.stack(ks).to(w.torch_dtype), torch.stack(vs).to(w.torch_dtype)

    def q(self, step: int = 0):
        """Decode queries [B, Hq, D] in the workload dtype."""
        w = self.w
        g = _gen(self.device, _seed(w, _STEP_Q, _SHARED, step))
        return torch.randn((w.B, w.Hq, w.D), generator=g, device=self.device).to(w.torch_dtype)


def to_oracle_input(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Host numpy view in the oracle's input convention: f32 values, or
    uint16 bit patterns for f16/bf16."""
    t = t.detach().contiguous().cpu()
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=False)
    return t.view(torch.int16).numpy().view(np.uint16)
