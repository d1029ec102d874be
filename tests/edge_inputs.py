"""Seeded inputs that put the quantizer on its edge cases, for the flush
kernel's device tests and their CPU check.  Pure numpy; no quantization
arithmetic beyond what is needed to place values (the oracle decides the
codes).

Every group (keys: one channel over G tokens; values: one token over G
channels) follows one pattern, chosen by its index:
  0 ties       min + (k + 1/2) s0 with s0 a power of two and max = min +
               (2^b - 1) s0, so the binary32 quotient (x - min) / s is exactly
               a half-integer (round-half-even decides)
  1 near ties  fp16 values whose binary32 quotient lies within 2^-12 of a
               half-integer without being one (fp16 inputs only; random
               normal values otherwise)
  2 constant   one value repeated (scale 0)
  3 zeros      +0 and -0 mixed (scale 0, the zero must come out +0)
  4 -0 minimum values in [0, 4] with some -0 entries (minimum -0)
  5 subnormal  fp16 subnormals k * 2^-24, both signs
  6 extremes   the largest finite magnitudes of the input format (+-65504 for
               fp16 and fp32 inputs, +-65280 for bf16) with random values
  7 normal     N(0, 1) values
All values are exactly representable in the input dtype (so the entry
rounding to fp16 leaves them as planted), except pattern 5 in bf16, whose
values the entry conversion rounds to fp16 subnormals."""
from __future__ import annotations

import numpy as np

NPAT = 8


def _fp(x, dtype):
    x = np.asarray(x, np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16  # round to nearest even bf16
        return u.astype(np.uint32).view(np.float32)
    return x.astype(np.float16).astype(np.float32)


def _near_ties(rng, G, bits):
    """fp16 group whose quotients sit within 2^-12 of half-integers (but not on them)."""
    L = np.float32((1 << bits) - 1)
    for _ in range(200):
        mn = np.float32(np.float16(rng.uniform(-3, 0)))
        mx = np.float32(np.float16(mn + rng.uniform(0.5, 6)))
        s = np.float32((mx - mn) / L)
        # every fp16 value in (mn, mx)
        lo, hi = np.float16(mn).view(np.uint16), np.float16(mx).view(np.uint16)
        cand = []
        for v in np.linspace(float(mn), float(mx), 4000).astype(np.float16):
            x = np.float32(v)
            if not (mn < x < mx):
                continue
            q = np.float32(x - mn) / s
            d = abs(q - (np.floor(q) + np.float32(0.5)))
            if 0 < d < 2.0 ** -12:
                cand.append(x)
        cand = np.unique(np.asarray(cand, np.float32))
        if cand.size >= 2:
            vals = rng.choice(cand, G - 2)
            g = np.concatenate([[mn, mx], vals]).astype(np.float32)
            return rng.permutation(g)
    raise RuntimeError("no near-tie group found")


def group(pattern, rng, G, bits, dtype):
    L = (1 << bits) - 1
    if pattern == 0:
        s0 = np.float32(2.0 ** rng.integers(-4, 1))
        mn = np.float32(rng.integers(-8, 9)) * s0 / 2
        k = rng.integers(0, L, G).astype(np.float32)
        g = mn + (k + np.float32(0.5)) * s0
        i, j = rng.choice(G, 2, replace=False)
        g[i], g[j] = mn, mn + L * s0
        return g.astype(np.float32)
    if pattern == 1:
        if dtype == "bf16":
            return _fp(rng.standard_normal(G), dtype)
        return _near_ties(rng, G, bits)
    if pattern == 2:
        return np.full(G, _fp(rng.standard_normal(), dtype), np.float32)
    if pattern == 3:
        return np.where(rng.random(G) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    if pattern == 4:
        g = _fp(rng.uniform(0, 4, G), dtype)
        g[rng.random(G) < 0.3] = np.float32(-0.0)
        g[rng.integers(G)] = np.float32(-0.0)
        return g
    if pattern == 5:
        g = rng.integers(-1023, 1024, G).astype(np.float32) * np.float32(2.0 ** -24)
        return g if dtype != "bf16" else _fp(g, dtype)
    if pattern == 6:
        big = np.float32(65280.0 if dtype == "bf16" else 65504.0)
        g = _fp(rng.uniform(-60000, 60000, G), dtype)
        i, j = rng.choice(G, 2, replace=False)
        g[i], g[j] = big, -big
        return g
    return _fp(rng.standard_normal(G), dtype)


def edge_kv(B, Hkv, N, D, G, kbits, vbits, dtype, seed):
    """K, V float32 [B, Hkv, N, D] holding the patterned groups (keys along
    tokens per channel, values along channels per token)."""
    rng = np.random.default_rng(seed)
    K = np.zeros((B, Hkv, N, D), np.float32)
    V = np.zeros((B, Hkv, N, D), np.float32)
    for b in range(B):
        for h in range(Hkv):
            for g0 in range(0, N, G):
                n = min(G, N - g0)
                for c in range(D):
                    p = (c * 7 + g0 // G + h) % NPAT
                    K[b, h, g0:g0 + n, c] = group(p, rng, G, kbits, dtype)[:n]
            for t in range(N):
                for j in range(D // G):
                    p = (t * 5 + j + b) % NPAT
                    V[b, h, t, j * G:(j + 1) * G] = group(p, rng, G, vbits, dtype)
    return K, V
