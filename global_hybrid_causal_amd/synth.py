"""Seeded synthetic inputs shaped like the OLMo 3 attention workloads.

This module only draws random numbers; it holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can be fed from it.  Each
tensor gets its own stream: the torch generator on the target device is
seeded with a 63-bit value derived from (seed, layer, tensor id) through
NumPy's SeedSequence.  Values are drawn in fp32 and rounded to the storage
dtype with torch's round-to-nearest-even conversion.

Distributions follow the workload descriptions: projected queries, keys and
values and pre-filled cache entries ~ N(0, 1); QK-norm gains ~ U(0.5, 1.5).
"""

from __future__ import annotations

import numpy as np
import torch

# tensor ids (part of each stream's seed)
Q_PRE, K_PRE, V_IN, Q_GAIN, K_GAIN, CACHE_K, CACHE_V = 1, 2, 3, 4, 5, 6, 7

_CHUNK = 1 << 26  # elements drawn per fp32 chunk for very large tensors


def derive_seed(seed: int, *keys: int) -> int:
    """63-bit generator seed for the stream (seed, *keys)."""
    state = np.random.SeedSequence([int(seed), *[int(k) for k in keys]]).generate_state(2, np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 63) - 1)


def _generator(device, seed, keys):
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, *keys))
    return g


def normal(shape, seed: int, *keys: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, 1) tensor of ``shape``; drawn in fp32 chunks, rounded to ``dtype``."""
    g = _generator(device, seed, keys)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        flat[i:i + m] = torch.randn(m, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def uniform(shape, lo: float, hi: float, seed: int, *keys: int, device="cpu",
            dtype=torch.bfloat16) -> torch.Tensor:
    """U(lo, hi) tensor of ``shape``, drawn in fp32, rounded to ``dtype``."""
    g = _generator(device, seed, keys)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return (lo + (hi - lo) * x).to(dtype)


def layer_inputs(seed: int, layer: int, B: int, T: int, H: int, G: int, d: int,
                 device="cpu", dtype=torch.bfloat16) -> dict:
    """Projected q/k/v of one call and the layer's QK-norm gains.

    q_pre [B, T, H*d], k_pre and v [B, T, G*d] ~ N(0, 1); q_gain [H*d] and
    k_gain [G*d] ~ U(0.5, 1.5)."""
    return {
        "q_pre": normal((B, T, H * d), seed, layer, Q_PRE, device=device, dtype=dtype),
        "k_pre": normal((B, T, G * d), seed, layer, K_PRE, device=device, dtype=dtype),
        "v": normal((B, T, G * d), seed, layer, V_IN, device=device, dtype=dtype),
        "q_gain": uniform((H * d,), 0.5, 1.5, seed, layer, Q_GAIN, device=device, dtype=dtype),
        "k_gain": uniform((G * d,), 0.5, 1.5, seed, layer, K_GAIN, device=device, dtype=dtype),
    }


def e4m3_codes(shape, seed: int, *keys: int, device="cpu", exp_lo: int = 5,
               exp_hi: int = 8, all_codes: bool = False) -> torch.Tensor:
    """Random e4m3 bytes (uint8): uniform sign bit, exponent field uniform in
    [exp_lo, exp_hi], uniform 3-bit mantissa.  The default fields give
    magnitudes 0.25 .. 3.75; no NaN code is drawn.  all_codes: every one of
    the 254 non-NaN codes equally likely instead (zeros, subnormals and the
    largest magnitude 448 included)."""
    g = _generator(device, seed, keys)
    if all_codes:
        k = torch.randint(0, 254, shape, generator=g, device=device, dtype=torch.int32)
        return (k + (k >= 0x7F).to(torch.int32)).to(torch.uint8)  # skip 0x7F; 0xFF is past the range
    sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
    exp = torch.randint(exp_lo, exp_hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    man = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
    return ((sign << 7) | (exp << 3) | man).to(torch.uint8)


def e4m3_cache_fill(seed: int, layer: int, B: int, G: int, capacity: int, d: int,
                    device="cpu", all_codes: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Pre-filled e4m3 K and V caches [B, G, capacity, d] of random codes
    (``e4m3_codes``; all_codes draws every non-NaN code)."""
    return (e4m3_codes((B, G, capacity, d), seed, layer, CACHE_K, device=device, all_codes=all_codes),
            e4m3_codes((B, G, capacity, d), seed, layer, CACHE_V, device=device, all_codes=all_codes))


def cache_fill(seed: int, layer: int, B: int, G: int, capacity: int, d: int,
               device="cpu", dtype=torch.bfloat16) -> tuple[torch.Tensor, torch.Tensor]:
    """Pre-filled K and V caches [B, G, capacity, d] ~ N(0, 1)."""
    k = normal((B, G, capacity, d), seed, layer, CACHE_K, device=device, dtype=dtype)
    v = normal((B, G, capacity, d), seed, layer, CACHE_V, device=device, dtype=dtype)
    return k, v
