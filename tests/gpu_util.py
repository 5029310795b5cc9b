"""Helpers of the GPU parity tests: run the HIP path through the binding and
compare with the CPU oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth

# Tolerance on attention outputs (bf16 I/O, fp32 accumulation):
# |gpu - ref| <= ATOL + RTOL * |ref| elementwise.
ATOL, RTOL = 2e-2, 1e-2
# fp32 path: every step in fp32, so rounding stays near 1e-6 relative.
ATOL_F32, RTOL_F32 = 1e-4, 1e-4

KINDS = {0: O.SLIDING, 1: O.FULL}


def prefill_q_scale(d: int, dtype=torch.bfloat16) -> float:
    """Factor the library's prefill holds its rotated queries times: the MFMA
    kernel (d = 128, bfloat16 operands) takes them times its base-2 softmax
    scale, fp32(log2(e) / sqrt(d)), rounded to bfloat16 once; other paths
    hold the queries themselves.  The rounded oracle's ``q_scale``."""
    if d == 128 and dtype != torch.float32:
        return float(np.float32(np.log2(np.e) / np.sqrt(np.float64(d))))
    return 1.0


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref, atol=ATOL, rtol=RTOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    if got.size == 0:
        return 0.0, 0.0
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements beyond tolerance; max |err| "
            f"{err.max():.3e}; first at {idx.tolist()}: got {got[tuple(idx[0])]:.5f} "
            f"ref {ref[tuple(idx[0])]:.5f}")
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return float(err.max()), float(rel[np.abs(ref) > 1e-3].max() if (np.abs(ref) > 1e-3).any() else 0.0)


def oracle_rope(rope: A.Rope) -> O.RopeParams:
    return O.RopeParams(theta=rope.theta, yarn=rope.yarn, factor=rope.factor,
                        orig_ctx=rope.orig_ctx, beta_fast=rope.beta_fast,
                        beta_slow=rope.beta_slow, attn_factor=rope.attn_factor)


def make_cache(B, G, cap, d, dtype, device, fill=None):
    if fill is None:
        k = torch.zeros((B, G, cap, d), dtype=dtype, device=device)
        v = torch.zeros((B, G, cap, d), dtype=dtype, device=device)
    else:
        k, v = fill
    return k, v


def gpu_prefill(x, k_cache, v_cache, *, window, layer_type, rope, eps=1e-6, H, pos_offset=0):
    B, T, _ = x["q_pre"].shape
    G, cap, d = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    out = torch.empty_like(x["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, layer_type, x["q_pre"].dtype, cap, x["q_pre"].device)
    A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], k_cache, v_cache,
                         out, ws, window=window, layer_type=layer_type, rope=rope, eps=eps,
                         pos_offset=pos_offset)
    return out


def gpu_decode(q, k, v, q_gain, k_gain, k_cache, v_cache, *, window, layer_type, rope, pos,
               eps=1e-6, H):
    B = q.shape[0]
    G, cap, d = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, layer_type, q.dtype, cap, q.device)
    A.olmo3_attn_decode(q, k, v, q_gain, k_gain, k_cache, v_cache, out, ws, window=window,
                        layer_type=layer_type, rope=rope, pos=pos, eps=eps)
    return out


def host_inputs(x):
    return {k: host(v) for k, v in x.items()}


def inputs(seed, layer, B, T, H, G, d, dtype, device="cuda"):
    return synth.layer_inputs(seed, layer, B, T, H, G, d, device=device, dtype=dtype)
