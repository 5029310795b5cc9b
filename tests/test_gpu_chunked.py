"""Chunked prefill: T new tokens at positions pos_offset .. pos_offset+T-1
attend to the positions the cache already holds and to each other ("Olmo-3
End-to-End Implementation", "Cache Operation Flow": cached keys and values
are joined with the new ones before attention, then the new ones are stored).
Every output element and every cache slot is compared with the fp64 oracle on
the same seeded inputs; the kernel's tile walk is compared bit for bit with
the mask at the same positions."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import (ATOL_F32, KINDS, RTOL_F32, assert_close, gpu_prefill, host, host_inputs,
                      inputs, oracle_rope)

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _log(*a):
    print(*a, flush=True)


CHUNK_CASES = [
    # B, T, H, G, d, window, layer_type, pos_offset, yarn, dtype
    (1, 100, 4, 4, 128, 64, 0, 64, False, BF16),     # ring exactly full, tile-aligned chunk
    (2, 77, 8, 2, 128, 100, 0, 250, False, BF16),    # wrapped ring, tiles cross the wrap
    (1, 300, 4, 1, 128, 256, 0, 1000, False, BF16),  # chunk longer than the window
    (1, 1, 4, 2, 128, 64, 0, 5, False, BF16),        # one token, ring not yet full
    (1, 200, 4, 4, 128, 128, 0, 37, False, BF16),    # unaligned prefix, ring not full
    (2, 130, 10, 2, 128, 4096, 1, 200, True, BF16),  # full layer, YaRN, GQA 5:1
    (1, 64, 4, 4, 128, 4096, 1, 63, False, BF16),    # full layer, unaligned prefix
    (1, 129, 4, 2, 128, 4096, 1, 4096, True, BF16),  # full layer, long prefix
    (1, 40, 4, 2, 128, 1, 0, 10, False, BF16),       # window 1: every query sees itself only
    (1, 70, 4, 2, 128, 16, 0, 100, False, BF16),     # ring shorter than a key tile
    (1, 50, 4, 2, 64, 40, 0, 77, False, BF16),       # plain kernel, ring
    (2, 33, 2, 1, 16, 4096, 1, 20, True, BF16),      # plain kernel, linear
    (1, 8, 2, 1, 16, 16, 0, 64, False, F32),         # fp32, ring
    (1, 8, 2, 1, 16, 16, 1, 64, False, F32),         # fp32, linear
    # the last positions a prefill takes (pos_offset + T = 2^30), on rings
    (1, 700, 4, 2, 128, 4096, 0, (1 << 30) - 700, False, BF16),
    (2, 300, 8, 2, 128, 256, 0, (1 << 30) - 300, False, BF16),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[str(c[:9]) + ("f32" if c[9] == F32 else "")
                                                   for c in CHUNK_CASES])
def test_chunk_onto_filled_cache(case):
    """Cache pre-filled with seeded rows holding positions 0 .. pos_offset-1
    (a ring keeps the last `window`), then one chunk."""
    B, T, H, G, d, w, lt, P, yarn, dt = case
    _log("chunk case", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=yarn, factor=8.0, orig_ctx=256)
    cap = w if kind == O.SLIDING else P + T + 5
    kc, vc = synth.cache_fill(37, lt, B, G, cap, d, device="cuda", dtype=dt)
    hk, hv = host(kc), host(vc)
    tags = O.ring_positions(kind, w, cap, P)
    x = inputs(37, 20 + lt, B, T, H, G, d, dt)
    out = gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=rope, H=H, pos_offset=P)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d)
    ref_cache.k[:] = hk
    ref_cache.v[:] = hv
    ref_cache.pos[:] = tags
    ref = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                        pos_offset=P, cache=ref_cache)
    tol = (ATOL_F32, RTOL_F32) if dt == F32 else ()
    err = assert_close(host(out), ref, *tol, what=f"chunk {case}")
    _log("  max abs / rel err", err)
    # slots of the chunk's kept positions: values bit-exact, keys to tolerance;
    # every other slot keeps its bytes
    new = np.nonzero(ref_cache.pos >= P)[0]
    kcg, vcg = host(kc), host(vc)
    assert np.array_equal(vcg[:, :, new], ref_cache.v[:, :, new]), "value slots"
    assert_close(kcg[:, :, new], ref_cache.k[:, :, new], *tol, what="key slots")
    old = np.setdiff1d(np.arange(cap), new)
    assert np.array_equal(kcg[:, :, old], hk[:, :, old]) and np.array_equal(vcg[:, :, old], hv[:, :, old])
    assert new.size == (min(T, w) if kind == O.SLIDING else T)


@pytest.mark.parametrize("lt", [0, 1])
@pytest.mark.parametrize("chunks", [(128, 1, 100, 71), (64, 64, 64, 108), (1, 299)])
def test_chunks_equal_one_prefill(lt, chunks):
    """A prompt prefilled in chunks gives the rows of the one-call prefill,
    and leaves the same cache (both checked against the oracle)."""
    B, H, G, d, w = 2, 8, 4, 128, 100
    T = sum(chunks)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=128)
    x = inputs(41, lt, B, T, H, G, d, BF16)
    hx = host_inputs(x)
    cap = w if lt == 0 else T
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d)
    ref = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                        cache=ref_cache)
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    p = 0
    for c in chunks:
        part = {k: (v[:, p:p + c].contiguous() if v.dim() == 3 else v) for k, v in x.items()}
        out = gpu_prefill(part, kc, vc, window=w, layer_type=lt, rope=rope, H=H, pos_offset=p)
        assert_close(host(out), ref[:, p:p + c], what=f"{kind} chunk at {p} of {chunks}")
        p += c
    held = np.nonzero(ref_cache.pos >= 0)[0]
    assert np.array_equal(host(vc)[:, :, held], ref_cache.v[:, :, held])
    assert_close(host(kc)[:, :, held], ref_cache.k[:, :, held], what="cache keys")


def test_ring_chunk_takes_the_workspace_without_split_states():
    """A sliding-layer chunk after a ring prefix never splits its keys, so it
    runs with the workspace of its rotated queries and keys alone, smaller
    than olmo3_workspace_bytes gives for a small grid (which holds split
    states for the call without a prefix), and matches the oracle."""
    B, T, H, G, d, w, P = 1, 300, 4, 2, 128, 256, 1000
    rope = A.Rope(theta=500000.0)
    x = inputs(43, 0, B, T, H, G, d, BF16)
    align = lambda n: (n + 255) // 256 * 256
    small = align(B * T * H * d * 2) + align(B * G * T * d * 2)
    full = A.olmo3_workspace_bytes(A.MODE_PREFILL, B, T, H, G, d, 0, A.DTYPE_BF16, w)
    assert full > small
    kc, vc = synth.cache_fill(43, 5, B, G, w, d, device="cuda", dtype=BF16)
    hk, hv = host(kc), host(vc)
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x["q_pre"])
    A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc, out, ws,
                         window=w, layer_type=0, rope=rope, pos_offset=P)
    ref_cache = O.KvCacheRef(O.SLIDING, w, w, B, G, d)
    ref_cache.k[:] = hk
    ref_cache.v[:] = hv
    ref_cache.pos[:] = O.ring_positions(O.SLIDING, w, w, P)
    ref = O.prefill_ref(**host_inputs(x), H=H, G=G, d=d, kind=O.SLIDING, window=w,
                        rope=oracle_rope(rope), pos_offset=P, cache=ref_cache)
    assert_close(host(out), ref, what="ring chunk, small workspace")


@pytest.mark.parametrize("T,P", [(1, 1), (5, 64), (64, 64), (127, 300), (300, 129), (1000, 4096),
                                 (200, 4000), (4096, 4096)])
@pytest.mark.parametrize("window", [1, 63, 100, 128, 4096])
@pytest.mark.parametrize("splits", [1, 2])
def test_probe_prefill_visits_with_offset(T, P, window, splits):
    for lt in (0, 1):
        got = A.olmo3_probe_prefill_visits(T, window, lt, pos_offset=P,
                                           kv_splits=splits).cpu().numpy()
        want = O.mask_at_positions(P + np.arange(T), np.arange(P + T), KINDS[lt], window)
        assert np.array_equal(got, want), (T, P, window, lt, np.argwhere(got != want)[:5])
