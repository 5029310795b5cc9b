"""Ragged batches: sequences of different lengths and positions in one call
(several prompts served together, "Olmo-3 End-to-End Implementation", "Next
Steps").  Each sequence is compared with the fp64 oracle run on that
sequence alone, with its own cache; equal lengths and positions must give
the bits of the uniform entry points."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import (ATOL_F32, KINDS, RTOL_F32, assert_close, gpu_decode, gpu_prefill, host,
                      host_inputs, inputs, oracle_rope)

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _log(*a):
    print(*a, flush=True)


def _filled_cache(kind, w, cap, B, G, d, dt, positions, seed, layer):
    """Seeded cache rows; sequence b holds the positions a cache filled from 0
    up to positions[b] - 1 would hold.  Returns device caches and the oracle's
    per-sequence caches."""
    kc, vc = synth.cache_fill(seed, layer, B, G, cap, d, device="cuda", dtype=dt)
    hk, hv = host(kc), host(vc)
    refs = []
    for b, p in enumerate(positions):
        c = O.KvCacheRef(kind, w, cap, 1, G, d)
        c.k[:] = hk[b:b + 1]
        c.v[:] = hv[b:b + 1]
        c.pos[:] = O.ring_positions(kind, w, cap, int(p))
        refs.append(c)
    return kc, vc, hk, hv, refs


def _check_caches(kc, vc, hk, hv, refs, starts, what, tol):
    """Slots of each sequence's new positions match its oracle cache (values
    bit for bit, keys to tolerance); every other slot keeps its bytes."""
    kcg, vcg = host(kc), host(vc)
    for b, (c, p0) in enumerate(zip(refs, starts)):
        new = np.nonzero(c.pos >= p0)[0]
        assert np.array_equal(vcg[b][:, new], c.v[0][:, new]), f"{what}: values of sequence {b}"
        assert_close(kcg[b][:, new], c.k[0][:, new], *tol, what=f"{what}: keys of sequence {b}")
        old = np.setdiff1d(np.arange(c.capacity), new)
        assert np.array_equal(kcg[b][:, old], hk[b][:, old]), f"{what}: sequence {b} slot overwritten"
        assert np.array_equal(vcg[b][:, old], hv[b][:, old])


DECODE_CASES = [
    # H, G, d, window, layer_type, positions, dtype
    (8, 2, 128, 128, 0, [0, 1, 127, 128, 1000], BF16),   # ring: empty, wrapping, long past
    (8, 2, 128, 4096, 1, [0, 5, 399, 64, 250], BF16),    # linear cache, mixed lengths
    (10, 2, 128, 4096, 1, [2999, 0, 1500], BF16),         # group 5, very different lengths
    (16, 2, 128, 300, 0, [4000, 10, 299, 300], BF16),     # group 8
    (6, 2, 64, 64, 0, [100, 3, 63], BF16),                # plain kernel
    (2, 1, 16, 16, 1, [30, 0, 7], F32),                   # fp32
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"{c[4]}-{c[2]}-{len(c[5])}seq" + ("-f32" if c[6] == F32 else "")
                                                    for c in DECODE_CASES])
def test_ragged_decode_vs_oracle(case):
    H, G, d, w, lt, positions, dt = case
    B = len(positions)
    _log("ragged decode", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    max_pos = max(positions)
    cap = w if kind == O.SLIDING else max_pos + 1
    kc, vc, hk, hv, refs = _filled_cache(kind, w, cap, B, G, d, dt, positions, 43, lt)
    x = inputs(43, 30 + lt, B, 1, H, G, d, dt)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    pos_t = torch.tensor(positions, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, dt, cap, "cuda")
    A.olmo3_attn_decode_ragged(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, pos_t,
                               max_pos=max_pos, window=w, layer_type=lt, rope=rope)
    hx = host_inputs(x)
    tol = (ATOL_F32, RTOL_F32) if dt == F32 else ()
    for b, p in enumerate(positions):
        ref = O.decode_ref(hx["q_pre"][b:b + 1, 0], hx["k_pre"][b:b + 1, 0], hx["v"][b:b + 1, 0],
                           hx["q_gain"], hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                           rope=oracle_rope(rope), pos=p, cache=refs[b])
        assert_close(host(out[b:b + 1]), ref, *tol, what=f"sequence {b} at {p}")
    _check_caches(kc, vc, hk, hv, refs, positions, "ragged decode", tol)


@pytest.mark.parametrize("lt", [0, 1])
def test_ragged_decode_equal_positions_is_uniform_decode(lt):
    B, H, G, d, w, pos = 4, 8, 2, 128, 256, 700
    rope = A.Rope(theta=500000.0, yarn=True)
    cap = w if lt == 0 else pos + 1
    x = inputs(47, lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    results = []
    for ragged in (False, True):
        kc, vc = synth.cache_fill(47, lt, B, G, cap, d, device="cuda", dtype=BF16)
        if ragged:
            out = torch.empty_like(q)
            ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, BF16, cap, "cuda")
            A.olmo3_attn_decode_ragged(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws,
                                       torch.full((B,), pos, dtype=torch.int32, device="cuda"),
                                       max_pos=pos, window=w, layer_type=lt, rope=rope)
        else:
            out = gpu_decode(q, k, v, x["q_gain"], x["k_gain"], kc, vc, window=w, layer_type=lt,
                             rope=rope, pos=pos, H=H)
        torch.cuda.synchronize()
        results.append((out, kc, vc))
    for a_, b_ in zip(*results):
        assert torch.equal(a_, b_)


PREFILL_CASES = [
    # H, G, d, window, layer_type, lengths, offsets, dtype
    (8, 2, 128, 100, 0, [1, 130, 64, 300], [0, 0, 70, 1000], BF16),     # ring, some with a prefix
    (8, 2, 128, 4096, 1, [1, 130, 64, 300], [0, 0, 70, 1000], BF16),    # linear, YaRN
    (10, 2, 128, 256, 0, [257, 0, 129], [5, 0, 300], BF16),             # group 5, an empty sequence
    (4, 4, 128, 4096, 1, [500, 1, 128], [0, 12, 128], BF16),            # block edges
    (6, 2, 64, 40, 0, [50, 7, 90], [77, 0, 3], BF16),                   # plain kernel
    (2, 1, 16, 16, 1, [8, 20, 1], [64, 0, 5], F32),                     # fp32
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"{c[4]}-{c[2]}-{len(c[5])}seq" + ("-f32" if c[7] == F32 else "")
                                                     for c in PREFILL_CASES])
def test_ragged_prefill_vs_oracle(case):
    H, G, d, w, lt, lengths, offsets, dt = case
    B = len(lengths)
    _log("ragged prefill", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=256)
    ends = [p + n for p, n in zip(offsets, lengths)]
    max_end, max_len, N = max(ends), max(lengths), sum(lengths)
    cap = w if kind == O.SLIDING else max_end + 2
    kc, vc, hk, hv, refs = _filled_cache(kind, w, cap, B, G, d, dt, offsets, 53, lt)
    per = [inputs(53, 40 + 7 * b + lt, 1, max(n, 1), H, G, d, dt) for b, n in enumerate(lengths)]
    packed = {k: torch.cat([p[k][0, :n] for p, n in zip(per, lengths)]).contiguous()
              for k in ("q_pre", "k_pre", "v")}
    gains = {k: per[0][k] for k in ("q_gain", "k_gain")}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    po = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    out = torch.full_like(packed["q_pre"], 9.0)
    ws = A.workspace(A.MODE_PREFILL, 1, N, H, G, d, lt, dt, cap, "cuda")
    A.olmo3_attn_prefill_ragged(packed["q_pre"], packed["k_pre"], packed["v"], gains["q_gain"],
                                gains["k_gain"], kc, vc, out, ws, cu, po, max_len=max_len,
                                max_end=max_end, window=w, layer_type=lt, rope=rope)
    tol = (ATOL_F32, RTOL_F32) if dt == F32 else ()
    hq, hk_pre, hv_in = host(packed["q_pre"]), host(packed["k_pre"]), host(packed["v"])
    hg = {k: host(t) for k, t in gains.items()}
    row = 0
    for b, (n, p) in enumerate(zip(lengths, offsets)):
        if n:
            ref = O.prefill_ref(hq[None, row:row + n], hk_pre[None, row:row + n],
                                hv_in[None, row:row + n], hg["q_gain"], hg["k_gain"], H=H, G=G,
                                d=d, kind=kind, window=w, rope=oracle_rope(rope), pos_offset=p,
                                cache=refs[b])
            assert_close(host(out[row:row + n])[None], ref, *tol, what=f"sequence {b}")
        row += n
    _check_caches(kc, vc, hk, hv, refs, offsets, "ragged prefill", tol)


@pytest.mark.parametrize("lt", [0, 1])
def test_ragged_prefill_equal_lengths_is_uniform_prefill(lt):
    """32 sequences of 200 rows x 8 heads are 512 query blocks x heads, so
    the uniform call keeps one workgroup per block (smaller grids split the
    keys and merge, which sums in another order) like the packed one: the
    two must agree bit for bit."""
    B, T, H, G, d, w = 32, 200, 8, 4, 128, 64
    rope = A.Rope(theta=500000.0, yarn=True)
    cap = w if lt == 0 else T
    x = inputs(59, lt, B, T, H, G, d, BF16)
    results = []
    for ragged in (False, True):
        kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
        vc = torch.zeros_like(kc)
        if ragged:
            flat = {k: (t.reshape(B * T, -1) if t.dim() == 3 else t) for k, t in x.items()}
            out = torch.empty_like(flat["q_pre"])
            ws = A.workspace(A.MODE_PREFILL, 1, B * T, H, G, d, lt, BF16, cap, "cuda")
            cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
            A.olmo3_attn_prefill_ragged(flat["q_pre"], flat["k_pre"], flat["v"], flat["q_gain"],
                                        flat["k_gain"], kc, vc, out, ws, cu, None, max_len=T,
                                        max_end=T, window=w, layer_type=lt, rope=rope)
            out = out.reshape(B, T, -1)
        else:
            out = gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=rope, H=H)
        torch.cuda.synchronize()
        results.append((out, kc, vc))
    for a_, b_ in zip(*results):
        assert torch.equal(a_, b_)


E4M3_DECODE_CASES = [
    # H, G, window, layer_type, positions
    (8, 8, 128, 0, [0, 1, 127, 128, 1000]),     # one query head per key/value head, ring
    (10, 2, 4096, 1, [2999, 0, 1500]),           # group 5 (grouped MFMA kernel), linear
    (16, 2, 300, 0, [4000, 10, 299, 300]),       # group 8, ring
]


@pytest.mark.parametrize("case", E4M3_DECODE_CASES, ids=[f"{c[3]}-g{c[0] // c[1]}-{len(c[4])}seq"
                                                         for c in E4M3_DECODE_CASES])
def test_ragged_decode_e4m3_vs_oracle(case):
    """Per-sequence positions against e4m3 caches: each sequence matches the
    oracle's e4m3 decode on its own cache, and its new codes land in its own
    slot."""
    H, G, w, lt, positions = case
    B, d, ks, vs = len(positions), 128, 0.37, 1.9
    _log("ragged e4m3 decode", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    max_pos = max(positions)
    cap = w if kind == O.SLIDING else max_pos + 1
    kc, vc = synth.e4m3_cache_fill(53, lt, B, G, cap, d, device="cuda")
    bk, bv = kc.cpu().numpy(), vc.cpu().numpy()  # codes, as uint8
    table = O.e4m3_values()
    x = inputs(53, 40 + lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    pos_t = torch.tensor(positions, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_decode_ragged_e4m3(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, pos_t,
                                    k_scale=ks, v_scale=vs, max_pos=max_pos, window=w,
                                    layer_type=lt, rope=rope)
    hx = host_inputs(x)
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    for b, p in enumerate(positions):
        c = O.KvCacheRef(kind, w, cap, 1, G, d, e4m3_scales=(ks, vs))
        c.k[:] = table[bk[b:b + 1]] * ks
        c.v[:] = table[bv[b:b + 1]] * vs
        c.pos[:] = O.ring_positions(kind, w, cap, int(p))
        ref = O.decode_e4m3_ref(hx["q_pre"][b:b + 1, 0], hx["k_pre"][b:b + 1, 0],
                                hx["v"][b:b + 1, 0], hx["q_gain"], hx["k_gain"], H=H, G=G, d=d,
                                kind=kind, window=w, rope=oracle_rope(rope), pos=p, cache=c)
        assert_close(host(out[b:b + 1]), ref, what=f"sequence {b} at {p}")
        slot = p % w if kind == O.SLIDING else p
        assert np.array_equal(got_v[b][:, slot], O.e4m3_store(hx["v"][b, 0].reshape(G, d), vs)), \
            f"sequence {b}: value codes"
        others = np.setdiff1d(np.arange(cap), [slot])
        assert np.array_equal(got_k[b][:, others], bk[b][:, others]), f"sequence {b}: key slots"
        assert np.array_equal(got_v[b][:, others], bv[b][:, others]), f"sequence {b}: value slots"


@pytest.mark.parametrize("lt", [0, 1])
def test_ragged_serving_flow(lt):
    """Prompts ingested together from empty caches, a second chunk of each at
    its own offset (read over the cache the first one left), then three
    decode steps at per-sequence positions: every output follows the
    oracle's cache flow for that sequence alone."""
    H, G, d, w = 8, 2, 128, 96
    first, second, steps = [70, 3, 130], [40, 100, 1], 3
    B = len(first)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=256)
    ends = [a + b + steps for a, b in zip(first, second)]
    cap = w if kind == O.SLIDING else max(ends)
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    refs = [O.KvCacheRef(kind, w, cap, 1, G, d) for _ in range(B)]

    def chunk(lengths, offsets, seed):
        per = [inputs(seed, b, 1, n, H, G, d, BF16) for b, n in enumerate(lengths)]
        packed = {k: torch.cat([p[k][0] for p in per]).contiguous() for k in ("q_pre", "k_pre", "v")}
        gains = {k: per[0][k] for k in ("q_gain", "k_gain")}
        N = sum(lengths)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
        po = torch.tensor(offsets, dtype=torch.int32, device="cuda")
        out = torch.empty_like(packed["q_pre"])
        ws = A.workspace(A.MODE_PREFILL, 1, N, H, G, d, lt, BF16, cap, "cuda")
        A.olmo3_attn_prefill_ragged(packed["q_pre"], packed["k_pre"], packed["v"], gains["q_gain"],
                                    gains["k_gain"], kc, vc, out, ws, cu, po, max_len=max(lengths),
                                    max_end=max(p + n for p, n in zip(offsets, lengths)), window=w,
                                    layer_type=lt, rope=rope)
        hq, hk_pre, hv_in = host(packed["q_pre"]), host(packed["k_pre"]), host(packed["v"])
        hg = {k: host(t) for k, t in gains.items()}
        got, row = host(out), 0
        for b, (n, p) in enumerate(zip(lengths, offsets)):
            ref = O.prefill_ref(hq[None, row:row + n], hk_pre[None, row:row + n],
                                hv_in[None, row:row + n], hg["q_gain"], hg["k_gain"], H=H, G=G,
                                d=d, kind=kind, window=w, rope=oracle_rope(rope), pos_offset=p,
                                cache=refs[b])
            assert_close(got[row:row + n][None], ref, what=f"chunk at {p} of sequence {b}")
            row += n
        return hg

    hg = chunk(first, [0] * B, 101)
    hg = chunk(second, first, 102)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, BF16, cap, "cuda")
    for step in range(steps):
        xs = inputs(103, step, B, 1, H, G, d, BF16)
        q, k, v = (xs[key][:, 0].contiguous() for key in ("q_pre", "k_pre", "v"))
        positions = [a + b + step for a, b in zip(first, second)]
        out = torch.empty_like(q)
        A.olmo3_attn_decode_ragged(q, k, v, xs["q_gain"], xs["k_gain"], kc, vc, out, ws,
                                   torch.tensor(positions, dtype=torch.int32, device="cuda"),
                                   max_pos=max(positions), window=w, layer_type=lt, rope=rope)
        hx = host_inputs(xs)
        got = host(out)
        for b, p in enumerate(positions):
            ref = O.decode_ref(hx["q_pre"][b:b + 1, 0], hx["k_pre"][b:b + 1, 0],
                               hx["v"][b:b + 1, 0], hx["q_gain"], hx["k_gain"], H=H, G=G, d=d,
                               kind=kind, window=w, rope=oracle_rope(rope), pos=p, cache=refs[b])
            assert_close(got[b:b + 1], ref, what=f"step {step}, sequence {b} at {p}")
