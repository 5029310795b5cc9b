"""Index work of the prefill path checked bit for bit through planted values
and through the prologue stage's own output.

Planted values: with q = 0 every visible key scores 0, so attention is the
plain mean of the visible value rows.  All value rows are 0 except one
planted at 1024 (or 1024 (b + 1) for sequence b of a packed call), so a row
reads exactly 1024/n, n = its number of visible keys, when it sees the
planted key and exactly 0 when it does not: any key taken across a window
edge, across the causal edge, across a ring's wrap or across a sequence
boundary moves an output off those values (mask of page "Case Study: OLMo
3", item 1; cache flow of page "Olmo-3 End-to-End Implementation", "Cache
Operation Flow").

Prologue stage: the rotated queries it writes to the workspace and the
rotated keys it writes to the cache are the bfloat16 rounding of the fp64
oracle's rms_norm -> rope_rotate value, bit for bit, except where the
kernel's fp32 arithmetic (error near 2^-24 of the rotated terms) can move
the value across a rounding boundary: next to a midpoint, or in a result
much smaller than its terms."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import KINDS, assert_close, gpu_prefill, host, inputs, oracle_rope, prefill_q_scale

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
PLANT = 1024.0
# Query blocks x heads x sequences below which a uniform call without a
# prefix splits each block's keys over two workgroups (sliding layers: only
# while the doubled grid stays within one round of 512).
SPLIT_BELOW = 512


def _log(*a):
    print(*a, flush=True)


def _kv_splits(B, T, H, lt):
    blocks = (T + 127) // 128 * H * B
    if blocks >= SPLIT_BELOW or (lt == 0 and 2 * blocks > SPLIT_BELOW):
        return 1
    return 2


def _visible_counts(kind, w, q_pos, chunk=512):
    """Number of keys each query position sees when every earlier position
    is present (the oracle's mask over positions 0 .. max(q_pos))."""
    keys = np.arange(int(q_pos.max()) + 1)
    return np.concatenate([O.mask_at_positions(q_pos[i:i + chunk], keys, kind, w).sum(axis=1)
                           for i in range(0, len(q_pos), chunk)])


def _check_planted(out, q_pos, s_star, kind, w, value, what):
    """out [rows, H*d] of queries at q_pos with one value row planted at key
    position s_star: value/n where the row sees it, 0 elsewhere."""
    sees = O.mask_at_positions(q_pos, np.array([s_star]), kind, w)[:, 0]
    assert (out[~sees] == 0.0).all(), (what, np.nonzero((out[~sees] != 0).any(axis=1))[0][:5])
    if sees.any():
        n = _visible_counts(kind, w, q_pos[sees])
        want = (value / n)[:, None] * np.ones((1, out.shape[1]))
        assert_close(out[sees], want, 0.0, 2 ** -8, what)
    return int(sees.sum())


# ------------------------------------------------ full 7B length, one workgroup per block
@pytest.mark.parametrize("lt,s_star", [(0, 0), (0, 4095), (0, 4096), (0, 4097), (0, 8191),
                                       (1, 0), (1, 4096), (1, 8191)])
def test_planted_full_length_one_workgroup_per_block(lt, s_star):
    """T = 8192, window 4096, 8 heads: 64 query blocks x 8 heads = 512
    workgroups, the instance without a key split, at the 7B length."""
    B, T, H, G, d, w = 1, 8192, 8, 8, 128, 4096
    assert _kv_splits(B, T, H, lt) == 1
    kind = KINDS[lt]
    _log("planted full length", lt, s_star)
    x = inputs(67, lt, B, T, H, G, d, BF16)
    x["q_pre"].zero_()
    x["v"].zero_()
    x["v"][:, s_star] = PLANT
    cap = w if lt == 0 else T
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    out = host(gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=A.Rope(), H=H))[0]
    seen = _check_planted(out, np.arange(T), s_star, kind, w, PLANT, f"full length {lt} {s_star}")
    assert seen > 0


# ------------------------------------------------ chunk after a prefix held in the cache
RING_CASES = [
    # B, H, G, window, layer_type, pos_offset, T, planted positions
    (1, 4, 2, 256, 0, 1000, 700, [744, 745, 767, 768, 999, 1000, 1300, 1699]),
    (2, 32, 8, 256, 0, 1000, 700, [745, 767, 768, 999, 1000, 1300]),
    (1, 8, 8, 4096, 0, 5000, 1000, [904, 905, 4095, 4096, 4999, 5000, 5999]),
    (1, 4, 2, 4096, 1, 700, 600, [0, 63, 64, 699, 700, 1299]),             # linear cache
]


@pytest.mark.parametrize("case", RING_CASES, ids=[str(c[:7]) for c in RING_CASES])
def test_planted_chunk_after_cached_prefix(case):
    """A chunk at pos_offset > 0 reads the previous keys from the cache: on a
    sliding layer from the ring, whose slots wrap (slot = position mod
    window) inside the tiles the chunk walks; the planted row sits in the
    cache (positions below pos_offset) or in the chunk."""
    B, H, G, w, lt, P, T, plants = case
    d = 128
    kind = KINDS[lt]
    cap = w if lt == 0 else P + T
    pos_held = O.ring_positions(kind, w, cap, P)
    q_pos = P + np.arange(T)
    for s_star in plants:
        _log("planted after prefix", case[:7], s_star)
        x = inputs(71, lt, B, T, H, G, d, BF16)
        x["q_pre"].zero_()
        x["v"].zero_()
        kc, _ = synth.cache_fill(71, 60 + lt, B, G, cap, d, device="cuda", dtype=BF16)
        vc = torch.zeros_like(kc)
        if s_star < P:
            slot = int(np.nonzero(pos_held == s_star)[0][0])
            vc[:, :, slot] = PLANT
        else:
            x["v"][:, s_star - P] = PLANT
        out = host(gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=A.Rope(), H=H,
                               pos_offset=P))
        for b in range(B):
            _check_planted(out[b], q_pos, s_star, kind, w, PLANT, f"{case[:7]} s*={s_star} b={b}")


# ------------------------------------------------ packed rows of several sequences
PACKED_CASES = [
    # H, G, window, layer_type, lengths, offsets, planted position per sequence
    (8, 2, 100, 0, [300, 1, 129, 700], [0, 5, 64, 1000], [299, 5, 64, 950]),
    (8, 2, 4096, 1, [300, 1, 129, 700], [0, 5, 64, 1000], [0, 0, 192, 1699]),
    (32, 8, 256, 0, [1000, 257, 0, 513], [0, 300, 7, 4000], [743, 299, 0, 3800]),
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=[f"{c[3]}-w{c[2]}-h{c[0]}" for c in PACKED_CASES])
def test_planted_packed_sequences(case):
    """Sequence b plants 1024 (b + 1) at its own position (in its cache or in
    its rows): its rows read 1024 (b + 1)/n or 0, so a key read from another
    sequence's rows or cache shows up as a foreign multiple."""
    H, G, w, lt, lengths, offsets, plants = case
    d, B = 128, len(lengths)
    kind = KINDS[lt]
    _log("planted packed", case)
    ends = [p + n for p, n in zip(offsets, lengths)]
    max_end, max_len, N = max(ends), max(lengths), sum(lengths)
    cap = w if lt == 0 else max_end + 2
    x = inputs(73, lt, 1, N, H, G, d, BF16)
    q = torch.zeros_like(x["q_pre"][0])
    k = x["k_pre"][0].contiguous()
    v = torch.zeros_like(x["v"][0])
    kc, _ = synth.cache_fill(73, 70 + lt, B, G, cap, d, device="cuda", dtype=BF16)
    vc = torch.zeros_like(kc)
    row0 = np.concatenate([[0], np.cumsum(lengths)])
    for b, (s_star, p) in enumerate(zip(plants, offsets)):
        val = PLANT * (b + 1)
        if s_star < p:
            held = O.ring_positions(kind, w, cap, p)
            slot = int(np.nonzero(held == s_star)[0][0])
            vc[b, :, slot] = val
        elif s_star < p + lengths[b]:
            v[row0[b] + s_star - p] = val
    cu = torch.tensor(row0, dtype=torch.int32, device="cuda")
    po = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 9.0)
    ws = A.workspace(A.MODE_PREFILL, 1, N, H, G, d, lt, BF16, cap, "cuda")
    A.olmo3_attn_prefill_ragged(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, cu, po,
                                max_len=max_len, max_end=max_end, window=w, layer_type=lt,
                                rope=A.Rope())
    hout = host(out)
    for b, (n, p) in enumerate(zip(lengths, offsets)):
        if n:
            _check_planted(hout[row0[b]:row0[b] + n], p + np.arange(n), plants[b], kind, w,
                           PLANT * (b + 1), f"sequence {b}")


# ------------------------------------------------ the prologue stage's rotated rows
def _rotated_ref(x_pre, gain, heads, d, eps, positions, inv_freq, mscale):
    """fp64 oracle value of the rotated rows [rows, heads, d] and the size of
    the terms the kernel adds in fp32 (for the midpoint allowance)."""
    normed = O.rms_norm(x_pre, gain, eps).reshape(len(positions), heads, d)
    exact = O.rope_rotate(normed[None], positions, inv_freq, mscale)[0]
    mag = np.concatenate([np.abs(normed[..., :d // 2]) + np.abs(normed[..., d // 2:])] * 2, axis=-1)
    return exact, mag * mscale


def _assert_bf16_of(got, exact, mag, what):
    """got == bf16_round(exact) everywhere, except where the kernel's fp32
    arithmetic may round another way: got must then be the bfloat16
    rounding of some value within delta = 2^-20 mag of exact (mag: the sum
    of the two rotated terms' sizes, so delta covers the fp32 norm, sincos
    and rotation, whose errors stay near 2^-24 mag).  Where bfloat16 steps
    exceed delta this admits the neighbour only when exact lies within delta
    of their midpoint; a result much smaller than its terms (cancellation)
    has finer steps than delta and may sit a few of them away."""
    want = O.bf16_round(exact)
    diff = got != want
    n_diff = int(diff.sum())
    if n_diff:
        g, e, m = got[diff], exact[diff], mag[diff]
        _, e2 = np.frexp(np.abs(g))
        half_step = np.ldexp(1.0, np.maximum(e2 - 1, -126) - 8)
        bad = np.abs(e - g) > half_step + 2.0 ** -20 * m
        assert not bad.any(), (f"{what}: {int(bad.sum())} values beyond the fp32 rounding "
                               f"allowance; first got {g[bad][:3]} want {want[diff][bad][:3]} "
                               f"exact {e[bad][:3]} term size {m[bad][:3]}")
    assert n_diff <= max(8, exact.size // 2000), f"{what}: {n_diff} values off the nearest rounding"
    return n_diff


PROLOGUE_CASES = [
    # B, T, H, G, window, layer_type, yarn, pos_offset
    (2, 300, 8, 2, 100, 0, False, 0),
    (1, 513, 32, 8, 4096, 1, True, 0),
    (2, 200, 40, 8, 4096, 1, True, 60000),   # large angles: fp64 reduction before fp32 sincos
    (1, 1000, 8, 8, 4096, 0, False, 3000),
]


@pytest.mark.parametrize("case", PROLOGUE_CASES, ids=[str(c) for c in PROLOGUE_CASES])
def test_prologue_stage_rotated_rows(case):
    """The prologue alone (phase 1): rotated queries read back from the
    workspace's first region ([rows][H][d] bfloat16, times the MFMA
    kernel's base-2 softmax scale); then the rest of the call, and the
    rotated keys read from the cache slots the call wrote."""
    B, T, H, G, w, lt, yarn, P = case
    d, eps = 128, 1e-6
    kind = KINDS[lt]
    _log("prologue stage", case)
    rope = A.Rope(theta=500000.0, yarn=yarn, factor=8.0, orig_ctx=8192)
    x = inputs(79, lt, B, T, H, G, d, BF16)
    cap = w if lt == 0 else P + T
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.empty_like(x["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, lt, BF16, cap, "cuda")
    args = (x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc, out, ws)
    kw = dict(window=w, layer_type=lt, rope=rope, eps=eps, pos_offset=P)
    A.olmo3_attn_prefill(*args, phases=A.PHASE_PROLOGUE, **kw)
    torch.cuda.synchronize()
    q_rot = host(ws[:B * T * H * d * 2].view(BF16).reshape(B, T, H, d))
    # the rest of the call (a sliding layer's chunk after a prefix appends
    # its keys to the ring only after the attention has read it)
    A.olmo3_attn_prefill(*args, phases=A.PHASE_ATTENTION, **kw)
    torch.cuda.synchronize()
    inv_freq, mscale = O.layer_rope(oracle_rope(rope), kind, d)
    positions = P + np.arange(T)
    hq, hk = host(x["q_pre"]), host(x["k_pre"])
    qg, kg = host(x["q_gain"]), host(x["k_gain"])
    held = O.ring_positions(kind, w, cap, P + T)
    slots = np.array([int(np.nonzero(held == p)[0][0]) for p in positions if (held == p).any()])
    kept = np.array([p for p in positions if (held == p).any()])
    hkc = host(kc)
    total = 0
    for b in range(B):
        e, m = _rotated_ref(hq[b], qg, H, d, eps, positions, inv_freq, mscale)
        qs = prefill_q_scale(d)
        total += _assert_bf16_of(q_rot[b], e * qs, m * qs, f"queries of sequence {b}")
        e, m = _rotated_ref(hk[b], kg, G, d, eps, positions, inv_freq, mscale)
        sel = kept - P
        got = np.transpose(hkc[b][:, slots], (1, 0, 2))
        total += _assert_bf16_of(got, e[sel], m[sel], f"cached keys of sequence {b}")
    _log("  values off the nearest rounding", total)
