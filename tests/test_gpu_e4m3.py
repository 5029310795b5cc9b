"""e4m3 key/value caches: stored codes and decode outputs against the fp64
oracle, with scales that are not powers of two so that a scale applied twice
or not at all shows, and decode positions on both sides of the ring's window
boundary (the failure mode of quantized caches on sliding-window layers that
the page "Olmo 3 7B" records, "SERVICEABILITY JOIN").

Value codes are compared bit for bit: both sides decide them in fp32 from
the same bf16 input.  Key codes come from rotated keys that the kernel
computes in fp32 and the oracle in fp64, so a code may differ from the
oracle's by one step, and only where the key lies at a rounding midpoint."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import KINDS, assert_close, host, host_inputs, inputs, oracle_rope

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
KS, VS = 0.37, 1.9
TABLE = O.e4m3_values()


def _log(*a):
    print(*a, flush=True)


def _codes(t):
    return t.cpu().numpy()


def _key_x32(k_rot, scale):
    """The fp32 quantity whose nearest code is stored (as the kernel forms it)."""
    return np.asarray(k_rot, dtype=np.float32) * np.float32(1.0 / np.float64(scale))


def _check_key_codes(got, x32, what):
    want = O.e4m3_encode(x32)
    diff = got != want
    if not diff.any():
        return
    mid = (TABLE[got[diff]] + TABLE[want[diff]]) / 2
    x = x32[diff].astype(np.float64)
    assert (np.abs(x - mid) <= 1e-4 * np.abs(x) + 1e-6).all(), f"{what}: key codes off a midpoint differ"
    assert diff.mean() < 1e-3, f"{what}: {int(diff.sum())} key codes differ"


def _rotated_keys(hx, kind, rope, positions, G, d):
    w_, m_ = O.layer_rope(oracle_rope(rope), kind, d)
    B, T = hx["k_pre"].shape[:2]
    kh = O.rms_norm(hx["k_pre"], hx["k_gain"], 1e-6).reshape(B, T, G, d)
    return O.rope_rotate(kh, np.asarray(positions), w_, m_)


def _check_slots(kc, vc, before_k, before_v, slots, k_rot, v_new, what):
    """slots[j] holds position j of k_rot / v_new [B, n, G, d]; other slots keep their bytes."""
    gk, gv = _codes(kc), _codes(vc)
    slots = np.asarray(slots)
    got_v = gv[:, :, slots].transpose(0, 2, 1, 3)
    assert np.array_equal(got_v, O.e4m3_store(v_new, VS)), f"{what}: value codes"
    _check_key_codes(gk[:, :, slots].transpose(0, 2, 1, 3), _key_x32(k_rot, KS), what)
    rest = np.setdiff1d(np.arange(gk.shape[2]), slots)
    assert np.array_equal(gk[:, :, rest], before_k[:, :, rest]), f"{what}: key slot overwritten"
    assert np.array_equal(gv[:, :, rest], before_v[:, :, rest]), f"{what}: value slot overwritten"


@pytest.mark.parametrize("lt,T,pos_offset,cap", [(0, 50, 0, 16), (0, 5, 30, 16), (1, 50, 5, 60)])
def test_e4m3_append(lt, T, pos_offset, cap):
    B, G, d, w = 2, 2, 128, 16
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=4.0, orig_ctx=64)
    x = inputs(61, lt, B, T, G, G, d, BF16)
    kc, vc = synth.e4m3_cache_fill(61, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    A.olmo3_kv_append_e4m3(x["k_pre"], x["v"], x["k_gain"], kc, vc, k_scale=KS, v_scale=VS,
                           window=w, layer_type=lt, rope=rope, pos_offset=pos_offset)
    hx = host_inputs(x)
    positions = pos_offset + np.arange(T)
    keep = positions[-w:] if kind == O.SLIDING else positions
    idx = keep - pos_offset
    slots = keep % w if kind == O.SLIDING else keep
    k_rot = _rotated_keys(hx, kind, rope, positions, G, d)[:, idx]
    v_new = hx["v"].reshape(B, T, G, d)[:, idx]
    _check_slots(kc, vc, bk, bv, slots, k_rot, v_new, f"append {lt} {T} {pos_offset}")


PREFILL = [
    # B, T, H, G, window, layer_type, yarn
    (1, 300, 4, 4, 64, 0, False),
    (2, 129, 10, 2, 4096, 1, True),
    (1, 1000, 8, 8, 4096, 1, True),
    (2, 77, 4, 2, 100, 0, False),
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(c) for c in PREFILL])
def test_e4m3_prefill_vs_oracle(case):
    """The chunk attends to its own keys at bf16 precision and stores codes."""
    B, T, H, G, w, lt, yarn = case
    d = 128
    _log("e4m3 prefill", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=yarn, factor=8.0, orig_ctx=256)
    cap = w if kind == O.SLIDING else T + 3
    x = inputs(67, lt, B, T, H, G, d, BF16)
    kc, vc = synth.e4m3_cache_fill(67, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    out = torch.empty_like(x["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_prefill_e4m3(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                              out, ws, k_scale=KS, v_scale=VS, window=w, layer_type=lt, rope=rope)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d, e4m3_scales=(KS, VS))
    ref = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                        cache=ref_cache)
    err = assert_close(host(out), ref, what=f"e4m3 prefill {case}")
    _log("  max abs / rel err", err)
    positions = np.arange(T)
    keep = positions[-w:] if kind == O.SLIDING else positions
    slots = keep % w if kind == O.SLIDING else keep
    k_rot = _rotated_keys(hx, kind, rope, positions, G, d)[:, keep]
    _check_slots(kc, vc, bk, bv, slots, k_rot, hx["v"].reshape(B, T, G, d)[:, keep],
                 f"e4m3 prefill {case}")


CHUNKED = [
    # B, T, H, G, d, window, layer_type, pos_offset, yarn
    (1, 200, 4, 4, 128, 64, 0, 300, False),    # wrapped ring, chunk longer than the window
    (2, 40, 6, 2, 128, 100, 0, 30, False),     # ring partly filled
    (2, 77, 8, 2, 128, 128, 0, 250, False),    # wrapped ring, tiles cross the wrap
    (2, 129, 10, 2, 128, 4096, 1, 500, True),  # linear cache, group 5
    (1, 300, 8, 8, 128, 4096, 1, 1000, True),  # linear cache, MHA
    (1, 1, 4, 2, 128, 4096, 1, 77, True),      # one token
    (1, 50, 4, 2, 64, 40, 0, 77, False),       # plain kernel, ring
]


@pytest.mark.parametrize("case", CHUNKED, ids=[str(c) for c in CHUNKED])
def test_e4m3_chunked_prefill_vs_oracle(case):
    """A later chunk: earlier positions are read from the cache as stored
    (code times scale), the chunk's own keys and values at bf16 precision;
    the chunk's codes then land in their slots and no other slot changes."""
    B, T, H, G, d, w, lt, P, yarn = case
    _log("e4m3 chunked prefill", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=yarn, factor=8.0, orig_ctx=256)
    cap = w if kind == O.SLIDING else P + T + 3
    x = inputs(79, lt, B, T, H, G, d, BF16)
    kc, vc = synth.e4m3_cache_fill(79, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    out = torch.empty_like(x["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_prefill_e4m3(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                              out, ws, k_scale=KS, v_scale=VS, window=w, layer_type=lt, rope=rope,
                              pos_offset=P)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d, e4m3_scales=(KS, VS))
    ref_cache.k[:] = TABLE[bk] * KS
    ref_cache.v[:] = TABLE[bv] * VS
    ref_cache.pos[:] = O.ring_positions(kind, w, cap, P)
    ref = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                        pos_offset=P, cache=ref_cache)
    err = assert_close(host(out), ref, what=f"e4m3 chunked prefill {case}")
    _log("  max abs / rel err", err)
    positions = P + np.arange(T)
    keep = positions[-w:] if kind == O.SLIDING else positions
    slots = keep % w if kind == O.SLIDING else keep
    k_rot = _rotated_keys(hx, kind, rope, positions, G, d)[:, keep - P]
    _check_slots(kc, vc, bk, bv, slots, k_rot, hx["v"].reshape(B, T, G, d)[:, keep - P],
                 f"e4m3 chunked prefill {case}")


DECODE = [
    # B, H, G, window, layer_type, pos, cap
    *[(3, 8, 2, 128, 0, p, 128) for p in (0, 126, 127, 128, 129, 255, 256, 1000)],
    (2, 10, 2, 4096, 1, 399, 400),        # group 5, linear
    (4, 16, 2, 300, 0, 5000, 300),        # group 8
    (1, 4, 1, 4096, 1, 19999, 20000),     # 64 splits
    (2, 8, 8, 4096, 0, 4096, 4096),       # the 7B window, first wrap
    (1, 12, 2, 4096, 1, 2046, 3000),      # group 6, several splits, ragged last stage
    (2, 14, 2, 100, 0, 500, 100),         # group 7, ring of 100 slots
    (3, 40, 8, 4096, 0, 5000, 4096),      # the 32B grouping on the 7B window
    (1, 2, 2, 4096, 1, 9999, 10000),      # one query head per key/value head, 40 splits
    (3, 4, 4, 100, 0, 250, 100),          # one query head per key/value head, ring of 100
    (2, 3, 3, 4096, 1, 64, 200),          # 65 rows: one past a 64-row iteration
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_e4m3_decode_vs_oracle(case):
    B, H, G, w, lt, pos, cap = case
    d = 128
    _log("e4m3 decode", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    kc, vc = synth.e4m3_cache_fill(71, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    x = inputs(71, 10 + lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_decode_e4m3(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, k_scale=KS,
                             v_scale=VS, window=w, layer_type=lt, rope=rope, pos=pos)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d, e4m3_scales=(KS, VS))
    ref_cache.k[:] = TABLE[bk] * KS
    ref_cache.v[:] = TABLE[bv] * VS
    ref_cache.pos[:] = O.ring_positions(kind, w, cap, pos)
    ref = O.decode_e4m3_ref(hx["q_pre"][:, 0], hx["k_pre"][:, 0], hx["v"][:, 0], hx["q_gain"],
                            hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                            rope=oracle_rope(rope), pos=pos, cache=ref_cache)
    err = assert_close(host(out), ref, what=f"e4m3 decode {case}")
    _log("  max abs / rel err", err)
    slot = pos % w if kind == O.SLIDING else pos
    k_rot = _rotated_keys({"k_pre": hx["k_pre"], "k_gain": hx["k_gain"]}, kind, rope, [pos], G, d)
    _check_slots(kc, vc, bk, bv, [slot], k_rot, hx["v"].reshape(B, 1, G, d), f"e4m3 decode {case}")


ALL_CODES_DECODE = [
    # B, H, G, window, layer_type, pos, cap
    (3, 8, 8, 128, 0, 1000, 128),         # one query head per key/value head (per-row kernel)
    (2, 10, 2, 4096, 1, 2999, 3000),      # group 5 (grouped MFMA kernel), several splits
    (4, 16, 2, 300, 0, 299, 300),         # group 8, ring just filled
]


@pytest.mark.parametrize("case", ALL_CODES_DECODE, ids=[str(c) for c in ALL_CODES_DECODE])
def test_e4m3_decode_every_code(case):
    """Caches holding every non-NaN code equally often (zeros, subnormals down
    to 2^-9 and the largest magnitudes 0x7E / 0xFE = +-448 included): every
    code's value reaches the scores and the weighted sum as the oracle's
    table gives it.  Scales 1/64 (keys: scores stay moderate with keys up to
    7) and 1/16 (values)."""
    B, H, G, w, lt, pos, cap = case
    d, ks, vs = 128, 1.0 / 64, 1.0 / 16
    _log("e4m3 decode, every code", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    kc, vc = synth.e4m3_cache_fill(75, lt, B, G, cap, d, device="cuda", all_codes=True)
    bk, bv = _codes(kc), _codes(vc)
    for c in (0x00, 0x01, 0x07, 0x08, 0x7E, 0x80, 0x81, 0xFE):
        assert (bk == c).any() and (bv == c).any(), hex(c)
    assert not ((bk & 0x7F) == 0x7F).any() and not ((bv & 0x7F) == 0x7F).any()
    x = inputs(75, 10 + lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_decode_e4m3(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, k_scale=ks,
                             v_scale=vs, window=w, layer_type=lt, rope=rope, pos=pos)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d, e4m3_scales=(ks, vs))
    ref_cache.k[:] = TABLE[bk] * ks
    ref_cache.v[:] = TABLE[bv] * vs
    ref_cache.pos[:] = O.ring_positions(kind, w, cap, pos)
    # with keys up to 7 the scores' error from holding the rotated query in
    # bf16 grows with |k|, and values up to 28 carry it into the outputs: the
    # oracle rounds the rotated query as the kernel holds it
    ref = O.decode_e4m3_ref(hx["q_pre"][:, 0], hx["k_pre"][:, 0], hx["v"][:, 0], hx["q_gain"],
                            hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                            rope=oracle_rope(rope), pos=pos, cache=ref_cache, round_rotated=True)
    err = assert_close(host(out), ref, what=f"e4m3 decode every code {case}")
    _log("  max abs / rel err", err)


VALUE_CODES_DECODE = [
    # B, H, G, layer_type: one query head per key/value head (per-row kernel)
    # and groups of 5 (grouped MFMA kernel), ring and linear caches
    (2, 2, 2, 0), (2, 2, 2, 1), (2, 10, 2, 0), (2, 10, 2, 1),
]


@pytest.mark.parametrize("case", VALUE_CODES_DECODE, ids=[str(c) for c in VALUE_CODES_DECODE])
def test_e4m3_decode_returns_value_codes_exactly(case):
    """Decode at position 0: the new row is the only visible key, so its
    weight is exactly 1 and each query head's output is the value row as the
    kernel decodes it from its codes, times v_scale.  The values are every
    non-NaN code's value times v_scale = 1/16 (a power of two, so the codes
    and every product are exact): the output must equal them bit for bit,
    which pins the kernel's code -> value conversion for every code (an
    output compared within tolerance cannot see one code decoded wrongly)."""
    B, H, G, lt = case
    d, cap, w, vs = 128, 128, 128, 1.0 / 16
    _log("e4m3 decode, value codes exact", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.int64)
    rng = np.random.default_rng(77 + lt)
    picks = np.concatenate([rng.permutation(codes) for _ in range((B * G * d) // len(codes) + 1)])
    vrow = (TABLE[picks[: B * G * d]] * vs).reshape(B, G, d)
    x = inputs(77, 10 + lt, B, 1, H, G, d, BF16)
    v = torch.tensor(vrow, dtype=torch.float32).to(BF16).cuda()
    assert np.array_equal(host(v).astype(np.float64), vrow), "values not exact in bf16"
    kc, vc = synth.e4m3_cache_fill(77, lt, B, G, cap, d, device="cuda")
    q, k = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous()
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_decode_e4m3(q, k, v.reshape(B, G * d), x["q_gain"], x["k_gain"], kc, vc, out, ws,
                             k_scale=KS, v_scale=vs, window=w, layer_type=lt, rope=rope, pos=0)
    got = host(out).astype(np.float64).reshape(B, H, d)
    want = vrow[:, np.arange(H) // (H // G), :]
    bad = got != want
    assert not bad.any(), (f"{int(bad.sum())} outputs differ; first codes "
                           f"{[hex(int(c)) for c in picks[: B * G * d].reshape(B, G, d)[:, np.arange(H) // (H // G), :][bad][:8]]}")
    assert np.array_equal(_codes(vc)[:, :, 0, :], picks[: B * G * d].reshape(B, G, d)), "stored value codes"


@pytest.mark.parametrize("lt", [0, 1])
def test_e4m3_append_saturates_and_keeps_nan(lt):
    """Scales so small (keys 1/512, values 1/1024) that most |x / scale|
    exceed 448: those store the saturated codes 0x7E / 0xFE, bit for bit as
    the interface's rule (``e4m3_store``) gives them; a NaN planted in one
    value element and in one token's projected key (whose norm then makes
    that token's whole key row NaN) is stored as a NaN code."""
    B, T, G, d, w, cap = 2, 40, 2, 128, 16, 48
    ks, vs = 1.0 / 512, 1.0 / 1024
    kind = KINDS[lt]
    cap = w if lt == 0 else cap
    rope = A.Rope(theta=500000.0, yarn=True, factor=4.0, orig_ctx=64)
    x = inputs(77, lt, B, T, G, G, d, BF16)
    t_nan_v, t_nan_k = T - 3, T - 5
    x["v"][1, t_nan_v, 7] = float("nan")
    x["k_pre"][0, t_nan_k, 130] = float("nan")
    kc, vc = synth.e4m3_cache_fill(77, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    A.olmo3_kv_append_e4m3(x["k_pre"], x["v"], x["k_gain"], kc, vc, k_scale=ks, v_scale=vs,
                           window=w, layer_type=lt, rope=rope)
    hx = host_inputs(x)
    positions = np.arange(T)
    keep = positions[-w:] if kind == O.SLIDING else positions
    slots = keep % w if kind == O.SLIDING else keep
    gk, gv = _codes(kc), _codes(vc)
    got_v = gv[:, :, slots].transpose(0, 2, 1, 3)
    want_v = O.e4m3_store(hx["v"].reshape(B, T, G, d)[:, keep], vs)
    nan_v = (want_v & 0x7F) == 0x7F
    assert nan_v.sum() == 1 and ((got_v[nan_v] & 0x7F) == 0x7F).all(), "value NaN code"
    assert np.array_equal(got_v[~nan_v], want_v[~nan_v]), "value codes"
    sat = (want_v[~nan_v] & 0x7F) == 0x7E
    assert sat.mean() > 0.5, sat.mean()
    k_rot = _rotated_keys(hx, kind, rope, positions, G, d)[:, keep]
    got_k = gk[:, :, slots].transpose(0, 2, 1, 3)
    x32 = _key_x32(k_rot, ks)
    nan_k = np.isnan(x32)
    assert nan_k.sum() == G * d and ((got_k[nan_k] & 0x7F) == 0x7F).all(), "key NaN codes"
    want_k = O.e4m3_encode(x32[~nan_k])
    assert ((want_k & 0x7F) == 0x7E).mean() > 0.25
    _check_key_codes(got_k[~nan_k], x32[~nan_k], f"saturating append {lt}")
    rest = np.setdiff1d(np.arange(cap), slots)
    assert np.array_equal(gk[:, :, rest], bk[:, :, rest]) and np.array_equal(gv[:, :, rest], bv[:, :, rest])


@pytest.mark.parametrize("lt,w,pos,back", [
    (0, 128, 127, 127), (0, 128, 128, 127), (0, 128, 129, 127), (0, 128, 401, 127),
    (0, 128, 128, 128), (0, 128, 401, 128),      # the evicted position: its slot holds the new token
    (0, 128, 300, 0), (1, 128, 300, 300), (1, 128, 300, 0), (1, 128, 300, 1)])
def test_e4m3_window_edge_planted_value(lt, w, pos, back):
    """q = 0 makes the weights uniform over the rows the decode reads.  Every
    value code is 0 except one planted at the slot of position pos - back, and
    the new token's value is 0, so each output is exactly v_scale * 2 / n when
    the planted row is read (n = min(pos+1, w) on the ring, pos+1 on the
    linear cache) and 0 when its slot now holds the new token: this fixes the
    window edge and that v_scale is applied once."""
    B, H, G, d = 2, 4, 2, 128
    kind = KINDS[lt]
    cap = w if lt == 0 else pos + 1
    kc, _ = synth.e4m3_cache_fill(73, lt, B, G, cap, d, device="cuda")
    vc = torch.zeros_like(kc)
    p_star = pos - back
    vc[:, :, p_star % cap] = 0x40  # code 0x40 = 2.0
    x = inputs(73, lt, B, 1, H, G, d, BF16)
    q = torch.zeros_like(x["q_pre"][:, 0])
    k = x["k_pre"][:, 0].contiguous()
    v = torch.zeros_like(x["v"][:, 0])
    out = torch.empty_like(q)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    A.olmo3_attn_decode_e4m3(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws, k_scale=KS,
                             v_scale=VS, window=w, layer_type=lt, rope=A.Rope(), pos=pos)
    got = host(out)
    n = min(pos + 1, w) if lt == 0 else pos + 1
    overwritten = p_star % cap == pos % cap  # the new token (value 0) took the slot
    want = 0.0 if overwritten else 2.0 * VS / n
    assert_close(got, np.full_like(got, want), 0.0, 2.0 ** -8, f"planted {lt} {pos} {back}")


RAGGED_PREFILL = [
    # H, G, window, layer_type, lengths
    (8, 2, 64, 0, [100, 37, 200]),     # ring shorter than two of the prompts
    (10, 2, 4096, 1, [129, 1, 300]),   # linear caches, group 5, a one-token prompt
    (4, 4, 4096, 0, [64, 65]),         # one query head per key/value head
]


@pytest.mark.parametrize("case", RAGGED_PREFILL, ids=[str(c) for c in RAGGED_PREFILL])
def test_e4m3_ragged_first_chunks_vs_oracle(case):
    """Prompts of different lengths packed row after row into e4m3 caches:
    each prompt matches the oracle's e4m3 prefill of that prompt alone, its
    kept positions hold their codes, and no other slot changes."""
    H, G, w, lt, lengths = case
    B, d = len(lengths), 128
    _log("e4m3 ragged first chunks", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=256)
    n = sum(lengths)
    max_len = max(lengths)
    cap = w if kind == O.SLIDING else max_len + 3
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = inputs(89, lt, 1, n, H, G, d, BF16)
    flat = {k: (t[0] if t.dim() == 3 else t) for k, t in x.items()}
    kc, vc = synth.e4m3_cache_fill(89, lt, B, G, cap, d, device="cuda")
    bk, bv = _codes(kc), _codes(vc)
    out = torch.empty_like(flat["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, 1, n, H, G, d, lt, A.DTYPE_BF16_E4M3, 0, "cuda")
    A.olmo3_attn_prefill_ragged_e4m3(flat["q_pre"], flat["k_pre"], flat["v"], flat["q_gain"],
                                     flat["k_gain"], kc, vc, out, ws,
                                     torch.tensor(cu, device="cuda"), k_scale=KS, v_scale=VS,
                                     max_len=max_len, window=w, layer_type=lt, rope=rope)
    hx = host_inputs(x)
    got = host(out)
    gk, gv = _codes(kc), _codes(vc)
    for b in range(B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        T = r1 - r0
        seq = {k: (v[:, r0:r1] if v.ndim == 3 else v) for k, v in hx.items()}
        ref_cache = O.KvCacheRef(kind, w, cap, 1, G, d, e4m3_scales=(KS, VS))
        ref = O.prefill_ref(**seq, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                            cache=ref_cache)
        assert_close(got[r0:r1][None], ref, what=f"prompt {b} ({T} tokens)")
        positions = np.arange(T)
        keep = positions[-w:] if kind == O.SLIDING else positions
        slots = keep % w if kind == O.SLIDING else keep
        k_rot = _rotated_keys(seq, kind, rope, positions, G, d)[0, keep]          # [n_keep, G, d]
        v_new = seq["v"][0].reshape(T, G, d)[keep]
        assert np.array_equal(gv[b][:, slots].transpose(1, 0, 2), O.e4m3_store(v_new, VS)), \
            f"prompt {b}: value codes"
        _check_key_codes(gk[b][:, slots].transpose(1, 0, 2), _key_x32(k_rot, KS), f"prompt {b}")
        rest = np.setdiff1d(np.arange(cap), slots)
        assert np.array_equal(gk[b][:, rest], bk[b][:, rest]), f"prompt {b}: key slot overwritten"
        assert np.array_equal(gv[b][:, rest], bv[b][:, rest]), f"prompt {b}: value slot overwritten"


@pytest.mark.parametrize("lt", [0, 1])
def test_e4m3_ragged_serving_flow(lt):
    """Prompts of different lengths ingested together, then four decode steps
    in which every sequence advances from its own position: each sequence's
    outputs follow the oracle's e4m3 cache flow (prefill, then one decode per
    step, the cache holding codes throughout)."""
    H, G, d, w = 8, 2, 128, 64
    lengths = [70, 3, 40]
    B = len(lengths)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=256)
    steps = 4
    cap = w if kind == O.SLIDING else max(lengths) + steps
    n = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = inputs(97, lt, 1, n, H, G, d, BF16)
    flat = {k: (t[0] if t.dim() == 3 else t) for k, t in x.items()}
    kc = torch.zeros((B, G, cap, d), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.empty_like(flat["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, 1, n, H, G, d, lt, A.DTYPE_BF16_E4M3, 0, "cuda")
    A.olmo3_attn_prefill_ragged_e4m3(flat["q_pre"], flat["k_pre"], flat["v"], flat["q_gain"],
                                     flat["k_gain"], kc, vc, out, ws,
                                     torch.tensor(cu, device="cuda"), k_scale=KS, v_scale=VS,
                                     max_len=max(lengths), window=w, layer_type=lt, rope=rope)
    hx = host_inputs(x)
    refs = []
    for b in range(B):
        seq = {k: (v[:, cu[b]:cu[b + 1]] if v.ndim == 3 else v) for k, v in hx.items()}
        c = O.KvCacheRef(kind, w, cap, 1, G, d, e4m3_scales=(KS, VS))
        ref = O.prefill_ref(**seq, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                            cache=c)
        assert_close(host(out)[cu[b]:cu[b + 1]][None], ref, what=f"prefill of prompt {b}")
        refs.append(c)
    wsd = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, A.DTYPE_BF16_E4M3, cap, "cuda")
    for step in range(steps):
        xs = inputs(97, 50 + step, B, 1, H, G, d, BF16)
        q, k, v = (xs[key][:, 0].contiguous() for key in ("q_pre", "k_pre", "v"))
        positions = [L + step for L in lengths]
        dout = torch.empty_like(q)
        A.olmo3_attn_decode_ragged_e4m3(q, k, v, flat["q_gain"], flat["k_gain"], kc, vc, dout, wsd,
                                        torch.tensor(positions, dtype=torch.int32, device="cuda"),
                                        k_scale=KS, v_scale=VS, max_pos=max(positions), window=w,
                                        layer_type=lt, rope=rope)
        hq = host_inputs(xs)
        got = host(dout)
        for b, p in enumerate(positions):
            ref = O.decode_e4m3_ref(hq["q_pre"][b:b + 1, 0], hq["k_pre"][b:b + 1, 0],
                                    hq["v"][b:b + 1, 0], hx["q_gain"], hx["k_gain"], H=H, G=G,
                                    d=d, kind=kind, window=w, rope=oracle_rope(rope), pos=p,
                                    cache=refs[b])
            assert_close(got[b:b + 1], ref, what=f"step {step}, sequence {b} at {p}")
