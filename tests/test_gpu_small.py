"""GPU parity at sizes the oracle evaluates whole: every output element and
every written cache slot is compared with the fp64 oracle on the same seeded
inputs.  Index work (mask, cache slots, decode rows) is compared bit for bit
through the probes and through planted values."""

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


def _check_cache(k_cache, v_cache, ref_cache, slots, what, atol=2e-2, rtol=1e-2):
    """Slots written by the call: v bit-exact, k within tolerance."""
    kc, vc = host(k_cache), host(v_cache)
    slots = np.asarray(slots)
    assert np.array_equal(vc[:, :, slots], ref_cache.v[:, :, slots]), f"{what}: v slots differ"
    assert_close(kc[:, :, slots], ref_cache.k[:, :, slots], atol, rtol, f"{what}: k slots")


# --------------------------------------------------------------- toy config
def test_toy_config_prefill_then_decode():
    """fp32, seed 0: B=1, T=64, H=2, G=1, d=16, layers s,s,s,f, window 16,
    theta 1e4, no YaRN; prefill 64 tokens then decode 8 more per layer."""
    B, T, H, G, d, w, n_dec = 1, 64, 2, 1, 16, 16, 8
    rope = A.Rope(theta=10000.0, yarn=False)
    kinds = O.layer_types(4)
    for layer, kind in enumerate(kinds):
        lt = O.layer_type_code(kind)
        assert A.olmo3_layer_type(layer, 4) == lt
        _log(f"toy layer {layer} {kind}")
        x = inputs(0, layer, B, T + n_dec, H, G, d, F32)
        cap = w if kind == O.SLIDING else T + n_dec
        kc = torch.zeros((B, G, cap, d), dtype=F32, device="cuda")
        vc = torch.zeros_like(kc)
        pre = {k: (v[:, :T].contiguous() if v.dim() == 3 else v) for k, v in x.items()}
        out = gpu_prefill(pre, kc, vc, window=w, layer_type=lt, rope=rope, H=H)
        hx = host_inputs(x)
        ref_cache = O.KvCacheRef(kind, w, cap, B, G, d)
        hpre = {k: (v[:, :T] if v.ndim == 3 else v) for k, v in hx.items()}
        ref = O.prefill_ref(**hpre, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                            cache=ref_cache)
        err = assert_close(host(out), ref, ATOL_F32, RTOL_F32, f"toy prefill layer {layer}")
        _log("  prefill max err", err)
        _check_cache(kc, vc, ref_cache, np.nonzero(ref_cache.pos >= 0)[0], f"toy layer {layer}",
                     ATOL_F32, RTOL_F32)
        for p in range(T, T + n_dec):
            o = gpu_decode(x["q_pre"][:, p].contiguous(), x["k_pre"][:, p].contiguous(),
                           x["v"][:, p].contiguous(), x["q_gain"], x["k_gain"], kc, vc,
                           window=w, layer_type=lt, rope=rope, pos=p, H=H)
            r = O.decode_ref(hx["q_pre"][:, p], hx["k_pre"][:, p], hx["v"][:, p], hx["q_gain"],
                             hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                             rope=oracle_rope(rope), pos=p, cache=ref_cache)
            assert_close(host(o), r, ATOL_F32, RTOL_F32, f"toy decode layer {layer} pos {p}")
        _check_cache(kc, vc, ref_cache, np.nonzero(ref_cache.pos >= 0)[0],
                     f"toy layer {layer} after decode", ATOL_F32, RTOL_F32)


# ---------------------------------------------------------- bf16 prefill
PREFILL_CASES = [
    # B, T, H, G, d, window, layer_type, yarn
    (1, 300, 4, 4, 128, 64, 0, False),     # MHA, ragged tail, window < query block
    (2, 700, 10, 2, 128, 200, 0, False),   # GQA, 5 query heads per key/value head
    (1, 513, 4, 1, 128, 1000, 0, False),   # window > T: plain causal
    (2, 389, 4, 2, 128, 1, 0, False),      # window 1: each token sees itself only
    (1, 1000, 8, 8, 128, 4096, 1, True),   # full layer with YaRN
    (2, 129, 6, 3, 128, 4096, 1, False),   # full, one query past a block edge
    (1, 1, 4, 2, 128, 16, 0, False),       # single token
    (1, 1, 4, 2, 128, 16, 1, True),
    (1, 200, 4, 2, 64, 32, 0, False),      # d = 64 (plain kernel)
    (2, 150, 2, 1, 32, 4096, 1, True),     # d = 32, full, YaRN
    (1, 77, 3, 1, 16, 9, 0, False),        # d = 16 bf16
    (1, 130, 64, 64, 128, 64, 0, False),   # 64 heads: the prologue's head limit
    (1, 600, 64, 8, 128, 4096, 1, True),   # group 8 with 64 query heads, full
    (3, 2100, 2, 1, 128, 256, 0, False),   # 6,300 rows: the one-wavefront-per-token prologue
    # 16 query blocks x 32 heads = 512 workgroups: the unsplit instance, with
    # the query blocks of 4 heads per XCD interleaved (grouped heads; full
    # layers), or the 10 full-window blocks of each head first, head after
    # head, and the rest interleaved (one query head per key/value head,
    # sliding)
    (1, 2048, 32, 8, 128, 700, 0, False),
    (1, 2048, 32, 8, 128, 4096, 1, True),
    (1, 2048, 32, 32, 128, 700, 0, False),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_prefill_bf16_vs_oracle(case):
    B, T, H, G, d, w, lt, yarn = case
    _log("prefill case", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=yarn, factor=8.0, orig_ctx=256)
    x = inputs(11, lt, B, T, H, G, d, BF16)
    cap = w if kind == O.SLIDING else T + 3
    kc = torch.full((B, G, cap, d), 7.0, dtype=BF16, device="cuda")
    vc = torch.full_like(kc, -7.0)
    out = gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=rope, H=H)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d)
    ref_cache.k[:] = 7.0
    ref_cache.v[:] = -7.0
    ref = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                        cache=ref_cache)
    err = assert_close(host(out), ref, what=f"prefill {case}")
    _log("  max abs / rel err", err)
    written = np.nonzero(ref_cache.pos >= 0)[0]
    _check_cache(kc, vc, ref_cache, written, f"prefill {case}")
    untouched = np.nonzero(ref_cache.pos < 0)[0]
    if untouched.size:
        assert (host(kc)[:, :, untouched] == 7.0).all() and (host(vc)[:, :, untouched] == -7.0).all()


# ----------------------------------------------------------- bf16 decode
DECODE_CASES = [
    # B, H, G, d, window, layer_type, pos, cap
    (3, 8, 2, 128, 128, 0, 0, 128),
    (3, 8, 2, 128, 128, 0, 50, 128),
    (3, 8, 2, 128, 128, 0, 127, 128),
    (3, 8, 2, 128, 128, 0, 128, 128),      # first wrap of the ring
    (3, 8, 2, 128, 128, 0, 1000, 128),
    (2, 10, 2, 128, 4096, 1, 399, 400),
    (2, 10, 2, 128, 4096, 1, 0, 400),
    (1, 4, 1, 128, 4096, 1, 19999, 20000),  # 64 splits
    (4, 16, 2, 128, 300, 0, 5000, 300),     # group 8
    (2, 4, 2, 128, 4096, 1, 777, 1000),     # group 2
    (2, 6, 2, 128, 256, 0, 300, 256),       # group 3
    (1, 12, 2, 128, 4096, 1, 2048, 3000),   # group 6
    (2, 14, 2, 128, 100, 0, 500, 100),      # group 7
    (2, 6, 2, 64, 64, 0, 100, 64),          # plain kernel
    (2, 6, 6, 32, 4096, 1, 70, 100),
    (2, 64, 64, 128, 256, 0, 700, 256),     # 64 heads: the decode prologue's 1,536 pair chunks
    (3, 64, 8, 128, 4096, 1, 300, 301),     # group 8 with 64 query heads
    (5, 1, 1, 128, 64, 0, 63, 64),          # a single head
    # the last position a decode takes (2^40 - 1), on rings
    (3, 8, 8, 128, 4096, 0, (1 << 40) - 1, 4096),
    (2, 10, 2, 128, 256, 0, (1 << 40) - 1, 256),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_decode_bf16_vs_oracle(case):
    B, H, G, d, w, lt, pos, cap = case
    _log("decode case", case)
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=512)
    kc, vc = synth.cache_fill(13, lt, B, G, cap, d, device="cuda", dtype=BF16)
    tags = O.ring_positions(kind, w, cap, pos)
    hk, hv = host(kc), host(vc)
    x = inputs(13, 10 + lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    out = gpu_decode(q, k, v, x["q_gain"], x["k_gain"], kc, vc, window=w, layer_type=lt,
                     rope=rope, pos=pos, H=H)
    hx = host_inputs(x)
    ref_cache = O.KvCacheRef(kind, w, cap, B, G, d)
    ref_cache.k[:] = hk
    ref_cache.v[:] = hv
    ref_cache.pos[:] = tags
    ref = O.decode_ref(hx["q_pre"][:, 0], hx["k_pre"][:, 0], hx["v"][:, 0], hx["q_gain"],
                       hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                       pos=pos, cache=ref_cache)
    err = assert_close(host(out), ref, what=f"decode {case}")
    _log("  max abs / rel err", err)
    slot = pos % w if kind == O.SLIDING else pos
    _check_cache(kc, vc, ref_cache, [slot], f"decode {case}")
    others = np.setdiff1d(np.arange(cap), [slot])
    assert np.array_equal(host(kc)[:, :, others], hk[:, :, others])
    assert np.array_equal(host(vc)[:, :, others], hv[:, :, others])


def test_prefill_then_decodes_match_longer_prefill():
    """prefill(T0) + decodes of positions T0..T-1 equal the last rows of
    prefill(T) (both through the GPU, each checked against the oracle)."""
    B, T0, T, H, G, d, w = 2, 190, 200, 8, 4, 128, 64
    rope = A.Rope(theta=500000.0)
    x = inputs(17, 0, B, T, H, G, d, BF16)
    hx = host_inputs(x)
    for lt in (0, 1):
        kind = KINDS[lt]
        cap = w if lt == 0 else T
        kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
        vc = torch.zeros_like(kc)
        ref_all = O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope))
        pre = {k: (v[:, :T0].contiguous() if v.dim() == 3 else v) for k, v in x.items()}
        out = gpu_prefill(pre, kc, vc, window=w, layer_type=lt, rope=rope, H=H)
        assert_close(host(out), ref_all[:, :T0], what=f"prefix {kind}")
        for p in range(T0, T):
            o = gpu_decode(x["q_pre"][:, p].contiguous(), x["k_pre"][:, p].contiguous(),
                           x["v"][:, p].contiguous(), x["q_gain"], x["k_gain"], kc, vc,
                           window=w, layer_type=lt, rope=rope, pos=p, H=H)
            assert_close(host(o), ref_all[:, p], what=f"decode {kind} pos {p}")


# ------------------------------------------------------------- kv append
@pytest.mark.parametrize("lt,T,pos_offset,cap", [(0, 50, 0, 16), (0, 5, 30, 16), (1, 50, 5, 60)])
def test_kv_append(lt, T, pos_offset, cap):
    """Ring collisions keep the last `window` positions; untouched slots keep
    their bytes; values are copied bit for bit; keys are rotated at their
    absolute positions."""
    B, G, d, w = 2, 2, 128, 16
    kind = KINDS[lt]
    rope = A.Rope(theta=500000.0, yarn=True, factor=4.0, orig_ctx=64)
    x = inputs(19, lt, B, T, G, G, d, BF16)
    kc = torch.full((B, G, cap, d), 3.0, dtype=BF16, device="cuda")
    vc = torch.full_like(kc, -3.0)
    A.olmo3_kv_append(x["k_pre"], x["v"], x["k_gain"], kc, vc, window=w, layer_type=lt,
                      rope=rope, pos_offset=pos_offset)
    hx = host_inputs(x)
    ref = O.KvCacheRef(kind, w, cap, B, G, d)
    ref.k[:] = 3.0
    ref.v[:] = -3.0
    wr, m = O.layer_rope(oracle_rope(rope), kind, d)
    kh = O.rms_norm(hx["k_pre"], hx["k_gain"], 1e-6).reshape(B, T, G, d)
    positions = pos_offset + np.arange(T)
    ref.append(O.rope_rotate(kh, positions, wr, m), hx["v"].reshape(B, T, G, d), positions)
    written = np.nonzero(ref.pos >= 0)[0]
    _check_cache(kc, vc, ref, written, f"append {lt} {T} {pos_offset}")
    rest = np.nonzero(ref.pos < 0)[0]
    assert (host(kc)[:, :, rest] == 3.0).all() and (host(vc)[:, :, rest] == -3.0).all()


# ----------------------------------------------------------------- probes
@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("T", [1, 5, 64, 127, 128, 129, 300, 1000, 4096])
@pytest.mark.parametrize("window", [1, 2, 63, 64, 100, 128, 4096])
def test_probe_prefill_visits_bit_exact(T, window, splits):
    """Every visible pair is accumulated exactly once (counts, not flags:
    a tile taken twice, or by both workgroups of a split block, reads 2),
    and no other pair."""
    for lt in (0, 1):
        got = A.olmo3_probe_prefill_visits(T, window, lt, kv_splits=splits).cpu().numpy()
        want = O.sliding_window_mask(T, window) if lt == 0 else O.causal_mask(T)
        assert np.array_equal(got, want), (T, window, lt, np.argwhere(got != want)[:5])


# (B, H, G, ...): H = G is the per-row kernel's walk, H/G >= 2 with bf16 caches
# the grouped MFMA kernel's, with e4m3 caches the per-row kernel's again
@pytest.mark.parametrize("B,H,G,window,lt,pos,cap,dtype", [
    (32, 32, 32, 4096, 0, 65535, 4096, 0), (32, 32, 32, 4096, 1, 65535, 65536, 0),
    (64, 40, 8, 4096, 0, 32767, 4096, 0), (64, 40, 8, 4096, 1, 32767, 32768, 0),
    (64, 40, 8, 4096, 0, 32767, 4096, 2), (64, 40, 8, 4096, 1, 32767, 32768, 2),
    (1, 1, 1, 4096, 0, 10, 4096, 0), (1, 1, 1, 4096, 1, 0, 1, 0), (1, 2, 1, 4096, 1, 0, 1, 0),
    (1, 8, 4, 4096, 1, 19999, 20000, 0), (3, 6, 2, 128, 0, 127, 128, 0), (3, 6, 2, 128, 0, 128, 128, 0),
    (2, 40, 8, 4096, 1, 100, 1000, 0), (5, 14, 2, 4096, 1, 1000, 1001, 0),
])
def test_probe_decode_reads_each_held_slot_once(B, H, G, window, lt, pos, cap, dtype):
    got = A.olmo3_probe_decode_reads(B, H, G, 128, window, lt, pos, cap, dtype=dtype).cpu().numpy()
    kind = KINDS[lt]
    n = O.cache_entries(kind, window, pos + 1)
    assert n == (min(pos + 1, window) if lt == 0 else pos + 1)
    want = np.zeros(cap, dtype=np.int32)
    want[:n] = 1
    assert np.array_equal(got, want)


# ------------------------------------------------------- planted values
@pytest.mark.parametrize("lt,T,w,s_star", [(0, 700, 200, 250), (0, 4500, 4096, 100), (1, 700, 4096, 250)])
def test_planted_value_window_edges(lt, T, w, s_star):
    """q = 0 makes attention uniform over the visible keys; one value row
    planted at 1024 shows up as exactly 1024/n in rows that see it and as
    exactly 0 elsewhere, which fixes both window edges bit for bit."""
    B, H, G, d = 1, 4, 2, 128
    kind = KINDS[lt]
    x = inputs(23, lt, B, T, H, G, d, BF16)
    x["q_pre"].zero_()
    x["v"].zero_()
    x["v"][:, s_star] = 1024.0
    cap = w if lt == 0 else T
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    out = host(gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=A.Rope(), H=H))[0]
    t = np.arange(T)
    sees = O.mask_at_positions(t, np.array([s_star]), kind, w)[:, 0]
    n = np.array([O.mask_at_positions(np.array([ti]), t, kind, w).sum() for ti in t])
    assert (out[~sees] == 0.0).all(), np.nonzero((out[~sees] != 0).any(axis=1))
    want = (1024.0 / n[sees])[:, None] * np.ones((1, H * d))
    assert_close(out[sees], want, 0.0, 2 ** -8, "planted rows")


WHOLE_VS_PHASES = [
    # B, H, G, window, layer_type, pos, cap, e4m3
    (3, 8, 8, 128, 0, 500, 128, False),        # per-row kernel, one query head per group
    (2, 40, 8, 4096, 1, 19999, 20001, False),  # grouped MFMA kernel, group 5, many splits
    (2, 8, 2, 4096, 1, 5000, 5002, True),      # e4m3 caches, group 4
    (1, 4, 4, 64, 0, 3, 64, False),            # four rows: one split
]


@pytest.mark.parametrize("case", WHOLE_VS_PHASES, ids=[str(c) for c in WHOLE_VS_PHASES])
def test_decode_whole_call_equals_phases(case):
    """A whole decode call and the three phase entry points run one after the
    other give the same bits, for each decode kernel, on two calls in a row
    that share one workspace which starts as 0xff bytes (nothing may depend
    on its contents on entry)."""
    B, H, G, w, lt, pos, cap, e4m3 = case
    d = 128
    _log("whole call vs phases", case)
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=512)
    kw = dict(window=w, layer_type=lt, rope=rope)
    if e4m3:
        kc0, vc0 = synth.e4m3_cache_fill(83, lt, B, G, cap, d, device="cuda")
        decode, dt, kw = A.olmo3_attn_decode_e4m3, A.DTYPE_BF16_E4M3, dict(kw, k_scale=0.37, v_scale=1.9)
    else:
        kc0, vc0 = synth.cache_fill(83, lt, B, G, cap, d, device="cuda")
        decode, dt = A.olmo3_attn_decode, BF16
    xs = [inputs(83, 30 + i, B, 1, H, G, d, BF16) for i in range(2)]
    toks = [(x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous(),
             x["q_gain"], x["k_gain"]) for x in xs]
    results = []
    for phased in (False, True):
        kc, vc = kc0.clone(), vc0.clone()
        ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, dt, cap, "cuda")
        ws.fill_(255)
        outs = []
        for i, (q, k, v, qg, kg) in enumerate(toks):
            out = torch.empty_like(q)
            args = (q, k, v, qg, kg, kc, vc, out, ws)
            if phased:
                for ph in (A.PHASE_PROLOGUE, A.PHASE_ATTENTION, A.PHASE_MERGE):
                    decode(*args, pos=pos + i, phases=ph, **kw)
            else:
                decode(*args, pos=pos + i, **kw)
            outs.append(out)
        torch.cuda.synchronize()
        results.append([o.clone() for o in outs] + [kc.clone(), vc.clone()])
    for a_, b_ in zip(*results):
        assert torch.equal(a_, b_)
    assert torch.isfinite(results[0][0].float()).all()


def test_phase_entry_points_equal_one_call():
    """Running the stages one by one gives bit-identical outputs and caches."""
    B, T, H, G, d, w = 1, 333, 8, 2, 128, 100
    rope = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=128)
    x = inputs(29, 0, B, T, H, G, d, BF16)
    for lt in (0, 1):
        cap = w if lt == 0 else T + 1
        outs = []
        for phased in (False, True):
            kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
            vc = torch.zeros_like(kc)
            out = torch.empty_like(x["q_pre"])
            ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, lt, BF16, cap, "cuda")
            kw = dict(window=w, layer_type=lt, rope=rope)
            if phased:
                A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                                     out, ws, phases=A.PHASE_PROLOGUE, **kw)
                A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                                     out, ws, phases=A.PHASE_ATTENTION, **kw)
            else:
                A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                                     out, ws, **kw)
            dq = synth.normal((2, H * d), 31, lt, 1, device="cuda")
            dk = synth.normal((2, G * d), 31, lt, 2, device="cuda")
            kc2 = kc.expand(2, -1, -1, -1).contiguous()
            vc2 = vc.expand(2, -1, -1, -1).contiguous()
            dout = torch.empty_like(dq)
            wsd = A.workspace(A.MODE_DECODE, 2, 1, H, G, d, lt, BF16, cap, "cuda")
            dargs = (dq, dk, dk.clone(), x["q_gain"], x["k_gain"], kc2, vc2, dout, wsd)
            pos = T if lt == 1 else T + 50
            if phased:
                for ph in (A.PHASE_PROLOGUE, A.PHASE_ATTENTION, A.PHASE_MERGE):
                    A.olmo3_attn_decode(*dargs, pos=pos, phases=ph, **kw)
            else:
                A.olmo3_attn_decode(*dargs, pos=pos, **kw)
            torch.cuda.synchronize()
            outs.append((out.clone(), kc.clone(), vc.clone(), dout.clone(), kc2.clone()))
        for a_, b_ in zip(outs[0], outs[1]):
            assert torch.equal(a_, b_)
