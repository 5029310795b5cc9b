"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on outputs the oracle computes one by one: sampled query
rows (including both window edges and the block edges) for sampled
key/value heads, and sampled sequences for decode.  Cache slots written by
the call are checked at the sampled heads."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import KINDS, assert_close, gpu_decode, gpu_prefill, host, inputs, oracle_rope

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
W = 4096
YARN = A.Rope(theta=500000.0, yarn=True, factor=8.0, orig_ctx=8192)
PLAIN = A.Rope(theta=500000.0)


def _log(*a):
    print(*a, flush=True)


def _sample_rows(T, seed, n_random=20):
    edges = [0, 1, 63, 64, 127, 128, W - 1, W, W + 1, T // 2, T - 2, T - 1]
    rng = np.random.default_rng(seed)
    rows = set(r for r in edges if 0 <= r < T) | set(rng.integers(0, T, n_random).tolist())
    return np.array(sorted(rows))


def _check_prefill_rows(x, out, kc, vc, *, T, H, G, d, lt, rope, kv_heads, seed, what):
    kind = KINDS[lt]
    rows = _sample_rows(T, seed)
    q_rows = host(x["q_pre"][0, rows])
    k_all = host(x["k_pre"][0])
    v_all = host(x["v"][0]).reshape(T, G, d)
    qg, kg = host(x["q_gain"]), host(x["k_gain"])
    ref = O.attention_rows_ref(q_rows, rows, k_all, v_all, np.arange(T), qg, kg, H=H, G=G, d=d,
                               kv_heads=kv_heads, kind=kind, window=W, rope=oracle_rope(rope))
    group = H // G
    heads = [g * group + j for g in kv_heads for j in range(group)]
    got = host(out[0, rows]).reshape(len(rows), H, d)[:, heads]
    err = assert_close(got, ref, what=what)
    _log(f"  {what}: {len(rows)} rows x {len(heads)} heads, max abs/rel err {err}")
    # cache slots of the sampled heads: keys rotated at their positions, values copied
    w_, m_ = O.layer_rope(oracle_rope(rope), kind, d)
    held = np.arange(T - W, T) if kind == O.SLIDING else np.arange(T)
    pick = np.random.default_rng(seed + 1).choice(held, size=min(64, held.size), replace=False)
    kh = O.rms_norm(k_all[pick], kg, 1e-6).reshape(len(pick), G, d)
    k_ref = O.rope_rotate(kh, pick, w_, m_)
    slots = pick % W if kind == O.SLIDING else pick
    kc_h = host(kc[0][:, slots]).transpose(1, 0, 2)  # [n, G, d]
    vc_h = host(vc[0][:, slots]).transpose(1, 0, 2)
    assert np.array_equal(vc_h, v_all[pick]), f"{what}: cached values differ"
    assert_close(kc_h, k_ref, what=f"{what} cached keys")


@pytest.mark.parametrize("lt", [0, 1], ids=["sliding", "full_yarn"])
@pytest.mark.parametrize("shape", [(32, 32), (40, 8)], ids=["7b", "32b"])
def test_prefill_full_size_sampled(shape, lt):
    """7B (H=G=32) and 32B (H=40, G=8) prefill, B=1, T=8192, window 4096."""
    H, G = shape
    B, T, d = 1, 8192, 128
    rope = YARN if lt == 1 else PLAIN
    _log(f"prefill H={H} G={G} T={T} layer_type={lt}")
    x = inputs(2 if H == 32 else 4, lt, B, T, H, G, d, BF16)
    cap = W if lt == 0 else T
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    out = gpu_prefill(x, kc, vc, window=W, layer_type=lt, rope=rope, H=H)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    kv_heads = [0, 13, G - 1] if G > 8 else [0, 5, G - 1]
    _check_prefill_rows(x, out, kc, vc, T=T, H=H, G=G, d=d, lt=lt, rope=rope, kv_heads=kv_heads,
                        seed=lt, what=f"prefill {H}/{G} lt={lt}")


@pytest.mark.parametrize("lt", [0, 1], ids=["sliding_ring", "full_linear"])
@pytest.mark.parametrize("shape", [(32, 32, 32, 65536), (64, 40, 8, 32768)], ids=["7b", "32b"])
def test_decode_full_size_sampled(shape, lt):
    """7B decode B=32 at cache length 65,536; 32B decode B=64 at 32,768.
    The cache holds positions 0 .. L-2 (ring: the last 4096 of them); the new
    token sits at L-1."""
    B, H, G, L = shape
    d = 128
    kind = KINDS[lt]
    pos = L - 1
    cap = W if lt == 0 else L
    rope = YARN if lt == 1 else PLAIN
    _log(f"decode B={B} H={H} G={G} L={L} layer_type={lt}")
    kc, vc = synth.cache_fill(3 if H == 32 else 4, 100 + lt, B, G, cap, d, device="cuda", dtype=BF16)
    bs, gs = [0, B - 1], [0, G - 1]
    before_k = {(b, g): host(kc[b, g]) for b in bs for g in gs}
    before_v = {(b, g): host(vc[b, g]) for b in bs for g in gs}
    x = inputs(3 if H == 32 else 4, 200 + lt, B, 1, H, G, d, BF16)
    q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
    out = gpu_decode(q, k, v, x["q_gain"], x["k_gain"], kc, vc, window=W, layer_type=lt, rope=rope,
                     pos=pos, H=H)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    tags = O.ring_positions(kind, W, cap, pos)
    assert (tags >= 0).sum() == (min(pos, W) if lt == 0 else pos)
    hq, hk, hv = host(q), host(k), host(v)
    qg, kg = host(x["q_gain"]), host(x["k_gain"])
    group = H // G
    slot = pos % W if lt == 0 else pos
    for b in bs:
        ck = np.stack([before_k[(b, g)] for g in gs])
        cv = np.stack([before_v[(b, g)] for g in gs])
        ref = O.decode_rows_ref(hq[b], hk[b], hv[b], qg, kg, ck, cv, tags, H=H, G=G, d=d, kv_heads=gs,
                                kind=kind, window=W, rope=oracle_rope(rope), pos=pos)
        heads = [g * group + j for g in gs for j in range(group)]
        got = host(out[b]).reshape(H, d)[heads]
        err = assert_close(got, ref, what=f"decode b={b}")
        _log(f"  decode b={b}: {len(heads)} heads, max abs/rel err {err}")
        for g in gs:
            assert np.array_equal(host(vc[b, g, slot]), hv[b].reshape(G, d)[g])
            others = host(vc[b, g])
            others[slot] = before_v[(b, g)][slot]
            assert np.array_equal(others, before_v[(b, g)]), "decode wrote outside its slot"


def test_long_context_stack_sampled():
    """32-layer attention-only stack, 7B head shapes, B=1, T=65,536: full
    layers (l mod 4 == 3 and the last) use YaRN (factor 8, original 8192),
    sliding layers plain RoPE with window 4096; per-layer seeds.  Every layer
    runs on the GPU; sampled rows of layers 0, 3, 30 and 31 are compared with
    the oracle."""
    B, T, H, G, d, n_layers = 1, 65536, 32, 32, 128, 32
    kinds = O.layer_types(n_layers)
    assert kinds.count(O.FULL) == 8
    for ell in range(n_layers):
        lt = A.olmo3_layer_type(ell, n_layers)
        assert lt == O.layer_type_code(kinds[ell])
        rope = YARN if lt == 1 else PLAIN
        x = inputs(5 + ell, ell, B, T, H, G, d, BF16)
        cap = W if lt == 0 else T
        kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
        vc = torch.zeros_like(kc)
        out = gpu_prefill(x, kc, vc, window=W, layer_type=lt, rope=rope, H=H)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"layer {ell}"
        if ell in (0, 3, 30, 31):
            _log(f"long-context layer {ell} ({kinds[ell]})")
            _check_prefill_rows(x, out, kc, vc, T=T, H=H, G=G, d=d, lt=lt, rope=rope,
                                kv_heads=[0, 31], seed=100 + ell, what=f"long layer {ell}")
        del x, kc, vc, out


def test_decode_stack_reads_effective_bytes_per_token():
    """32-layer attention-only decode stack, 7B head shapes, B=2, cache
    length 65,536 (new token at 65,535), per-layer seeds.  Every layer's
    decode runs on the GPU and is compared with the oracle on two key/value
    heads of both sequences.  The rows the decode kernel reads, counted by
    its probe and summed over the stack, give the cache bytes per token of
    context that the page "Olmo 3 7B" states for the per-layer-type cache:
    155,648 B at 65,536 (against 524,288 B if every layer were full)."""
    B, H, G, d, L, n_layers = 2, 32, 32, 128, 65536, 32
    pos = L - 1
    kinds = O.layer_types(n_layers)
    gs = [0, G - 1]
    group = H // G
    heads = [g * group + j for g in gs for j in range(group)]
    rows_read = 0
    for ell, kind in enumerate(kinds):
        lt = O.layer_type_code(kind)
        cap = W if lt == 0 else L
        rope = YARN if lt == 1 else PLAIN
        kc, vc = synth.cache_fill(6, ell, B, G, cap, d, device="cuda", dtype=BF16)
        before = {b: (host(kc[b, gs]), host(vc[b, gs])) for b in range(B)}
        x = inputs(6, 100 + ell, B, 1, H, G, d, BF16)
        q, k, v = x["q_pre"][:, 0].contiguous(), x["k_pre"][:, 0].contiguous(), x["v"][:, 0].contiguous()
        out = gpu_decode(q, k, v, x["q_gain"], x["k_gain"], kc, vc, window=W, layer_type=lt,
                         rope=rope, pos=pos, H=H)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"layer {ell}"
        tags = O.ring_positions(kind, W, cap, pos)
        hq, hk, hv = host(q), host(k), host(v)
        qg, kg = host(x["q_gain"]), host(x["k_gain"])
        for b in range(B):
            ref = O.decode_rows_ref(hq[b], hk[b], hv[b], qg, kg, before[b][0], before[b][1], tags,
                                    H=H, G=G, d=d, kv_heads=gs, kind=kind, window=W,
                                    rope=oracle_rope(rope), pos=pos)
            assert_close(host(out[b]).reshape(H, d)[heads], ref, what=f"stack layer {ell} b={b}")
        count = A.olmo3_probe_decode_reads(B, H, G, d, W, lt, pos, cap).cpu().numpy()
        assert count.max() == 1
        rows_read += int(count.sum())
        del kc, vc, x, out
    _log(f"decode stack: {rows_read} rows read per (sequence, key/value head)")
    bytes_per_token = rows_read * G * d * 2 * 2 // L
    assert bytes_per_token == O.kv_bytes_per_token(kinds, G, d, W, L) == 155648
    assert O.kv_bytes_per_token([O.FULL] * n_layers, G, d, W, L) == 524288


def _rotated_keys_of(k_pre_rows, positions, k_gain, kind, rope, G, d):
    """The oracle's rotated keys for projected key rows [n, G*d] at `positions`."""
    w_, m_ = O.layer_rope(oracle_rope(rope), kind, d)
    kh = O.rms_norm(k_pre_rows, k_gain, 1e-6).reshape(len(positions), G, d)
    return O.rope_rotate(kh, np.asarray(positions), w_, m_)


def _chunk_rows_ref(x, b, row0, n_rows, P, rows, pre_k, pre_v, tags, gs, kind, rope, H, G, d):
    """Oracle outputs of chunk rows `rows` (within the chunk) of sequence b:
    queries and keys rows row0 .. row0 + n_rows - 1 of x at positions P ..,
    attending to the cache's held rows pre_k / pre_v [len(gs), cap, d]
    (positions `tags`) and to the chunk, for key/value heads gs."""
    held = np.nonzero(tags >= 0)[0]
    n = held.size + n_rows
    sl = slice(row0, row0 + n_rows)
    k_chunk = _rotated_keys_of(host(x["k_pre"][b, sl]), P + np.arange(n_rows), host(x["k_gain"]),
                               kind, rope, G, d)
    keys = np.zeros((n, G, d))   # only the sampled heads are filled
    vals = np.zeros((n, G, d))
    keys[:, gs] = np.concatenate([pre_k[:, held].transpose(1, 0, 2), k_chunk[:, gs]], axis=0)
    vals[:, gs] = np.concatenate([pre_v[:, held].transpose(1, 0, 2),
                                  host(x["v"][b, sl]).reshape(n_rows, G, d)[:, gs]], axis=0)
    key_pos = np.concatenate([tags[held], P + np.arange(n_rows)])
    return O.attention_rows_ref(host(x["q_pre"][b, row0 + rows]), P + rows, keys, vals, key_pos,
                                host(x["q_gain"]), host(x["k_gain"]), H=H, G=G, d=d,
                                kv_heads=gs, kind=kind, window=W, rope=oracle_rope(rope),
                                k_is_rotated=True)


@pytest.mark.parametrize("lt", [0, 1], ids=["sliding_ring", "full_linear"])
def test_chunked_prefill_full_size_sampled(lt):
    """7B shapes: a 4096-token chunk at positions 8192 .. 12287 onto a cache
    pre-filled with seeded rows (the ring holds 4096 .. 8191), as the bench's
    kernels run it; sampled query rows (both window edges, the chunk edges)
    of two key/value heads against the oracle."""
    B, P, T, H, G, d = 1, 8192, 4096, 32, 32, 128
    kind = KINDS[lt]
    rope = YARN if lt == 1 else PLAIN
    cap = W if lt == 0 else P + T
    kc, vc = synth.cache_fill(8, lt, B, G, cap, d, device="cuda", dtype=BF16)
    gs = [0, G - 1]
    pre_k, pre_v = host(kc[0, gs]), host(vc[0, gs])           # [2, cap, d], before the call
    tags = O.ring_positions(kind, W, cap, P)
    x = inputs(8, 30 + lt, B, T, H, G, d, BF16)
    out = gpu_prefill(x, kc, vc, window=W, layer_type=lt, rope=rope, H=H, pos_offset=P)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, T // 2, T - 2, T - 1} |
                           set(np.random.default_rng(9).integers(0, T, 12).tolist())))
    # keys: the held prefix (rotated, as stored) and the chunk (rotated by the oracle)
    got = host(out[0, rows]).reshape(len(rows), H, d)[:, gs]
    ref = _chunk_rows_ref(x, 0, 0, T, P, rows, pre_k, pre_v, tags, gs, kind, rope, H, G, d)
    err = assert_close(got, ref, what=f"chunked prefill {kind}")
    _log(f"chunked prefill {kind}: {len(rows)} rows, max abs/rel err {err}")


@pytest.mark.parametrize("lt", [0, 1], ids=["sliding_ring", "full_linear"])
def test_ragged_prefill_7b_shapes_sampled(lt):
    """7B heads, three packed sequences of 2000, 100 and 3000 tokens at
    position offsets 5000, 0 and 300 onto seeded caches; sampled rows of each
    sequence against the oracle run on that sequence alone."""
    H, G, d = 32, 32, 128
    lengths, offsets = [2000, 100, 3000], [5000, 0, 300]
    B, N = len(lengths), sum(lengths)
    kind = KINDS[lt]
    rope = YARN if lt == 1 else PLAIN
    max_end = max(p + n for p, n in zip(offsets, lengths))
    cap = W if lt == 0 else max_end
    kc, vc = synth.cache_fill(9, lt, B, G, cap, d, device="cuda", dtype=BF16)
    gs = [0, G - 1]
    pre = [(host(kc[b, gs]), host(vc[b, gs])) for b in range(B)]
    x = inputs(9, 40 + lt, 1, N, H, G, d, BF16)
    flat = {k: (v[0] if v.dim() == 3 else v) for k, v in x.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    po = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    out = torch.empty_like(flat["q_pre"])
    ws = A.workspace(A.MODE_PREFILL, 1, N, H, G, d, lt, BF16, cap, "cuda")
    A.olmo3_attn_prefill_ragged(flat["q_pre"], flat["k_pre"], flat["v"], flat["q_gain"],
                                flat["k_gain"], kc, vc, out, ws, cu, po, max_len=max(lengths),
                                max_end=max_end, window=W, layer_type=lt, rope=rope)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    row0 = 0
    for b, (n, P) in enumerate(zip(lengths, offsets)):
        rows = np.array(sorted({0, n - 1, n // 2} | set(np.random.default_rng(b).integers(0, n, 6).tolist())))
        tags = O.ring_positions(kind, W, cap, P)
        ref = _chunk_rows_ref(x, 0, row0, n, P, rows, pre[b][0], pre[b][1], tags, gs, kind, rope,
                              H, G, d)
        got = host(out[row0 + rows]).reshape(len(rows), H, d)[:, gs]
        err = assert_close(got, ref, what=f"ragged sequence {b} ({kind})")
        _log(f"ragged {kind} sequence {b}: {len(rows)} rows, max abs/rel err {err}")
        row0 += n
