"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each ``check_*`` function raises AssertionError when the oracle disagrees
with a value printed on the pages, a closed form, a library routine, or an
invariant.  ``test_oracle_pins.py`` runs them all; ``test_oracle_mutations.py``
plants plausible mistakes in the oracle and requires some check to fail.
"""

from __future__ import annotations

import copy
import math
import os

import numpy as np
import torch

import oracle.olmo3_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=1e-10, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _inputs(rng, B, T, H, G, d):
    return dict(q_pre=rng.standard_normal((B, T, H * d)),
                k_pre=rng.standard_normal((B, T, G * d)),
                v=rng.standard_normal((B, T, G * d)),
                q_gain=rng.uniform(0.5, 1.5, H * d),
                k_gain=rng.uniform(0.5, 1.5, G * d))


# ----------------------------------------------------------------- layers
def check_layer_types_golden():
    """Page "OLMo 3's Sliding-Window Attention Pattern", "Which layers are full"."""
    for row in _golden("layer_types.txt"):
        if row[0] == "count":
            n, ns, nf = int(row[1]), int(row[3]), int(row[5])
            kinds = O.layer_types(n)
            assert kinds.count(O.SLIDING) == ns and kinds.count(O.FULL) == nf
        else:
            n = int(row[0])
            want = [O.FULL if c == "f" else O.SLIDING for c in row[1:]]
            assert len(want) == n
            assert O.layer_types(n) == want, (n, O.layer_types(n))


def check_layer_types_rule():
    """Last layer always full; otherwise full iff l mod 4 == 3."""
    for n in range(1, 70):
        kinds = O.layer_types(n)
        assert kinds[-1] == O.FULL
        for layer in range(n - 1):
            assert (kinds[layer] == O.FULL) == (layer % 4 == 3)


# ------------------------------------------------------------------ masks
def check_mask_table_golden():
    """The printed T = 5, window = 2 table."""
    want = np.array([[int(x) for x in r] for r in _golden("mask_T5_window2.txt")], dtype=bool)
    got = O.sliding_window_mask(5, 2)
    assert got.dtype == bool and np.array_equal(got, want), got.astype(int)


def check_mask_row_counts():
    """Row t allows min(t + 1, window) keys (page 5, "Hint")."""
    for T in (1, 2, 7, 33, 64):
        for w in (1, 2, 3, 16, 31, 64, 100):
            m = O.sliding_window_mask(T, w)
            t = np.arange(T)
            assert np.array_equal(m.sum(axis=1), np.minimum(t + 1, w)), (T, w)


def check_mask_window_ge_T_is_tril():
    """window >= T is the ordinary causal mask (page 5, "Requirements")."""
    for T in (1, 5, 17):
        for w in (T, T + 1, 10 * T):
            assert np.array_equal(O.sliding_window_mask(T, w), np.tril(np.ones((T, T), dtype=bool)))
        assert np.array_equal(O.causal_mask(T), np.tril(np.ones((T, T), dtype=bool)))


def check_window3_example():
    """Window 3: token 4 sees {2,3,4} sliding and {0..4} full (page 3, item 4)."""
    rows = {r[0]: [int(x) for x in r[1:]] for r in _golden("worked_examples.txt")
            if r[0].startswith("window3")}
    masks = O.attention_masks(5, 4, 3)  # 4 layers: s, s, s, f
    assert list(np.nonzero(masks[0][4])[0]) == rows["window3_t4_sliding"]
    assert list(np.nonzero(masks[3][4])[0]) == rows["window3_t4_full"]


def check_mask_at_positions():
    """The position-level predicate equals the table at positions 0..T-1, is
    invariant to a common shift, and rejects empty slots (-1)."""
    for T, w in ((9, 4), (20, 7), (5, 2)):
        p = np.arange(T)
        assert np.array_equal(O.mask_at_positions(p, p, O.SLIDING, w), O.sliding_window_mask(T, w))
        assert np.array_equal(O.mask_at_positions(p, p, O.FULL, w), O.causal_mask(T))
        assert np.array_equal(O.mask_at_positions(p + 1000, p + 1000, O.SLIDING, w),
                              O.sliding_window_mask(T, w))
    assert not O.mask_at_positions(np.array([5]), np.array([-1]), O.FULL, 4).any()


# --------------------------------------------------------------- QK-norm
def check_qknorm_example():
    """(30, 40) -> about (0.85, 1.13); dot 2500 -> 2.0 (page 3, item 2)."""
    ex = {r[0]: r[1:] for r in _golden("worked_examples.txt")}
    x = np.array([float(v) for v in ex["qknorm_input"]])
    want = [float(v) for v in ex["qknorm_output"][:2]]
    dec = int(ex["qknorm_output"][3])
    assert float(x @ x) == float(ex["qknorm_dot_before"][0])
    y = O.rms_norm(x, np.ones(2), 1e-6)
    assert np.array_equal(np.round(y, dec), np.array(want)), y
    assert abs(float(y @ y) - float(ex["qknorm_dot_after"][0])) < 1e-6


def check_rms_invariants():
    """Unit gain, eps 0: mean square 1; invariant to scaling x; zero maps to
    zero when eps > 0; the gain multiplies feature-wise."""
    rng = _rng(1)
    x = rng.standard_normal((4, 96))
    y = O.rms_norm(x, np.ones(96), 0.0)
    _close(np.mean(y * y, axis=-1), np.ones(4), 1e-12, "mean square")
    _close(O.rms_norm(7.5 * x, np.ones(96), 0.0), y, 1e-12, "scale invariance")
    assert not O.rms_norm(np.zeros((2, 8)), np.ones(8), 1e-6).any()
    g = rng.uniform(0.5, 1.5, 96)
    _close(O.rms_norm(x, g, 0.0), y * g, 1e-12, "gain")


def check_qknorm_spans_all_heads():
    """One statistic per token over all H*d features: the ratio of two heads'
    norms survives QK-norm (a per-head norm would equalise them), and the
    result equals x / sqrt(mean(x^2) + eps) with the mean over H*d."""
    rng = _rng(2)
    H, d = 4, 8
    x = rng.standard_normal((3, H * d))
    x[:, :d] *= 10.0
    y = O.rms_norm(x, np.ones(H * d), 0.0)
    r_in = np.linalg.norm(x[:, :d], axis=1) / np.linalg.norm(x[:, d:2 * d], axis=1)
    r_out = np.linalg.norm(y[:, :d], axis=1) / np.linalg.norm(y[:, d:2 * d], axis=1)
    _close(r_in, r_out, 1e-12, "head ratio")
    _close(np.sum(y * y, axis=1), np.full(3, H * d), 1e-9, "sum of squares = H*d")


def check_param_counts_pin_gain_widths():
    """The published counts come out exactly only with QK-norm gains of
    width H*d and G*d (page "Count OLMo 3's Parameters")."""
    for row in _golden("param_counts.txt"):
        V, D, L, H, G, F, tied, total = (int(v) for v in row[1:9])
        d = D // H
        wq, wk = O.qk_gain_widths(H, G, d)
        per_layer = D * H * d + 2 * D * G * d + H * d * D + wq + wk + 3 * D * F + 2 * D
        count = (1 if tied else 2) * V * D + L * per_layer + D
        assert count == total, (row[0], count, total)
        if len(row) > 9:
            assert per_layer == int(row[9])


# ------------------------------------------------------------------- RoPE
def check_rope_rates_golden():
    """Slowest pair at d = 128: theta^(-126/128) rad per position, printed as
    1.15e-4 (theta 1e4, ~54,000 positions a turn) and 2.5e-6 (theta 5e5,
    ~2.6 million) (page 3, item 3)."""
    ex = _golden("worked_examples.txt")
    d = int([r for r in ex if r[0] == "rope_head_dim"][0][1])
    for r in ex:
        if r[0] != "rope_slowest_rate":
            continue
        theta, rate, turn = float(r[1]), float(r[2]), float(r[4])
        w = O.rope_inv_freq(theta, d)[-1]
        sig = len(r[2].split("e")[0].replace(".", "")) - 1  # printed significant digits - 1
        assert float(f"{w:.{sig}e}") == rate, (theta, w)
        assert abs(2 * math.pi / w - turn) / turn < 0.05, (theta, 2 * math.pi / w)
    w = O.rope_inv_freq(10000.0, 128)
    assert w[0] == 1.0 and np.all(np.diff(w) < 0)


def check_rope_complex_multiplication():
    """Rotate-half RoPE is complex multiplication of x_i + 1j*x_{i+d/2} by
    exp(1j * p * omega_i) (dimension i paired with i + d/2, page 3 item 3)."""
    rng = _rng(3)
    d, P, Hh = 16, 7, 3
    x = rng.standard_normal((P, Hh, d))
    pos = np.array([0, 1, 2, 5, 100, 4095, 65535])
    w = O.rope_inv_freq(500000.0, d)
    got = O.rope_rotate(x, pos, w, 1.0)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * w[None, None, :])
    _close(got, np.concatenate([z.real, z.imag], axis=-1), 1e-12, "complex form")


def check_rope_invariants():
    """Position 0 is the identity; pair norms are kept; the multiplier scales
    lengths; dot products depend only on the position difference."""
    rng = _rng(4)
    d = 32
    x = rng.standard_normal((1, 2, d))
    w = O.rope_inv_freq(10000.0, d)
    _close(O.rope_rotate(x, np.array([0]), w), x, 0.0, "pos 0")
    y = O.rope_rotate(x, np.array([777]), w)
    _close(x[..., :d // 2] ** 2 + x[..., d // 2:] ** 2, y[..., :d // 2] ** 2 + y[..., d // 2:] ** 2,
           1e-12, "pair norm")
    _close(O.rope_rotate(x, np.array([777]), w, 1.25), 1.25 * y, 1e-12, "mscale")
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    dots = [float(np.sum(O.rope_rotate(q, np.array([p + 13]), w) * O.rope_rotate(k, np.array([p]), w)))
            for p in (0, 50, 9999)]
    _close(dots, [dots[0]] * 3, 1e-9, "relative position")


def check_yarn_reductions():
    """YaRN: factor 1 gives plain RoPE; rates with many turns over the
    original context (r > beta_fast) are kept; rates with less than
    beta_slow turns are divided by the factor exactly; every rate lies in
    [omega/s, omega]; the temperature at s = 8 is 0.1 ln 8 + 1."""
    theta, d, L = 500000.0, 128, 8192
    w = O.rope_inv_freq(theta, d)
    _close(O.yarn_inv_freq(theta, d, 1.0, L), w, 0.0, "s=1")
    s = 8.0
    y = O.yarn_inv_freq(theta, d, s, L, 32.0, 1.0)
    r = L * w / (2 * math.pi)
    hi, lo = r > 32.0, r < 1.0
    assert hi.any() and lo.any() and (~hi & ~lo).any()
    _close(y[hi], w[hi], 0.0, "high-frequency dims kept")
    _close(y[lo], w[lo] / s, 1e-18, "low-frequency dims interpolated")
    assert np.all(y <= w * (1 + 1e-15)) and np.all(y >= w / s * (1 - 1e-15))
    ratio = y / w
    assert np.all(np.diff(ratio) <= 1e-15), "interpolation grows towards long wavelengths"
    assert abs(O.yarn_mscale(8.0) - (0.1 * math.log(8.0) + 1.0)) < 1e-15
    assert O.yarn_mscale(1.0) == 1.0
    rope = O.RopeParams(theta=theta, yarn=True, factor=s, orig_ctx=L)
    wf, mf = O.layer_rope(rope, O.FULL, d)
    ws, ms = O.layer_rope(rope, O.SLIDING, d)
    _close(wf, y, 0.0, "full layer uses YaRN")
    _close(ws, w, 0.0, "sliding layer uses plain RoPE")
    assert abs(mf - 1.2079441541679836) < 1e-12 and ms == 1.0


# -------------------------------------------------------------- attention
def _sdpa(q, k, v, mask):
    """torch's scaled_dot_product_attention (default scale 1/sqrt(d)) in fp64
    on the CPU, heads first; GQA by repeating each key/value head."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    H, G = q.shape[1], k.shape[1]
    kt = torch.from_numpy(np.repeat(k, H // G, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, H // G, axis=1)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    return o[0].permute(1, 0, 2).numpy()


def _hf_olmo3_config(H, G, d, theta, factor, orig_ctx, window=4096, n_layers=4):
    """transformers' OLMo 3 configuration with the given attention shapes:
    plain RoPE on sliding layers, YaRN on full layers (factor, original
    context, beta_fast 32, beta_slow 1), hidden size H*d."""
    from transformers import Olmo3Config
    rope = {"sliding_attention": {"rope_type": "default", "rope_theta": theta},
            "full_attention": {"rope_type": "yarn", "rope_theta": theta, "factor": factor,
                               "original_max_position_embeddings": orig_ctx,
                               "beta_fast": 32.0, "beta_slow": 1.0}}
    return Olmo3Config(hidden_size=H * d, intermediate_size=8, num_hidden_layers=n_layers,
                       num_attention_heads=H, num_key_value_heads=G, head_dim=d,
                       max_position_embeddings=int(orig_ctx * factor), rope_parameters=rope,
                       sliding_window=window, rms_norm_eps=1e-6, attention_bias=False)


def check_yarn_matches_transformers():
    """YaRN rates and temperature equal those of an independent
    implementation, the transformers library's (the code model
    configurations with rope_type "yarn" run), interior of the ramp
    included; it computes in fp32, hence the 1e-6 relative bound."""
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    for theta, d, s, L in [(500000.0, 128, 8.0, 8192), (10000.0, 64, 4.0, 2048),
                           (1e6, 128, 16.0, 4096), (500000.0, 128, 8.0, 256)]:
        cfg = _hf_olmo3_config(2, 1, d, theta, s, L)
        inv, att = ROPE_INIT_FUNCTIONS["yarn"](cfg, None, layer_type="full_attention")
        inv = inv.double().numpy()
        ours = O.yarn_inv_freq(theta, d, s, L)
        w = O.rope_inv_freq(theta, d)
        interior = (ours < w * (1 - 1e-9)) & (ours > w / s * (1 + 1e-9))
        assert interior.sum() >= 3, (theta, d, s, L)
        _close(ours / inv, np.ones(d // 2), 1e-6, f"YaRN rates {theta, d, s, L}")
        assert abs(att - O.yarn_mscale(s)) < 1e-12


def check_attention_layer_matches_transformers():
    """A whole attention call (QK-norm over H*d / G*d, RoPE or YaRN at
    absolute positions, GQA grouping, 1/sqrt(d) scale, softmax, weighted
    values) equals the transformers library's OLMo 3 attention module run in
    fp64 (its norm, rotation angles and softmax in fp32: 1e-5 relative) on
    the same projections, with its output projection set to the identity
    and the oracle's mask passed in: this pins the rotation direction, the
    grouping order, the scale and the YaRN temperature."""
    from transformers.models.olmo3.modeling_olmo3 import Olmo3Attention, Olmo3RotaryEmbedding
    H, G, d, T, w, theta, s, L, p0 = 4, 2, 32, 48, 10, 10000.0, 8.0, 64, 100
    cfg = _hf_olmo3_config(H, G, d, theta, s, L, window=w)
    gen = torch.Generator().manual_seed(11)
    rope = O.RopeParams(theta=theta, yarn=True, factor=s, orig_ctx=L)
    for layer_idx, kind in ((0, O.SLIDING), (3, O.FULL)):
        assert cfg.layer_types[layer_idx] == ("sliding_attention" if kind == O.SLIDING else "full_attention")
        att = Olmo3Attention(cfg, layer_idx).double().eval()
        with torch.no_grad():
            for lin in (att.q_proj, att.k_proj, att.v_proj):
                lin.weight.copy_(torch.randn(lin.weight.shape, generator=gen, dtype=torch.float64) / 8)
            att.o_proj.weight.copy_(torch.eye(H * d, dtype=torch.float64))
            for nrm in (att.q_norm, att.k_norm):
                nrm.weight.copy_(0.5 + torch.rand(nrm.weight.shape, generator=gen, dtype=torch.float64))
            x = torch.randn((1, T, H * d), generator=gen, dtype=torch.float64)
            pos = p0 + np.arange(T)
            rot = Olmo3RotaryEmbedding(cfg)
            cos, sin = rot(x, torch.as_tensor(pos)[None], cfg.layer_types[layer_idx])
            allowed = O.mask_at_positions(pos, pos, kind, w)
            mask = torch.where(torch.as_tensor(allowed), 0.0, -torch.inf).double()[None, None]
            got, _ = att(x, (cos.double(), sin.double()), mask)
            xn = x[0].numpy()
            ref = O.prefill_ref(xn[None] @ att.q_proj.weight.numpy().T, xn[None] @ att.k_proj.weight.numpy().T,
                                xn[None] @ att.v_proj.weight.numpy().T, att.q_norm.weight.numpy(),
                                att.k_norm.weight.numpy(), H=H, G=G, d=d, kind=kind, window=w,
                                rope=rope, pos_offset=p0)
        scale = float(np.abs(ref).max())
        _close(got.numpy(), ref, 1e-5 * scale, f"attention layer {kind}")


def check_attend_matches_sdpa():
    """The masked softmax core equals torch's SDPA with the explicit mask."""
    rng = _rng(5)
    for (T, H, G, d, kind, w) in ((37, 4, 2, 16, O.SLIDING, 8), (29, 3, 3, 8, O.FULL, 5),
                                  (50, 10, 2, 16, O.SLIDING, 1), (16, 2, 1, 32, O.SLIDING, 40)):
        q = rng.standard_normal((T, H, d))
        k = rng.standard_normal((T, G, d))
        v = rng.standard_normal((T, G, d))
        p = np.arange(T)
        got = O.attend(q, p, k, v, p, kind, w, row_block=7)
        want = _sdpa(q, k, v, O.mask_at_positions(p, p, kind, w))
        _close(got, want, 1e-12, f"sdpa {kind} T={T} H={H} G={G}")


def check_single_token_returns_v0():
    """T = 1: the only allowed key is the token itself, so out = v_0 per group."""
    rng = _rng(6)
    H, G, d = 6, 2, 8
    x = _inputs(rng, 2, 1, H, G, d)
    rope = O.RopeParams(theta=10000.0)
    for kind in (O.SLIDING, O.FULL):
        out = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=4, rope=rope)
        v = x["v"].reshape(2, 1, G, d)
        want = np.repeat(v, H // G, axis=2).reshape(2, 1, H * d)
        _close(out, want, 1e-12, "T=1")


def check_zero_query_uniform_average():
    """q_pre = 0: every score is 0, so each row is the plain mean of the
    values its mask allows: min(t+1, w) rows on a sliding layer."""
    rng = _rng(7)
    B, T, H, G, d, w = 2, 23, 4, 2, 8, 5
    x = _inputs(rng, B, T, H, G, d)
    x["q_pre"] = np.zeros_like(x["q_pre"])
    rope = O.RopeParams(theta=10000.0)
    v = x["v"].reshape(B, T, G, d)
    for kind in (O.SLIDING, O.FULL):
        out = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope).reshape(B, T, H, d)
        for t in range(T):
            lo = max(0, t - w + 1) if kind == O.SLIDING else 0
            mean = v[:, lo:t + 1].mean(axis=1)  # [B, G, d]
            for h in range(H):
                _close(out[:, t, h], mean[:, h // (H // G)], 1e-12, f"uniform {kind} t={t} h={h}")


def check_sliding_wide_window_equals_full():
    """window >= T on a sliding layer equals a full layer (no YaRN)."""
    rng = _rng(8)
    B, T, H, G, d = 1, 19, 4, 1, 16
    x = _inputs(rng, B, T, H, G, d)
    rope = O.RopeParams(theta=10000.0, yarn=False)
    a = O.prefill_ref(**x, H=H, G=G, d=d, kind=O.SLIDING, window=T, rope=rope)
    b = O.prefill_ref(**x, H=H, G=G, d=d, kind=O.FULL, window=3, rope=rope)
    _close(a, b, 1e-12, "wide window")


def check_gqa_equals_repeated_mha():
    """GQA equals MHA with every key/value head (and its key gains) repeated
    H/G times; with G = H it is plain MHA."""
    rng = _rng(9)
    B, T, H, G, d = 2, 21, 6, 2, 8
    x = _inputs(rng, B, T, H, G, d)
    rope = O.RopeParams(theta=10000.0)
    rep = H // G
    kx = x["k_pre"].reshape(B, T, G, d).repeat(rep, axis=2).reshape(B, T, H * d)
    vx = x["v"].reshape(B, T, G, d).repeat(rep, axis=2).reshape(B, T, H * d)
    gx = x["k_gain"].reshape(G, d).repeat(rep, axis=0).reshape(H * d)
    for kind in (O.SLIDING, O.FULL):
        a = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=6, rope=rope)
        b = O.prefill_ref(x["q_pre"], kx, vx, x["q_gain"], gx, H=H, G=H, d=d, kind=kind,
                          window=6, rope=rope)
        _close(a, b, 1e-12, f"gqa {kind}")


def check_position_shift_invariance():
    """Prefill outputs depend on relative positions only (plain RoPE)."""
    rng = _rng(10)
    B, T, H, G, d = 1, 17, 2, 1, 16
    x = _inputs(rng, B, T, H, G, d)
    rope = O.RopeParams(theta=10000.0)
    for kind in (O.SLIDING, O.FULL):
        a = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=5, rope=rope, pos_offset=0)
        b = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=5, rope=rope, pos_offset=4321)
        _close(a, b, 1e-9, f"shift {kind}")


def check_cache_holds_rotated_keys_at_absolute_positions():
    """The first token (position 0) is stored unrotated; position p is the
    key rotated by p; v is stored untouched; slots follow p (full) or
    p mod w (sliding) and the ring keeps the last w positions."""
    rng = _rng(11)
    B, T, H, G, d, w = 2, 11, 2, 2, 8, 4
    x = _inputs(rng, B, T, H, G, d)
    rope = O.RopeParams(theta=10000.0)
    kh = O.rms_norm(x["k_pre"], x["k_gain"], 1e-6).reshape(B, T, G, d)
    vv = x["v"].reshape(B, T, G, d)
    wr = O.rope_inv_freq(10000.0, d)
    for kind, cap in ((O.FULL, T), (O.SLIDING, w)):
        c = O.KvCacheRef(kind, w, cap, B, G, d)
        O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope, cache=c)
        first = T - min(T, cap) if kind == O.SLIDING else 0
        assert sorted(c.pos.tolist()) == list(range(first, T)), c.pos
        for p in range(first, T):
            s = p % w if kind == O.SLIDING else p
            assert c.pos[s] == p
            _close(c.v[:, :, s], vv[:, p], 0.0, "v copied")
            want = O.rope_rotate(kh[:, p][:, None], np.array([p]), wr)[:, 0]
            _close(c.k[:, :, s], want, 1e-12, "k rotated by its position")
        if kind == O.FULL:
            _close(c.k[:, :, 0], kh[:, 0], 0.0, "position 0 unrotated")


def check_prefill_then_decode_equals_longer_prefill():
    """prefill(T0) then decode of positions T0..T-1 reproduces the last rows of
    prefill(T), on the ring (wrapping several times) and on the linear cache,
    with both key-storage variants (rotated or not)."""
    rng = _rng(12)
    B, T, T0, H, G, d, w = 2, 26, 9, 4, 2, 8, 6
    x = _inputs(rng, B, T, H, G, d)
    for yarn in (False, True):
        rope = O.RopeParams(theta=10000.0, yarn=yarn, factor=4.0, orig_ctx=16)
        for kind, cap in ((O.SLIDING, w), (O.FULL, T)):
            full = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope)
            for rotated in (True, False):
                c = O.KvCacheRef(kind, w, cap, B, G, d, rotated=rotated)
                head = {k: (v[:, :T0] if v.ndim == 3 else v) for k, v in x.items()}
                a = O.prefill_ref(**head, H=H, G=G, d=d, kind=kind, window=w, rope=rope, cache=c)
                _close(a, full[:, :T0], 1e-12, "prefix")
                for p in range(T0, T):
                    o = O.decode_ref(x["q_pre"][:, p], x["k_pre"][:, p], x["v"][:, p],
                                     x["q_gain"], x["k_gain"], H=H, G=G, d=d, kind=kind,
                                     window=w, rope=rope, pos=p, cache=c)
                    _close(o, full[:, p], 1e-10, f"decode {kind} rotated={rotated} p={p}")
                    held = int((c.pos >= 0).sum())
                    assert held == (min(p + 1, w) if kind == O.SLIDING else p + 1)


def check_planted_value_window_edges():
    """Uniform attention (q = 0) with one value row planted at a large
    constant: the plant shows up as c/n exactly when it lies inside the
    window of row t and is absent otherwise (s = t-w, t-w+1, t, t+1)."""
    B, T, H, G, d, w = 1, 30, 2, 1, 8, 7
    rng = _rng(13)
    base = _inputs(rng, B, T, H, G, d)
    base["q_pre"] = np.zeros_like(base["q_pre"])
    base["v"] = np.zeros_like(base["v"])
    rope = O.RopeParams(theta=10000.0)
    t = 20
    for s in (t - w, t - w + 1, t, t + 1):
        x = dict(base)
        x["v"] = base["v"].copy()
        x["v"][0, s, :] = 1024.0
        out = O.prefill_ref(**x, H=H, G=G, d=d, kind=O.SLIDING, window=w, rope=rope)
        inside = (s <= t) and (t - s < w)
        want = 1024.0 / w if inside else 0.0
        _close(out[0, t], np.full(H * d, want), 1e-9, f"plant s={s}")


def check_kv_bytes_golden():
    """Page "Olmo 3 7B": 524,288 B/token naive, 16,384 B/layer/token,
    131,072 + 1,610,612,736/c effective, 3.37x at 65,536 and 1.6x at 8k;
    page 3 item 4: the cache is about 0.30 of full-everywhere at 65,536."""
    g = {r[0]: r[1:] for r in _golden("kv_bytes.txt") if r[0] != "overpay_at"}
    over = [r[1:] for r in _golden("kv_bytes.txt") if r[0] == "overpay_at"]
    L, G, d, w = (int(g[k][0]) for k in ("layers", "kv_heads", "head_dim", "window"))
    kinds = O.layer_types(L)
    naive = O.kv_bytes_per_token([O.FULL] * L, G, d, w, 65536)
    assert naive == int(g["naive_bytes_per_token"][0])
    assert O.kv_bytes_per_token([O.FULL], G, d, w, 123) == int(g["bytes_per_layer_per_token"][0])
    for c in (4096, 8192, 65536, 10000):
        eff = O.kv_bytes_per_token(kinds, G, d, w, c)
        if c >= w:
            assert abs(eff - (int(g["effective_constant"][0]) + int(g["effective_over_c"][0]) / c)) < 1e-6
    for c, ratio, _, dec in over:
        eff = O.kv_bytes_per_token(kinds, G, d, w, int(c))
        assert round(naive / eff, int(dec)) == float(ratio), (c, naive / eff)
    frac = O.kv_bytes_per_token(kinds, G, d, w, 65536) / naive
    assert round(frac, int(g["cache_fraction_65536"][2])) == float(g["cache_fraction_65536"][0])
    kinds64 = O.layer_types(64)
    frac64 = O.kv_bytes_per_token(kinds64, 8, 128, w, 65536) / O.kv_bytes_per_token([O.FULL] * 64, 8, 128, w, 65536)
    assert abs(frac64 - frac) < 1e-15


def check_sampled_functions_equal_whole_output():
    """The row- and head-sampled evaluations used at full workload sizes give
    the same numbers as the whole-output prefill and decode."""
    rng = _rng(14)
    T, H, G, d, w = 50, 6, 2, 8, 9
    x = _inputs(rng, 1, T, H, G, d)
    rows = np.array([0, 7, 8, 9, 30, 49])
    for kind, cap in ((O.SLIDING, w), (O.FULL, T)):
        rope = O.RopeParams(theta=1e4, yarn=True, factor=4.0, orig_ctx=16)
        full = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope).reshape(T, H, d)
        got = O.attention_rows_ref(x["q_pre"][0, rows], rows, x["k_pre"][0],
                                   x["v"][0].reshape(T, G, d), np.arange(T), x["q_gain"],
                                   x["k_gain"], H=H, G=G, d=d, kv_heads=[1], kind=kind, window=w,
                                   rope=rope)
        _close(got, full[rows][:, 3:6], 1e-12, f"rows {kind}")
        c = O.KvCacheRef(kind, w, cap, 1, G, d)
        head = {k: (v[:, :T - 1] if v.ndim == 3 else v) for k, v in x.items()}
        O.prefill_ref(**head, H=H, G=G, d=d, kind=kind, window=w, rope=rope, cache=c)
        assert np.array_equal(c.pos, O.ring_positions(kind, w, cap, T - 1))
        ck, cv, cp = c.k[0].copy(), c.v[0].copy(), c.pos.copy()
        ref = O.decode_ref(x["q_pre"][:, T - 1], x["k_pre"][:, T - 1], x["v"][:, T - 1],
                           x["q_gain"], x["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                           rope=rope, pos=T - 1, cache=c)
        got = O.decode_rows_ref(x["q_pre"][0, T - 1], x["k_pre"][0, T - 1], x["v"][0, T - 1],
                                x["q_gain"], x["k_gain"], ck[[1]], cv[[1]], cp, H=H, G=G, d=d,
                                kv_heads=[1], kind=kind, window=w, rope=rope, pos=T - 1)
        _close(got, ref[0].reshape(H, d)[3:6], 1e-12, f"decode rows {kind}")


# ------------------------------------------------------------- e4m3 cache
# The format is the OCP 8-bit floating point E4M3 format (the pages fix none):
# its table and its round-to-nearest-even encoding are pinned to torch's own
# float8_e4m3fn conversion, an implementation independent of the oracle's
# brute force, and to closed forms of the format's definition.

def check_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_values()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])


def check_e4m3_encode_matches_torch_in_range():
    rng = _rng(71)
    table = O.e4m3_values()
    pos_vals = np.sort(table[:0x7F])
    mids = (pos_vals[:-1] + pos_vals[1:]) / 2          # exact ties
    x = np.concatenate([rng.normal(0, 1, 2000), rng.normal(0, 100, 2000),
                        rng.normal(0, 0.01, 2000), rng.uniform(-448, 448, 2000),
                        mids, -mids, pos_vals, -pos_vals, [0.0, -0.0, 448.0, -448.0]])
    x = x[np.abs(x) <= 448.0].astype(np.float32)        # in range: no saturation
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def check_e4m3_closed_forms():
    v = O.e4m3_value
    assert v(0x7E) == 1.75 * 2 ** 8 == O.E4M3_MAX
    assert v(0x01) == 2.0 ** -9 and v(0x08) == 2.0 ** -6 and v(0x38) == 1.0
    assert v(0x07) == 7 * 2.0 ** -9 and v(0xB8) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    table = O.e4m3_values()
    assert len(set(table[~np.isnan(table)].tolist())) == 253   # 254 finite codes, +-0 equal
    enc = O.e4m3_encode
    assert list(enc([1e6, -1e6, 449.0, 463.9, 464.0, 1e30])) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E, 0x7E]
    # infinities saturate like any magnitude past 448; a NaN stays a NaN
    # (the code torch's float8_e4m3fn conversion gives it)
    assert list(enc([math.inf, -math.inf])) == [0x7E, 0xFE]
    nan_code = int(torch.tensor([math.nan]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    assert nan_code == 0x7F and list(enc([math.nan, -math.nan])) == [0x7F, 0xFF]
    # ties go to the even mantissa: 1 + 1/16 -> 1.0, 1 + 3/16 -> 1.25, 2^-10 -> 0
    assert list(enc([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10])) == [0x38, 0x3A, 0x00, 0x02]
    # half-ulp error: relative 2^-4 on normals, absolute 2^-10 on subnormals
    rng = _rng(73)
    x = np.concatenate([rng.uniform(2.0 ** -6, 448, 5000), rng.uniform(0, 2.0 ** -6, 5000)])
    err = np.abs(table[enc(x)] - x)
    normal = x >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * x[normal]).all()
    assert (err[~normal] <= 2.0 ** -10).all()


def check_e4m3_cache_stores_scale_once():
    """A value that is exactly code * scale is stored exactly: a scale applied
    twice, or not at all, moves it (x * fp32(1/3) lands within 3e-8 relative of
    the code, far from any tie)."""
    rng = _rng(79)
    table = O.e4m3_values()
    B, G, d, w = 1, 2, 8, 4
    for ks, vs in ((0.5, 3.0), (3.0, 0.5)):
        c = O.KvCacheRef(O.SLIDING, w, w, B, G, d, e4m3_scales=(ks, vs))
        ck = rng.integers(0, 0x7F, (B, 3, G, d)) | rng.integers(0, 2, (B, 3, G, d)) * 0x80
        cv = rng.integers(0, 0x7F, (B, 3, G, d)) | rng.integers(0, 2, (B, 3, G, d)) * 0x80
        k, v = table[ck] * ks, table[cv] * vs
        c.append(k, v, np.array([5, 6, 7]))
        kk, vv, pos = c.contents()
        order = np.argsort(pos)
        assert np.array_equal(kk[:, order], k) and np.array_equal(vv[:, order], v)
        assert list(pos[order]) == [5, 6, 7]
    # and an arbitrary value lands within half a step of the grid times the scale
    c = O.KvCacheRef(O.FULL, w, 8, 1, 1, 4, e4m3_scales=(0.37, 0.37))
    x = rng.normal(0, 1, (1, 1, 1, 4))
    c.append(x, x, np.array([0]))
    assert (np.abs(c.k[0, 0, 0] - x[0, 0, 0]) <= 2.0 ** -4 * np.abs(x[0, 0, 0]) + 0.37 * 2.0 ** -10).all()


def check_decode_e4m3_equals_decode_on_the_grid():
    """When every cached row and the new token's key and value are exact
    e4m3 multiples of the scales (the new key is zero: k_pre = 0 normalises to
    0), storing codes changes nothing, so e4m3 decode equals plain decode;
    it also means the new token is stored before the attention reads."""
    rng = _rng(83)
    table = O.e4m3_values()
    B, H, G, d, w, pos = 2, 4, 2, 16, 6, 9
    rope = O.RopeParams(theta=10000.0)
    for kind in (O.SLIDING, O.FULL):
        cap = w if kind == O.SLIDING else pos + 1
        ks, vs = 0.25, 2.0
        ck = rng.integers(0x20, 0x48, (B, G, cap, d)) | rng.integers(0, 2, (B, G, cap, d)) * 0x80
        cv = rng.integers(0x20, 0x48, (B, G, cap, d)) | rng.integers(0, 2, (B, G, cap, d)) * 0x80
        caches = []
        for e4 in (False, True):
            c = O.KvCacheRef(kind, w, cap, B, G, d, e4m3_scales=(ks, vs) if e4 else None)
            c.k[:] = table[ck] * ks
            c.v[:] = table[cv] * vs
            c.pos[:] = O.ring_positions(kind, w, cap, pos)
            caches.append(c)
        q = rng.normal(0, 1, (B, H * d))
        k0 = np.zeros((B, G * d))
        v_new = table[rng.integers(0x20, 0x48, (B, G * d))] * vs
        qg, kg = rng.uniform(0.5, 1.5, H * d), rng.uniform(0.5, 1.5, G * d)
        # with and without bf16 rounding of the rotated query (the cached
        # values are e4m3 multiples, which bf16 holds exactly)
        for rr in (False, True):
            cs = [copy.deepcopy(c) for c in caches]
            a = O.decode_ref(q, k0, v_new, qg, kg, H=H, G=G, d=d, kind=kind, window=w, rope=rope,
                             pos=pos, cache=cs[0], round_rotated=rr)
            b = O.decode_e4m3_ref(q, k0, v_new, qg, kg, H=H, G=G, d=d, kind=kind, window=w,
                                  rope=rope, pos=pos, cache=cs[1], round_rotated=rr)
            _close(a, b, 1e-12, f"e4m3 decode on the grid, {kind}, round_rotated {rr}")
        assert np.abs(a - O.decode_ref(q, k0, v_new, qg, kg, H=H, G=G, d=d, kind=kind, window=w,
                                       rope=rope, pos=pos, cache=copy.deepcopy(caches[0]))).max() > 0


# ------------------------------------------------------------ bf16 rounding
def _bf16_neighbours(rng, n):
    """n random finite bfloat16 values b (normal and subnormal, both signs)
    with the next value away from zero, as fp64 (exact: bf16 values are)."""
    bits = rng.integers(0x0001, 0x7F7F, n).astype(np.uint32)
    sign = rng.integers(0, 2, n).astype(np.uint32) << 15
    lo = ((bits | sign) << 16).view(np.float32).astype(np.float64)
    hi = (((bits + 1) | sign) << 16).view(np.float32).astype(np.float64)
    return lo, hi


def check_bf16_round_matches_torch():
    """On values exactly representable in fp32, torch's fp32 -> bfloat16
    conversion (round to nearest even) gives the same values, for random
    magnitudes from fp32 subnormals to past the bfloat16 maximum, and for the
    exact midpoints between neighbouring bfloat16 values."""
    rng = _rng(91)
    mant = rng.standard_normal(40000)
    x = (mant * np.exp2(rng.integers(-140, 126, mant.size).astype(np.float64))).astype(np.float32)
    lo, hi = _bf16_neighbours(rng, 20000)
    mids = ((lo + hi) / 2).astype(np.float32)           # exact: 9 significant bits
    near_max = np.float32(O.BF16_MAX) * np.array([1.0, 1.001, 1.0019, 1.002, 1.003], np.float32)
    x = np.concatenate([x, mids, lo.astype(np.float32), near_max, -near_max,
                        np.array([0.0, -0.0, 1e-45, -1e-45], np.float32)])
    assert np.isfinite(x).all()
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.isinf(got).any() and (got[np.isinf(got)] == want[np.isinf(want)]).all()


def check_bf16_round_closed_forms():
    """Spacing 2^-7 at 1; halves go to the even neighbour; a value just past a
    half goes up even when fp32 cannot hold it (rounded once, from fp64);
    at most half a step from x (relative 2^-8 on normals); fixed points are
    the bfloat16 values; signs, zeros and NaN kept."""
    r = O.bf16_round
    one = 1.0
    assert list(r([one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -40,
                   -(one + 2.0 ** -8), 2.0 ** -134, 3 * 2.0 ** -134])) == \
        [1.0, one + 2.0 ** -6, one + 2.0 ** -7, -1.0, 0.0, 2.0 ** -132]
    assert r(O.BF16_MAX) == O.BF16_MAX and r(-O.BF16_MAX) == -O.BF16_MAX
    assert r(O.BF16_MAX + 2.0 ** 119) == np.inf and r(O.BF16_MAX + 2.0 ** 118) == O.BF16_MAX
    assert np.signbit(r(-0.0)) and r(0.0) == 0.0 and np.isnan(r(np.nan))
    rng = _rng(92)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-100, 100, 20000).astype(np.float64))
    y = r(x)
    assert (np.abs(y - x) <= 2.0 ** -8 * np.abs(x)).all()
    assert np.array_equal(r(y), y)
    lo, hi = _bf16_neighbours(rng, 5000)
    assert np.array_equal(r(lo), lo) and np.array_equal(r(hi), hi)
    t = 0.25 * lo + 0.75 * hi                            # strictly nearer hi
    assert np.array_equal(r(t), hi) and np.array_equal(r(0.75 * lo + 0.25 * hi), lo)


def check_round_rotated_matches_sdpa_on_rounded_operands():
    """With round_rotated, prefill equals torch's SDPA over the rotated
    queries and keys rounded by torch's bfloat16 conversion (both of them,
    the values untouched).  torch converts fp64 through fp32, which can only
    differ from one rounding when an fp64 value lies within an fp32 half
    step of a bfloat16 midpoint; the test asserts that no operand does."""
    rng = _rng(93)
    B, T, H, G, d, w = 1, 23, 4, 2, 16, 7
    x = _inputs(rng, B, T, H, G, d)
    x["q_gain"] = x["q_gain"] * 3.0
    x["k_gain"] = x["k_gain"] * 3.0
    for kind, yarn in ((O.SLIDING, False), (O.FULL, True)):
        rope = O.RopeParams(theta=10000.0, yarn=yarn, factor=4.0, orig_ctx=8)
        wr, m = O.layer_rope(rope, kind, d)
        p = np.arange(T)
        q = O.rope_rotate(O.rms_norm(x["q_pre"], x["q_gain"], 1e-6).reshape(T, H, d), p, wr, m)
        k = O.rope_rotate(O.rms_norm(x["k_pre"], x["k_gain"], 1e-6).reshape(T, G, d), p, wr, m)
        # a query scale as a kernel's base-2 softmax scale (fp32 log2(e)/sqrt(d))
        qs = float(np.float32(math.log2(math.e) / math.sqrt(d)))
        for t in (q, k, q * qs):
            _, e2 = np.frexp(np.abs(t))
            frac = np.abs(t) / np.ldexp(1.0, np.maximum(e2 - 1, -126) - 7) % 1.0
            assert (np.abs(frac - 0.5) > 2.0 ** -15).all(), "operand next to a bf16 midpoint"
        def tb(t):
            return torch.from_numpy(t).to(torch.bfloat16).to(torch.float64).numpy()
        mask = O.mask_at_positions(p, p, kind, w)
        want = _sdpa(tb(q), tb(k), x["v"].reshape(T, G, d), mask)
        got = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope,
                            round_rotated=True).reshape(T, H, d)
        _close(got, want, 1e-12, f"round_rotated vs sdpa {kind}")
        plain = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope)
        assert np.abs(plain.reshape(T, H, d) - want).max() > 1e-4, "rounding had no effect"
        # queries held as bf16 of qs times their value, divided by qs after
        want_s = _sdpa(tb(q * qs) / qs, tb(k), x["v"].reshape(T, G, d), mask)
        got_s = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope,
                              round_rotated=True, q_scale=qs).reshape(T, H, d)
        _close(got_s, want_s, 1e-12, f"round_rotated with a query scale vs sdpa {kind}")
        assert np.abs(got_s - want).max() > 1e-4, "the query scale had no effect"


def check_round_rotated_cache_flow():
    """With round_rotated, prefill(T0) then decodes reproduce prefill(T) on
    the ring and the linear cache, with rotated and unrotated key storage:
    cached keys are rounded once, as the new ones are."""
    rng = _rng(94)
    B, T, T0, H, G, d, w = 1, 19, 7, 2, 1, 8, 5
    x = _inputs(rng, B, T, H, G, d)
    rope = O.RopeParams(theta=10000.0, yarn=True, factor=4.0, orig_ctx=8)
    for kind, cap in ((O.SLIDING, w), (O.FULL, T)):
        full = O.prefill_ref(**x, H=H, G=G, d=d, kind=kind, window=w, rope=rope,
                             round_rotated=True)
        for rotated in (True, False):
            c = O.KvCacheRef(kind, w, cap, B, G, d, rotated=rotated)
            head = {k: (v[:, :T0] if v.ndim == 3 else v) for k, v in x.items()}
            O.prefill_ref(**head, H=H, G=G, d=d, kind=kind, window=w, rope=rope, cache=c,
                          round_rotated=True)
            for p in range(T0, T):
                o = O.decode_ref(x["q_pre"][:, p], x["k_pre"][:, p], x["v"][:, p],
                                 x["q_gain"], x["k_gain"], H=H, G=G, d=d, kind=kind,
                                 window=w, rope=rope, pos=p, cache=c, round_rotated=True)
                _close(o, full[:, p], 1e-12, f"rounded decode {kind} rotated={rotated} p={p}")


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_") and callable(v)]
