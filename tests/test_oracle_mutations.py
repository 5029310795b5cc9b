"""Plants plausible mistakes in the CPU oracle and requires that at least one
pin in ``oracle_pins`` fails for each: evidence that the pins would notice a
dropped term, a wrong sign or index, or a transposed operand."""

import inspect
import math

import numpy as np
import pytest

import oracle.olmo3_oracle as O
from oracle_pins import ALL_CHECKS

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _mask_le_window(T, window):
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    return (s <= t) & (t - s <= window)


def _mask_at_le_window(q_pos, k_pos, kind, window):
    t = np.asarray(q_pos)[:, None]
    s = np.asarray(k_pos)[None, :]
    ok = (s >= 0) & (s <= t)
    if kind == O.SLIDING:
        ok &= (t - s) <= window
    return ok


def _mask_at_noncausal(q_pos, k_pos, kind, window):
    t = np.asarray(q_pos)[:, None]
    s = np.asarray(k_pos)[None, :]
    ok = s >= 0
    if kind == O.SLIDING:
        ok &= np.abs(t - s) < window
    return ok


def _layer_types_no_last(n):
    return [O.FULL if layer % 4 == 3 else O.SLIDING for layer in range(n)]


def _layer_types_mod4_eq0(n):
    return [O.FULL if (layer % 4 == 0 or layer == n - 1) else O.SLIDING for layer in range(n)]


def _rms_mean_abs(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * gain


def _rms_no_gain(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    if np.asarray(gain).shape != x.shape[-1:]:
        raise ValueError("gain")
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rms_per_head(x, gain, eps, d=8):
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % d:
        return _orig["rms_norm"](x, gain, eps)
    y = x.reshape(*x.shape[:-1], n // d, d)
    y = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return y.reshape(x.shape) * gain


def _gain_widths_per_head(H, G, d):
    return d, d


def _rope_sign(x, positions, inv_freq, mscale=1.0):
    return _orig["rope_rotate"](x, -np.asarray(positions), inv_freq, mscale)


def _rope_adjacent(x, positions, inv_freq, mscale=1.0):
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x2 * cos + x1 * sin
    return out * mscale


def _rope_no_mscale(x, positions, inv_freq, mscale=1.0):
    return _orig["rope_rotate"](x, positions, inv_freq, 1.0)


def _inv_freq_i_over_d(theta, d):
    i = np.arange(d // 2, dtype=np.float64)
    return np.float64(theta) ** (-1.0 * i / d)


def _yarn_ramp(theta, d, factor, orig_ctx, beta_fast, beta_slow, truncate=True, swap=False):
    w = O.rope_inv_freq(theta, d)
    if factor == 1.0:
        return w
    c = [d * math.log(orig_ctx / (2 * math.pi * b)) / (2 * math.log(theta)) for b in (beta_fast, beta_slow)]
    lo, hi = (math.floor(c[0]), math.ceil(c[1])) if truncate else (c[0], c[1])
    lo, hi = max(lo, 0), min(hi, d - 1)
    u = np.clip((np.arange(d // 2) - lo) / (hi - lo), 0.0, 1.0)
    if swap:
        u = 1.0 - u
    return (1.0 - u) * w + u * w / factor


def _yarn_swapped(theta, d, factor, orig_ctx, beta_fast=32.0, beta_slow=1.0):
    return _yarn_ramp(theta, d, factor, orig_ctx, beta_fast, beta_slow, swap=True)


def _yarn_untruncated(theta, d, factor, orig_ctx, beta_fast=32.0, beta_slow=1.0):
    return _yarn_ramp(theta, d, factor, orig_ctx, beta_fast, beta_slow, truncate=False)


def _yarn_ramp_in_rotations(theta, d, factor, orig_ctx, beta_fast=32.0, beta_slow=1.0):
    """The ramp written linear in the number of rotations r instead of the
    pair index."""
    w = O.rope_inv_freq(theta, d)
    if factor == 1.0:
        return w
    r = orig_ctx * w / (2 * math.pi)
    gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - gamma) * (w / factor) + gamma * w


def _yarn_mscale_log2(factor):
    return 1.0 if factor <= 1.0 else 0.1 * math.log2(factor) + 1.0


def _layer_rope_yarn_everywhere(rope, kind, d):
    return _orig["layer_rope"](rope, O.FULL if rope.yarn else kind, d)


def _attend_factory(scale_fn=None, group_fn=None, transpose_p=False):
    def attend(q, q_pos, k, v, k_pos, kind, window, row_block=1024):
        Tq, H, d = q.shape
        N, G, _ = k.shape
        group = H // G
        scale = scale_fn(d) if scale_fn else 1.0 / math.sqrt(d)
        out = np.zeros((Tq, H, d))
        allowed = O.mask_at_positions(q_pos, k_pos, kind, window)
        for h in range(H):
            g = group_fn(h, G, group) if group_fn else h // group
            s = (q[:, h, :] @ k[:, g, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            if transpose_p and p.shape[0] == p.shape[1]:
                p = p.T
            out[:, h, :] = p @ v[:, g, :]
        return out
    return attend


class _RingOffByOne(O.KvCacheRef):
    def slot(self, p):
        return p % (self.window + 1) % self.capacity if self.kind == O.SLIDING else p


class _RingKeepsFirst(O.KvCacheRef):
    def append(self, k, v, positions):
        for j, p in reversed(list(enumerate(np.asarray(positions)))):
            s = self.slot(int(p))
            self.k[:, :, s, :] = k[:, j]
            self.v[:, :, s, :] = v[:, j]
            self.pos[s] = p


def _cache_entries_all(kind, window, context):
    return context


def _e4m3_value_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp, man = (code >> 3) & 0xF, code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -7
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 8)


def _e4m3_encode_factory(mode):
    def enc(x):
        x = np.asarray(x, dtype=np.float64)
        mag = np.minimum(np.abs(x), 448.0)
        codes = np.arange(0x7F)
        vals = np.array([_orig["e4m3_value"](c) for c in codes])
        if mode == "truncate":
            pick = np.searchsorted(vals, mag, side="right") - 1
        else:  # ties away from zero
            dist = np.abs(mag[..., None] - vals)
            best = dist.min(axis=-1, keepdims=True)
            pick = vals.size - 1 - np.argmax((dist == best)[..., ::-1], axis=-1)
        out = codes[pick].astype(np.uint8)
        return np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)
    return enc


def _e4m3_encode_nan_saturates(x):
    x = np.asarray(x, dtype=np.float64)
    return _orig["e4m3_encode"](np.where(np.isnan(x), -448.0, x))


def _e4m3_store_twice(x, scale):
    inv = np.float32(1.0 / np.float64(scale))
    return _orig["e4m3_encode"](np.asarray(x, dtype=np.float32) * inv * inv)


def _decode_e4m3_drops_new_token(q_pre, k_pre, v, q_gain, k_gain, *, H, G, d, kind, window, rope,
                                 eps=1e-6, pos, cache, round_rotated=False):
    keys, vals, key_pos = cache.contents()
    q_pre = np.asarray(q_pre, dtype=np.float64)[:, None, :]
    B = q_pre.shape[0]
    qh = O.rms_norm(q_pre, q_gain, eps).reshape(B, 1, H, d)
    w, m = O.layer_rope(rope, kind, d)
    p = np.array([pos])
    q_rot = O.rope_rotate(qh, p, w, m)
    if round_rotated:
        q_rot = O.bf16_round(q_rot)
    return np.stack([O.attend(q_rot[b], p, keys[b], vals[b], key_pos, kind, window)
                     for b in range(B)]).reshape(B, H * d)


def _bf16_factory(mode):
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        mag = np.abs(x)
        _, e2 = np.frexp(mag)
        bits = 8 if mode == "8 bits" else 7
        step = np.ldexp(1.0, np.maximum(e2 - 1, -126) - bits)
        q = mag / step
        if mode == "truncate":
            r = np.floor(q)
        elif mode == "away":
            r = np.floor(q + 0.5)
        else:
            r = np.rint(q)
        return np.copysign(r * step, x)
    return rnd


def _prefill_edited(old, new):
    """prefill_ref with one source line replaced (same module globals)."""
    src = inspect.getsource(_orig["prefill_ref"])
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    return ns["prefill_ref"]


def _decode_e4m3_edited(old, new):
    """decode_e4m3_ref with one source line replaced (same module globals)."""
    src = inspect.getsource(_orig["decode_e4m3_ref"])
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    return ns["decode_e4m3_ref"]


MUTANTS = {
    "mask t-s <= window": dict(sliding_window_mask=_mask_le_window, mask_at_positions=_mask_at_le_window),
    "mask not causal": dict(mask_at_positions=_mask_at_noncausal),
    "last layer not full": dict(layer_types=_layer_types_no_last),
    "full when l mod 4 == 0": dict(layer_types=_layer_types_mod4_eq0),
    "rms uses mean |x|": dict(rms_norm=_rms_mean_abs),
    "rms drops gain": dict(rms_norm=_rms_no_gain),
    "rms per head": dict(rms_norm=_rms_per_head),
    "gain widths per head": dict(qk_gain_widths=_gain_widths_per_head),
    "rope sign flipped": dict(rope_rotate=_rope_sign),
    "rope adjacent pairs": dict(rope_rotate=_rope_adjacent),
    "rope drops mscale": dict(rope_rotate=_rope_no_mscale),
    "rope exponent i/d": dict(rope_inv_freq=_inv_freq_i_over_d),
    "yarn ramp swapped": dict(yarn_inv_freq=_yarn_swapped),
    "yarn ramp bounds not rounded": dict(yarn_inv_freq=_yarn_untruncated),
    "yarn ramp linear in rotations": dict(yarn_inv_freq=_yarn_ramp_in_rotations),
    "yarn mscale log2": dict(yarn_mscale=_yarn_mscale_log2),
    "yarn on sliding layers": dict(layer_rope=_layer_rope_yarn_everywhere),
    "scale 1/d": dict(attend=_attend_factory(scale_fn=lambda d: 1.0 / d)),
    "scale missing": dict(attend=_attend_factory(scale_fn=lambda d: 1.0)),
    "gqa h mod G": dict(attend=_attend_factory(group_fn=lambda h, G, grp: h % G)),
    "probabilities transposed": dict(attend=_attend_factory(transpose_p=True)),
    "ring slot p mod (w+1)": dict(KvCacheRef=_RingOffByOne),
    "ring keeps first writer": dict(KvCacheRef=_RingKeepsFirst),
    "no window bound on cache": dict(cache_entries=_cache_entries_all),
    "e4m3 exponent bias 8": dict(e4m3_value=_e4m3_value_bias8),
    "e4m3 truncates": dict(e4m3_encode=_e4m3_encode_factory("truncate")),
    "e4m3 ties away from zero": dict(e4m3_encode=_e4m3_encode_factory("away")),
    "e4m3 scale applied twice": dict(e4m3_store=_e4m3_store_twice),
    "e4m3 NaN saturates": dict(e4m3_encode=_e4m3_encode_nan_saturates),
    "e4m3 decode drops the new token": dict(decode_e4m3_ref=_decode_e4m3_drops_new_token),
    "e4m3 round_rotated skips queries": dict(decode_e4m3_ref=_decode_e4m3_edited(
        "q_rot = bf16_round(q_rot)", "q_rot = q_rot")),
    "bf16 truncates": dict(bf16_round=_bf16_factory("truncate")),
    "bf16 ties away from zero": dict(bf16_round=_bf16_factory("away")),
    "bf16 keeps 8 mantissa bits": dict(bf16_round=_bf16_factory("8 bits")),
    "round_rotated skips keys": dict(prefill_ref=_prefill_edited(
        "k_rot = rnd(rope_rotate(kh,", "k_rot = (rope_rotate(kh,")),
    "round_rotated skips queries": dict(prefill_ref=_prefill_edited(
        "q_rot = bf16_round(q_rot * q_scale) / q_scale", "q_rot = q_rot")),
    "round_rotated rounds queries without their scale": dict(prefill_ref=_prefill_edited(
        "q_rot = bf16_round(q_rot * q_scale) / q_scale", "q_rot = bf16_round(q_rot)")),
    "round_rotated keeps the query scale": dict(prefill_ref=_prefill_edited(
        "q_rot = bf16_round(q_rot * q_scale) / q_scale", "q_rot = bf16_round(q_rot * q_scale)")),
    "round_rotated skips cached keys": dict(prefill_ref=_prefill_edited(
        "past_k = rnd(rope_rotate(", "past_k = (rope_rotate(")),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        monkeypatch.setattr(O, attr, fn)
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin noticed the planted mistake '{name}'"
