"""Plain fp64 NumPy oracle of OLMo 3's per-layer attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code, tables or constants with the HIP
library, and it imports nothing from the product package.

What it computes, per attention layer and per call (prefill over T tokens, or
decode of one token, which is the same computation with T = 1):

1. layer type: full or sliding (page "OLMo 3's Sliding-Window Attention
   Pattern", section "Which layers are full");
2. QK-norm: one RMSNorm over each token's whole projected query vector (H*d
   features) and whole key vector (G*d features), with a learned gain per
   feature (page "Case Study: OLMo 3", architecture item 2 "QK-norm"; page
   "Count OLMo 3's Parameters", "What to count": gains of width H*d and G*d;
   page "Olmo-3 End-to-End Implementation", "Technical Details": eps = 1e-6);
3. RoPE of the "rotate half" layout, dimension i paired with i + d/2, base
   theta, at absolute position pos_offset + j (page "Case Study: OLMo 3",
   item 3 "Rotary embeddings"; page "Olmo-3 End-to-End Implementation",
   "Inference Pipeline": RoPE with position offsets), rescaled with YaRN on
   full layers (page "Case Study: OLMo 3", item 7 "long-context scaling");
4. KV-cache append: a ring of `window` slots on sliding layers, a linear
   cache on full layers (page "Olmo 3 7B", "SERVICEABILITY JOIN": per-layer-
   type cache management; page "Olmo-3 End-to-End Implementation", "KV Cache
   Implementation" and "Cache Operation Flow");
5. causal attention under an explicit boolean mask: s <= t, and t - s < window
   on sliding layers (page "OLMo 3's Sliding-Window Attention Pattern",
   section "The sliding-window mask"), softmax of q.k / sqrt(d), weighted sum
   of values.

Readings taken where the pages are silent:
softmax scale 1/sqrt(d); the rotation direction x_i + i*x_{i+d/2} times
exp(+i*angle); contiguous GQA grouping g(h) = h // (H/G); YaRN as the
NTK-by-parts interpolation of Peng et al. (2023) in the form its authors'
code computes it (a ramp over the pair index between the floor and ceiling
of the indices where beta_fast = 32 and beta_slow = 1 rotations fit in the
original context; see ``yarn_inv_freq``), and an attention temperature
m = 0.1*ln(s) + 1 multiplied into both q and k.  The pages pin none of
these; the tests pin them to an independent implementation of the model's
attention (the transformers library's OLMo 3 attention and its YaRN rates).

No intermediate is rounded: inputs are taken exactly as given (bf16 values
are exactly representable in fp64) and everything is computed in fp64.  Two
exceptions: the optional e4m3 cache, whose stored code is an integer that
floating point decides; the library's interface fixes that decision (the
code nearest to the fp32 product of the value and fp32(1/scale), ties to the
even mantissa, saturated at +-448, NaN kept as a NaN code), and the oracle
implements that contract, see ``e4m3_store``;
and the opt-in ``round_rotated`` switch of ``prefill_ref`` / ``decode_ref``,
which rounds the rotated queries and keys to bfloat16, the type every
operand of a bfloat16 model's attention has (page "Olmo-3 End-to-End
Implementation", "Technical Details": bfloat16 throughout), see
``bf16_round``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "SLIDING", "FULL", "layer_types", "layer_type_code", "sliding_window_mask",
    "causal_mask", "attention_masks", "mask_at_positions", "rms_norm",
    "qk_gain_widths", "rope_inv_freq", "yarn_inv_freq", "yarn_mscale",
    "RopeParams", "layer_rope", "rope_rotate", "KvCacheRef", "cache_entries",
    "kv_bytes_per_token", "attend", "prefill_ref", "decode_ref",
    "attention_rows_ref", "decode_rows_ref", "ring_positions",
    "E4M3_MAX", "e4m3_value", "e4m3_values", "e4m3_encode", "e4m3_store", "decode_e4m3_ref",
    "BF16_MAX", "bf16_round",
]

SLIDING = "sliding"
FULL = "full"


# --------------------------------------------------------------------------
# Layer types and masks
# --------------------------------------------------------------------------

def layer_types(n_layers: int) -> list[str]:
    """Layer kinds of a model of ``n_layers`` layers, counted from 0.

    Page "OLMo 3's Sliding-Window Attention Pattern", section "Which layers are
    full": layer l is full when l mod 4 equals 3, and the last layer is full
    whatever its index; every other layer is sliding.
    """
    if n_layers <= 0:
        raise ValueError("n_layers must be positive")
    return [FULL if (layer % 4 == 3 or layer == n_layers - 1) else SLIDING
            for layer in range(n_layers)]


def layer_type_code(kind: str) -> int:
    """Integer code of a layer kind: 0 sliding, 1 full (our numbering)."""
    return {SLIDING: 0, FULL: 1}[kind]


def sliding_window_mask(T: int, window: int) -> np.ndarray:
    """Boolean (T, T) table; entry [t, s] is True when query t may see key s.

    Page "OLMo 3's Sliding-Window Attention Pattern", section "The
    sliding-window mask": allowed when s <= t (causal) and t - s < window (the
    key is one of the last `window` tokens, the query itself included).  Built
    by broadcasting a column of query positions against a row of key
    positions, as that page's hint describes.
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    return (s <= t) & (t - s < window)


def causal_mask(T: int) -> np.ndarray:
    """Plain causal (lower-triangle) mask of a full layer.

    Page "OLMo 3's Sliding-Window Attention Pattern", "What to implement": a
    full layer gets the ordinary causal mask.
    """
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    return s <= t


def attention_masks(T: int, n_layers: int, window: int) -> list[np.ndarray]:
    """One mask per layer, following ``layer_types`` (same page and section)."""
    return [causal_mask(T) if kind == FULL else sliding_window_mask(T, window)
            for kind in layer_types(n_layers)]


def mask_at_positions(q_pos: np.ndarray, k_pos: np.ndarray, kind: str,
                      window: int) -> np.ndarray:
    """The same predicate at arbitrary absolute positions.

    Query at absolute position t and key at absolute position s: allowed when
    s <= t, and on sliding layers also t - s < window.  Negative key positions
    mark empty cache slots and are never allowed.
    """
    t = np.asarray(q_pos, dtype=np.int64)[:, None]
    s = np.asarray(k_pos, dtype=np.int64)[None, :]
    ok = (s >= 0) & (s <= t)
    if kind == SLIDING:
        ok &= (t - s) < window
    elif kind != FULL:
        raise ValueError(kind)
    return ok


# --------------------------------------------------------------------------
# QK-norm
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with a per-feature gain and no bias.

    Page "Case Study: OLMo 3", item 2 "QK-norm": queries and keys are
    RMS-normalised before attention; page "Olmo-3 End-to-End Implementation",
    "Technical Details": eps = 1e-6.  Reading: eps is added to the mean of
    squares inside the square root, and the gain multiplies after
    normalising.  The statistic runs over the whole last axis, which for
    QK-norm is the whole H*d (or G*d) vector of a token, since the gain has
    one entry per feature of that vector (page "Count OLMo 3's Parameters").
    """
    x = np.asarray(x, dtype=np.float64)
    gain = np.asarray(gain, dtype=np.float64)
    if gain.shape != x.shape[-1:]:
        raise ValueError(f"gain shape {gain.shape} does not match features {x.shape[-1]}")
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def qk_gain_widths(H: int, G: int, d: int) -> tuple[int, int]:
    """Widths of the query-norm and key-norm gains: one gain per feature of the
    normalised vector, i.e. H*d and G*d (page "Count OLMo 3's Parameters",
    "What to count", and its hint that the key norm depends on G)."""
    return H * d, G * d


# --------------------------------------------------------------------------
# RoPE and YaRN
# --------------------------------------------------------------------------

def rope_inv_freq(theta: float, d: int) -> np.ndarray:
    """Per-pair angular rates omega_i = theta**(-2i/d), i = 0 .. d/2 - 1.

    Page "Case Study: OLMo 3", item 3: with d = 128 the slowest pair (i = 63)
    turns by theta**(-126/128) per position, which fixes the exponent 2i/d.
    """
    if d % 2:
        raise ValueError("d must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * i / d)


def yarn_inv_freq(theta: float, d: int, factor: float, orig_ctx: int,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """YaRN rates (Peng et al., 2023, "NTK-by-parts" interpolation).

    Page "Case Study: OLMo 3", item 7: full layers are rescaled with YaRN from
    8,192 to 65,536 positions (factor 8); page "Olmo 3 7B" says the scaling
    comes from the model's configuration.  The pages give no formula, so the
    method's published definition in the form its authors' code computes it
    (the form model configurations are run with) is taken:
    - pair i turns r_i = orig_ctx * omega_i / (2 pi) times over the original
      context; r_i = beta falls at the (fractional) pair index
      c(beta) = d * ln(orig_ctx / (2 pi beta)) / (2 ln theta);
    - the ramp runs over the pair index between lo = floor(c(beta_fast)) and
      hi = ceil(c(beta_slow)) (clipped to [0, d - 1]; hi moved 0.001 past lo
      if they meet): u_i = clip((i - lo) / (hi - lo), 0, 1);
    - omega'_i = (1 - u_i) * omega_i + u_i * omega_i / factor: pairs below
      lo (many turns) keep their rate, pairs from hi on (under one turn) are
      interpolated by the factor.
    """
    w = rope_inv_freq(theta, d)
    if factor == 1.0:
        return w
    def pair_index(beta):
        return d * math.log(orig_ctx / (2.0 * math.pi * beta)) / (2.0 * math.log(theta))
    lo = max(math.floor(pair_index(beta_fast)), 0)
    hi = min(math.ceil(pair_index(beta_slow)), d - 1)
    if lo == hi:
        hi += 0.001
    u = np.clip((np.arange(d // 2, dtype=np.float64) - lo) / (hi - lo), 0.0, 1.0)
    return (1.0 - u) * w + u * (w / factor)


def yarn_mscale(factor: float) -> float:
    """YaRN attention temperature multiplier applied to q and to k.

    Peng et al. (2023): sqrt(1/t) = 0.1*ln(s) + 1, so the logits grow by its
    square; 1 when s <= 1.
    """
    return 1.0 if factor <= 1.0 else 0.1 * math.log(factor) + 1.0


@dataclass(frozen=True)
class RopeParams:
    """RoPE / YaRN settings of a model.  ``yarn`` applies to full layers only
    (page "Case Study: OLMo 3", item 7; page "Olmo 3 7B": YaRN factor 8 from an
    8192 base).  ``attn_factor <= 0`` means "derive 0.1*ln(factor) + 1"."""

    theta: float = 500000.0
    yarn: bool = False
    factor: float = 8.0
    orig_ctx: int = 8192
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    attn_factor: float = 0.0


def layer_rope(rope: RopeParams, kind: str, d: int) -> tuple[np.ndarray, float]:
    """(rates, multiplier) used on a layer of kind ``kind``: YaRN rates and
    temperature on full layers when YaRN is on, plain RoPE otherwise."""
    if rope.yarn and kind == FULL:
        w = yarn_inv_freq(rope.theta, d, rope.factor, rope.orig_ctx,
                          rope.beta_fast, rope.beta_slow)
        m = rope.attn_factor if rope.attn_factor > 0 else yarn_mscale(rope.factor)
        return w, float(m)
    return rope_inv_freq(rope.theta, d), 1.0


def rope_rotate(x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray,
                mscale: float = 1.0) -> np.ndarray:
    """Rotate every head vector of ``x`` by its absolute position.

    ``x`` has shape [..., P, heads, d] and ``positions`` shape [P].  Pair
    (i, i + d/2) turns by angle a = p * omega_i ("rotate half" layout, page
    "Case Study: OLMo 3", item 3):
        x'_i       = x_i cos a - x_{i+d/2} sin a
        x'_{i+d/2} = x_{i+d/2} cos a + x_i sin a
    then both halves are multiplied by ``mscale``.  Values are unchanged by
    RoPE (page "Olmo-3 End-to-End Implementation", "Technical Details").
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    if inv_freq.shape != (half,):
        raise ValueError("inv_freq must have d/2 entries")
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)
    return out * mscale


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------
# bfloat16 is the upper half of an IEEE binary32: sign, 8 exponent bits (bias
# 127), 7 stored mantissa bits.  A normal value of binade 2^e is a multiple
# of 2^(e-7); below 2^-126 the values are the subnormal multiples of 2^-133.

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value to each fp64 value, returned as fp64: the
    multiple of the binade's spacing nearest to x, halfway cases to the even
    multiple (IEEE round to nearest even, taken once from the fp64 value);
    magnitudes that round past BF16_MAX become infinities; signs, zeros and
    NaNs are kept."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)                       # mag = f * 2^e2, f in [0.5, 1)
    binade = np.maximum(e2 - 1, -126)           # floor(log2 |x|), normal range
    step = np.ldexp(1.0, binade - 7)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(mag / step) * step          # rint: halves to even
        r = np.where(r > BF16_MAX, np.inf, r)
    return np.copysign(r, x)


# --------------------------------------------------------------------------
# e4m3 cache codes
# --------------------------------------------------------------------------
# The pages name quantization only as a next step (page "Olmo-3 End-to-End
# Implementation", "Next Steps") and as a failure mode of quantized caches on
# sliding-window layers (page "Olmo 3 7B", "SERVICEABILITY JOIN"); they fix
# no format.  The format used is the 8-bit E4M3 format of the OCP 8-bit
# floating point specification: sign bit, 4 exponent bits with bias 7, 3
# mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the all-ones
# exponent with mantissa 7 is NaN; there are no infinities, so the largest
# finite value is 1.75 * 2^8 = 448.

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The value a code stands for, from its bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_values() -> np.ndarray:
    """Values of all 256 codes (NaN for the two NaN codes)."""
    return np.array([e4m3_value(c) for c in range(256)])


def e4m3_encode(x) -> np.ndarray:
    """Nearest code to each value, as uint8.  Magnitudes above 448 saturate to
    448; a value halfway between two codes takes the one whose mantissa is
    even (consecutive non-negative codes differ by one in their low bit); the
    sign bit is the value's sign (so -0.0 and small negatives give 0x80); a
    NaN gives the NaN code 0x7F (0xFF with the sign bit set).
    Brute force: compare against all 127 finite non-negative codes."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    x = np.where(nan, np.copysign(0.0, x), x)    # keeps a NaN's sign bit
    mag = np.minimum(np.abs(x), E4M3_MAX)
    codes = np.arange(0x7F)                      # 0x00 .. 0x7E, increasing values
    vals = np.array([e4m3_value(c) for c in codes])
    dist = np.abs(mag[..., None] - vals)         # [..., 127]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                          # one code, or two on a tie
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    out = codes[pick].astype(np.uint8)
    out = np.where(nan, np.uint8(0x7F), out)
    return np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)


def e4m3_store(x, scale: float) -> np.ndarray:
    """Code stored for value x with cache scale `scale`, as the library's
    interface defines it for every e4m3 entry point: the fp32 product
    x * fp32(1/scale), then its nearest code (``e4m3_encode``: ties to the
    even mantissa, saturated at +-448, NaN to a NaN code)."""
    inv = np.float32(1.0 / np.float64(scale))
    return e4m3_encode(np.asarray(x, dtype=np.float32) * inv)


# --------------------------------------------------------------------------
# Per-layer-type KV cache
# --------------------------------------------------------------------------

def cache_entries(kind: str, window: int, context: int) -> int:
    """Number of positions a layer's cache holds at context length ``context``:
    at most ``window`` on a sliding layer, all of them on a full layer (page
    "Olmo 3 7B", "KV OVERPAY": windowed layers hold at most w tokens)."""
    return min(context, window) if kind == SLIDING else context


def kv_bytes_per_token(kinds: list[str], G: int, d: int, window: int,
                       context: int, elem_bytes: int = 2) -> float:
    """Cache bytes per token of context, summed over layers: each held position
    stores a key and a value of G*d elements (page "Olmo 3 7B", "KV" and
    "KV OVERPAY")."""
    total = sum(cache_entries(k, window, context) * G * d * 2 * elem_bytes for k in kinds)
    return total / context


class KvCacheRef:
    """One layer's cache, laid out [B][G][capacity][d] like the page's
    [B, H_kv, T_total, D] (page "Olmo-3 End-to-End Implementation", "KV Cache
    Implementation"), plus a tag per slot with the absolute position it holds
    (-1 = empty).

    Sliding layers use a ring of ``window`` slots, slot = position mod window;
    full layers use slot = position (page "Olmo 3 7B": a windowed layer keeps a
    bounded, rotating cache).  When two positions of one append share a slot,
    the later one is kept.  ``rotated`` chooses whether keys are stored after
    RoPE or before it (the pages say both; the outputs must agree).
    """

    def __init__(self, kind: str, window: int, capacity: int, B: int, G: int,
                 d: int, rotated: bool = True, e4m3_scales: tuple | None = None):
        if kind == SLIDING and capacity != window:
            raise ValueError("a sliding layer's ring has exactly `window` slots")
        self.kind, self.window, self.capacity = kind, window, capacity
        self.B, self.G, self.d, self.rotated = B, G, d, rotated
        # e4m3 storage: (k_scale, v_scale); a stored key is the value of its
        # code times k_scale (see e4m3_store), a value likewise
        self.e4m3_scales = e4m3_scales
        self.k = np.zeros((B, G, capacity, d))
        self.v = np.zeros((B, G, capacity, d))
        self.pos = np.full(capacity, -1, dtype=np.int64)

    def slot(self, p: int) -> int:
        s = p % self.window if self.kind == SLIDING else p
        if not 0 <= s < self.capacity:
            raise IndexError(f"position {p} does not fit a cache of {self.capacity}")
        return s

    def append(self, k: np.ndarray, v: np.ndarray, positions: np.ndarray) -> None:
        """k, v: [B, n, G, d] for the absolute ``positions`` (length n)."""
        if self.e4m3_scales is not None:
            ks, vs = self.e4m3_scales
            table = e4m3_values()
            k = table[e4m3_store(k, ks)] * ks
            v = table[e4m3_store(v, vs)] * vs
        for j, p in enumerate(np.asarray(positions, dtype=np.int64)):
            s = self.slot(int(p))
            self.k[:, :, s, :] = k[:, j]
            self.v[:, :, s, :] = v[:, j]
            self.pos[s] = p

    def contents(self) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(k [B, n, G, d], v [B, n, G, d], positions [n]) of the filled slots,
        in slot order."""
        idx = np.nonzero(self.pos >= 0)[0]
        return (self.k[:, :, idx, :].transpose(0, 2, 1, 3),
                self.v[:, :, idx, :].transpose(0, 2, 1, 3), self.pos[idx].copy())


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attend(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
           k_pos: np.ndarray, kind: str, window: int,
           row_block: int = 1024) -> np.ndarray:
    """Masked softmax attention of one sequence.

    q [Tq, H, d] at positions q_pos; k, v [N, G, d] at positions k_pos.  Query
    head h reads key/value head h // (H/G) (page "Case Study: OLMo 3", item 1:
    each key/value head serves H/G query heads; contiguous grouping is our
    reading).  Scores are q.k / sqrt(d); forbidden pairs get -inf; the row
    maximum is subtracted before exp; rows are normalised to sum 1.  Query rows
    are processed in blocks only to bound memory.
    """
    Tq, H, d = q.shape
    N, G, _ = k.shape
    if H % G:
        raise ValueError("H must be a multiple of G")
    group = H // G
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((Tq, H, d))
    for r0 in range(0, Tq, row_block):
        r1 = min(Tq, r0 + row_block)
        allowed = mask_at_positions(q_pos[r0:r1], k_pos, kind, window)
        for h in range(H):
            g = h // group
            s = (q[r0:r1, h, :] @ k[:, g, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[r0:r1, h, :] = p @ v[:, g, :]
    return out


def _project_heads(q_pre, k_pre, v, q_gain, k_gain, H, G, d, eps):
    B, T = q_pre.shape[:2]
    qh = rms_norm(q_pre, q_gain, eps).reshape(B, T, H, d)
    kh = rms_norm(k_pre, k_gain, eps).reshape(B, T, G, d)
    vh = np.asarray(v, dtype=np.float64).reshape(B, T, G, d)
    return qh, kh, vh


def prefill_ref(q_pre, k_pre, v, q_gain, k_gain, *, H: int, G: int, d: int,
                kind: str, window: int, rope: RopeParams, eps: float = 1e-6,
                pos_offset: int = 0, cache: KvCacheRef | None = None,
                round_rotated: bool = False, q_scale: float = 1.0) -> np.ndarray:
    """One attention call over T new tokens at positions pos_offset .. +T-1.

    q_pre [B, T, H*d], k_pre and v [B, T, G*d] (projected, before QK-norm);
    returns out [B, T, H*d] (heads concatenated in head order).

    Steps in the order of page "Olmo-3 End-to-End Implementation", "Cache
    Operation Flow": the keys attended to are the cache's previous contents
    (if any) together with the new keys; new queries and keys are rotated at
    their absolute positions; attention runs under the mask; the new keys and
    values are then stored.  On a cache holding unrotated keys, each cached
    key is rotated by its own absolute position when it is read.

    ``round_rotated``: every rotated query and key (cached keys rotated on
    reading included) is rounded to bfloat16 before the scores, as a model
    computing in bfloat16 holds them.  With large QK-norm gains the scores
    grow with the gains and that rounding moves outputs by more than the
    fp32 accumulation does; it is off by default.  ``q_scale`` (with
    ``round_rotated``): the queries are rounded as q_scale times their value
    and divided by q_scale after, as a model that holds its queries times
    its softmax scale in bfloat16 does; 1 rounds the queries themselves.
    """
    q_pre = np.asarray(q_pre, dtype=np.float64)
    B, T = q_pre.shape[:2]
    qh, kh, vh = _project_heads(q_pre, k_pre, v, q_gain, k_gain, H, G, d, eps)
    w, m = layer_rope(rope, kind, d)
    positions = pos_offset + np.arange(T, dtype=np.int64)
    rnd = bf16_round if round_rotated else (lambda t: t)
    q_rot = rope_rotate(qh, positions, w, m)
    if round_rotated:
        q_rot = bf16_round(q_rot * q_scale) / q_scale
    k_rot = rnd(rope_rotate(kh, positions, w, m))

    if cache is not None:
        past_k, past_v, past_pos = cache.contents()
        if not cache.rotated and past_pos.size:
            past_k = rnd(rope_rotate(past_k, past_pos, w, m))
    else:
        past_k = np.zeros((B, 0, G, d))
        past_v = np.zeros((B, 0, G, d))
        past_pos = np.zeros(0, dtype=np.int64)

    keys = np.concatenate([past_k, k_rot], axis=1)
    vals = np.concatenate([past_v, vh], axis=1)
    key_pos = np.concatenate([past_pos, positions])

    out = np.zeros((B, T, H, d))
    for b in range(B):
        out[b] = attend(q_rot[b], positions, keys[b], vals[b], key_pos, kind, window)

    if cache is not None:
        cache.append(k_rot if cache.rotated else kh, vh, positions)
    return out.reshape(B, T, H * d)


def decode_ref(q_pre, k_pre, v, q_gain, k_gain, *, H: int, G: int, d: int,
               kind: str, window: int, rope: RopeParams, eps: float = 1e-6,
               pos: int, cache: KvCacheRef, round_rotated: bool = False) -> np.ndarray:
    """Single-token decode: the prefill computation with T = 1 at position
    ``pos`` against the cache (page "Olmo-3 End-to-End Implementation",
    "Inference Pipeline": generate one token at a time, reuse the cache).
    q_pre [B, H*d], k_pre and v [B, G*d]; returns [B, H*d]."""
    q_pre = np.asarray(q_pre, dtype=np.float64)[:, None, :]
    k_pre = np.asarray(k_pre, dtype=np.float64)[:, None, :]
    v = np.asarray(v, dtype=np.float64)[:, None, :]
    out = prefill_ref(q_pre, k_pre, v, q_gain, k_gain, H=H, G=G, d=d, kind=kind,
                      window=window, rope=rope, eps=eps, pos_offset=pos, cache=cache,
                      round_rotated=round_rotated)
    return out[:, 0, :]


def decode_e4m3_ref(q_pre, k_pre, v, q_gain, k_gain, *, H: int, G: int, d: int,
                    kind: str, window: int, rope: RopeParams, eps: float = 1e-6,
                    pos: int, cache: KvCacheRef, round_rotated: bool = False) -> np.ndarray:
    """Single-token decode against an e4m3 cache: the token's rotated key and
    its value are stored as codes at the slot of ``pos`` first, and the query
    then attends to the cache as stored, the new token's dequantized key and
    value included.  q_pre [B, H*d], k_pre and v [B, G*d]; returns [B, H*d].
    ``round_rotated``: the rotated query is rounded to bfloat16 before the
    scores, as in ``prefill_ref`` (the keys are the codes' values, which
    bfloat16 holds exactly)."""
    if cache.e4m3_scales is None:
        raise ValueError("decode_e4m3_ref needs a cache with e4m3 storage")
    q_pre = np.asarray(q_pre, dtype=np.float64)[:, None, :]
    k_pre = np.asarray(k_pre, dtype=np.float64)[:, None, :]
    v = np.asarray(v, dtype=np.float64)[:, None, :]
    B = q_pre.shape[0]
    qh, kh, vh = _project_heads(q_pre, k_pre, v, q_gain, k_gain, H, G, d, eps)
    w, m = layer_rope(rope, kind, d)
    p = np.array([pos], dtype=np.int64)
    q_rot = rope_rotate(qh, p, w, m)
    if round_rotated:
        q_rot = bf16_round(q_rot)
    cache.append(rope_rotate(kh, p, w, m), vh, p)
    keys, vals, key_pos = cache.contents()
    out = np.zeros((B, 1, H, d))
    for b in range(B):
        out[b] = attend(q_rot[b], p, keys[b], vals[b], key_pos, kind, window)
    return out.reshape(B, H * d)


def attention_rows_ref(q_pre_rows, q_rows_pos, k_pre_keys, v_keys, k_keys_pos,
                       q_gain, k_gain, *, H: int, G: int, d: int, kv_heads,
                       kind: str, window: int, rope: RopeParams,
                       eps: float = 1e-6, k_is_rotated: bool = False) -> np.ndarray:
    """Outputs of selected query rows and selected key/value heads of ONE
    sequence, for checks at sizes where the whole output is too costly.

    q_pre_rows [R, H*d] are the full projected query vectors of the sampled
    rows (the norm needs every feature); k_pre_keys [N, G*d] the full
    projected key vectors of the keys (or, with ``k_is_rotated``, the already
    rotated keys [N, G, d] read back from a cache filled from host data),
    v_keys [N, G, d]; ``kv_heads`` lists the key/value heads to evaluate.
    Returns [R, len(kv_heads) * H/G, d] for the query heads of those groups,
    in head order.  Same steps as ``prefill_ref``.
    """
    group = H // G
    w, m = layer_rope(rope, kind, d)
    q_pre_rows = np.asarray(q_pre_rows, dtype=np.float64)
    R = q_pre_rows.shape[0]
    qh = rms_norm(q_pre_rows, q_gain, eps).reshape(R, H, d)
    q_rot = rope_rotate(qh, q_rows_pos, w, m)
    kv_heads = list(kv_heads)
    if k_is_rotated:
        sub_k = np.asarray(k_pre_keys, dtype=np.float64)[:, kv_heads, :]
    else:
        N = k_pre_keys.shape[0]
        kh = rms_norm(np.asarray(k_pre_keys, dtype=np.float64), k_gain, eps).reshape(N, G, d)
        sub_k = rope_rotate(kh[:, kv_heads, :], k_keys_pos, w, m)
    heads = [g * group + j for g in kv_heads for j in range(group)]
    sub_q = q_rot[:, heads, :]
    sub_v = np.asarray(v_keys, dtype=np.float64)[:, kv_heads, :]
    return attend(sub_q, np.asarray(q_rows_pos), sub_k, sub_v,
                  np.asarray(k_keys_pos), kind, window)


def ring_positions(kind: str, window: int, capacity: int, pos: int) -> np.ndarray:
    """Absolute position held by each slot of a cache into which positions
    0 .. pos-1 have been appended (-1 = empty): slot s holds s on a linear
    cache, and on a ring the latest p < pos with p mod window == s."""
    slots = np.arange(capacity, dtype=np.int64)
    if kind == FULL:
        return np.where(slots < pos, slots, -1)
    held = (pos - 1) - ((pos - 1 - slots) % window)
    return np.where((slots < window) & (held >= 0), held, -1)


def decode_rows_ref(q_pre_b, k_pre_b, v_b, q_gain, k_gain, cache_k, cache_v, cache_pos, *,
                    H: int, G: int, d: int, kv_heads, kind: str, window: int,
                    rope: RopeParams, eps: float = 1e-6, pos: int) -> np.ndarray:
    """Decode of ONE sequence, evaluated for the query heads of ``kv_heads``
    only, for checks where the whole cache is too large for the host.

    q_pre_b [H*d], k_pre_b and v_b [G*d] are the token's full projected
    vectors (QK-norm needs every feature); cache_k, cache_v
    [len(kv_heads), capacity, d] are those heads' cache rows before the call
    (rotated keys) and cache_pos [capacity] the position each slot holds.
    Steps as ``decode_ref``: normalise and rotate the new query and key at
    ``pos``, store key and value at the slot of ``pos``, attend over the
    filled slots.  Returns [len(kv_heads) * H/G, d] in head order.
    """
    group = H // G
    kv_heads = list(kv_heads)
    w, m = layer_rope(rope, kind, d)
    qh = rms_norm(np.asarray(q_pre_b, dtype=np.float64)[None], q_gain, eps).reshape(1, H, d)
    kh = rms_norm(np.asarray(k_pre_b, dtype=np.float64)[None], k_gain, eps).reshape(1, G, d)
    p = np.array([pos], dtype=np.int64)
    q_rot = rope_rotate(qh, p, w, m)
    k_rot = rope_rotate(kh, p, w, m)
    slot = pos % window if kind == SLIDING else pos
    ck = np.array(cache_k, dtype=np.float64)
    cv = np.array(cache_v, dtype=np.float64)
    cp = np.array(cache_pos, dtype=np.int64)
    ck[:, slot] = k_rot[0, kv_heads]
    cv[:, slot] = np.asarray(v_b, dtype=np.float64).reshape(G, d)[kv_heads]
    cp[slot] = pos
    filled = cp >= 0
    heads = [g * group + j for g in kv_heads for j in range(group)]
    keys = ck[:, filled].transpose(1, 0, 2)
    vals = cv[:, filled].transpose(1, 0, 2)
    return attend(q_rot[0][None, heads].reshape(1, len(heads), d), p, keys, vals,
                  cp[filled], kind, window)[0]
