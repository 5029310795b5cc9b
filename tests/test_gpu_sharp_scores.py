"""GPU parity at sharp softmax: QK-norm gains of 3 scale every score by 9
(by about 13 with the YaRN temperature on full layers), so row maxima jump
by more than the kernels' lazy-rescale slack many times per row, and the
rescale branches of the prefill and both decode kernels run often.

At such scores the bfloat16 rounding of the rotated queries and keys (they
are stored and multiplied in bf16) moves outputs by more than the fp32
accumulation does, so the oracle is asked for the same rounding
(``round_rotated``) and the tolerance stays the ordinary one."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from gpu_util import (KINDS, assert_close, gpu_decode, gpu_prefill, host, host_inputs, inputs,
                      oracle_rope, prefill_q_scale)

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
GAIN = 3.0


@pytest.mark.parametrize("chunks", [(1296,), (700, 596)])
@pytest.mark.parametrize("H,G", [(4, 4), (8, 2)])
@pytest.mark.parametrize("lt", [0, 1])
def test_sharp_scores_prefill_then_decode(H, G, lt, chunks):
    """Prefill of 1,296 tokens (ten 128-query blocks and a ragged tail; the
    sliding layer's 512-slot ring wraps twice), whole or as a first chunk of
    700 and a second of 596 that also attends to the cache, then four decode
    steps, with every gain 3; one key/value head per query head takes the
    vector decode kernel, four query heads per key/value head the MFMA one."""
    B, T, T0, d, w = 1, 1300, sum(chunks), 128, 512
    kind = KINDS[lt]
    print(f"sharp scores H={H} G={G} {kind} chunks={chunks}", flush=True)
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=256)
    x = inputs(7, lt, B, T, H, G, d, BF16)
    x["q_gain"] = torch.full_like(x["q_gain"], GAIN)
    x["k_gain"] = torch.full_like(x["k_gain"], GAIN)
    cap = w if kind == O.SLIDING else T
    kc = torch.zeros((B, G, cap, d), dtype=BF16, device="cuda")
    vc = torch.zeros_like(kc)
    hx = host_inputs(x)
    c = O.KvCacheRef(kind, w, cap, B, G, d)
    p0 = 0
    for n in chunks:
        pre = {k: (v[:, p0:p0 + n].contiguous() if v.dim() == 3 else v) for k, v in x.items()}
        out = gpu_prefill(pre, kc, vc, window=w, layer_type=lt, rope=rope, H=H, pos_offset=p0)
        hpre = {k: (v[:, p0:p0 + n] if v.ndim == 3 else v) for k, v in hx.items()}
        ref = O.prefill_ref(**hpre, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                            pos_offset=p0, cache=c, round_rotated=True,
                            q_scale=prefill_q_scale(d))
        err = assert_close(host(out), ref, what=f"sharp prefill {kind} at {p0}")
        print(f"  prefill at {p0} max err", err, flush=True)
        p0 += n
    for p in range(T0, T):
        o = gpu_decode(x["q_pre"][:, p].contiguous(), x["k_pre"][:, p].contiguous(),
                       x["v"][:, p].contiguous(), x["q_gain"], x["k_gain"], kc, vc, window=w,
                       layer_type=lt, rope=rope, pos=p, H=H)
        r = O.decode_ref(hx["q_pre"][:, p], hx["k_pre"][:, p], hx["v"][:, p], hx["q_gain"],
                         hx["k_gain"], H=H, G=G, d=d, kind=kind, window=w,
                         rope=oracle_rope(rope), pos=p, cache=c, round_rotated=True)
        assert_close(host(o), r, what=f"sharp decode {kind} p={p}")
