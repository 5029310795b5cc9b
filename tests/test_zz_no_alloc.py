"""The decode entry point that allocates nothing (olmo3_attn_decode_noalloc,
for callers that cannot allocate device memory): through the C-ABI, on two
calls in a row, the second smaller than the first, it gives the bits of
olmo3_attn_decode with a workspace of its own on the same inputs, in the
outputs and in the caches."""

import pytest
import torch

from global_hybrid_causal_amd import attn as A
from global_hybrid_causal_amd import synth
from gpu_util import inputs

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32

CALLS = [
    # B, H, G, window, layer_type, pos, cap, dtype: the first call is the largest
    (8, 32, 8, 4096, 1, 6000, 6001, BF16),    # split rows over workgroups, merged
    (2, 16, 4, 512, 0, 700, 512, BF16),       # ring, fewer rows and sequences
    (1, 4, 4, 64, 0, 3, 64, F32),             # fp32: the per-query kernel
]


def _one(case, seed):
    B, H, G, w, lt, pos, cap, dt = case
    d = 128
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=4096)
    kc0, vc0 = synth.cache_fill(seed, lt, B, G, cap, d, device="cuda", dtype=dt)
    x = inputs(seed, 90 + lt, B, 1, H, G, d, dt)
    q, k, v = (x[n][:, 0].contiguous() for n in ("q_pre", "k_pre", "v"))
    kw = dict(window=w, layer_type=lt, rope=rope, pos=pos)
    kc_a, vc_a = kc0.clone(), vc0.clone()
    out_a = torch.full_like(q, 5.0)
    ws = A.workspace(A.MODE_DECODE, B, 1, H, G, d, lt, dt, cap, "cuda")
    A.olmo3_attn_decode(q, k, v, x["q_gain"], x["k_gain"], kc_a, vc_a, out_a, ws, **kw)
    kc_b, vc_b = kc0.clone(), vc0.clone()
    out_b = torch.full_like(q, -5.0)
    A.olmo3_attn_decode_noalloc(q, k, v, x["q_gain"], x["k_gain"], kc_b, vc_b, out_b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), case
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b), case
    assert torch.isfinite(out_b.float()).all()


def test_noalloc_decode_equals_decode_on_calls_in_a_row():
    for i, case in enumerate(CALLS):
        print("no-alloc decode", case, flush=True)
        _one(case, 101 + i)
