"""How far the QK-norm gains can grow before the fp64 oracle and the kernels
part: the configurations draw gains from U(0.5, 1.5); here they are scaled
by up to 6.  The kernels hold the rotated queries and keys in bfloat16
(page "Olmo-3 End-to-End Implementation", "Technical Details": bfloat16
throughout), which moves every score by a relative 2^-9 of its terms; the
scores grow with the square of the gains (and with the YaRN temperature on
full layers), so past the configurations' range (1x) the default oracle,
which rounds nothing, is no longer within the output tolerance everywhere
(at 1.5x a few elements per million leave it).  The oracle with its
``round_rotated`` switch holds the same bfloat16 operands (the prefill
kernel's queries times its softmax scale, ``q_scale``) and stays within
it, save a few elements per hundred thousand where a rotated value that
lies at a bfloat16 midpoint rounds the other way in the kernel's fp32
arithmetic (the queries' product by the softmax scale included) and the
large scores magnify that one step."""

import numpy as np
import pytest
import torch

import oracle as O
from global_hybrid_causal_amd import attn as A
from gpu_util import (ATOL, KINDS, RTOL, gpu_prefill, host, host_inputs, inputs, oracle_rope,
                      prefill_q_scale)

pytestmark = pytest.mark.gpu

B, T, H, G, d = 1, 1024, 8, 8, 128


def _beyond(out, ref):
    return float((np.abs(out - ref) > ATOL + RTOL * np.abs(ref)).mean())


@pytest.mark.parametrize("lt", [0, 1], ids=["sliding", "full_yarn"])
@pytest.mark.parametrize("gain", [1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
def test_prefill_gain_range(lt, gain):
    kind = KINDS[lt]
    w = 256 if lt == 0 else 4096
    rope = A.Rope(theta=500000.0, yarn=lt == 1, factor=8.0, orig_ctx=256)
    x = inputs(81, lt, B, T, H, G, d, torch.bfloat16)
    x["q_gain"] = (x["q_gain"].float() * gain).to(torch.bfloat16)
    x["k_gain"] = (x["k_gain"].float() * gain).to(torch.bfloat16)
    cap = w if lt == 0 else T
    kc = torch.zeros((B, G, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    out = host(gpu_prefill(x, kc, vc, window=w, layer_type=lt, rope=rope, H=H))
    hx = host_inputs(x)
    refs = [O.prefill_ref(**hx, H=H, G=G, d=d, kind=kind, window=w, rope=oracle_rope(rope),
                          round_rotated=rr, q_scale=prefill_q_scale(d)) for rr in (False, True)]
    plain, rounded = _beyond(out, refs[0]), _beyond(out, refs[1])
    print(f"gain x{gain} {kind}: beyond tolerance {plain:.2e} (default oracle), "
          f"{rounded:.2e} (rotated q/k rounded to bf16)", flush=True)
    if gain == 1.0:
        assert plain == 0.0
    assert rounded <= 3e-5
