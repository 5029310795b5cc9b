"""The prefill kernel's work order, read through the library's host probe
(`olmo3_probe_prefill_order`, the kernel's own functions run on the host).

Every (sequence, head, query block, key split) must be taken by exactly one
workgroup, or some output rows would never be written.  Beyond that the
order is a performance choice, pinned here by its stated properties:
workgroups are dealt round-robin over the 8 XCDs (workgroup i on XCD
i mod 8), every (sequence, head) keeps its blocks on one XCD when the pairs
split evenly over them, and each XCD starts its longest blocks first."""

import random

import numpy as np
import pytest

from global_hybrid_causal_amd import attn as A

SLIDING, FULL = A.LAYER_SLIDING, A.LAYER_FULL
BQ = 128

CASES = [
    # B, T, H, G, window, layer_type, pos_offset, kv_splits
    (1, 8192, 32, 32, 4096, SLIDING, 0, 1),   # 7B layer
    (1, 8192, 32, 32, 4096, FULL, 0, 1),
    (1, 8192, 40, 8, 4096, SLIDING, 0, 1),    # 32B layer
    (1, 8192, 40, 8, 4096, FULL, 0, 1),
    (1, 65536, 32, 32, 4096, SLIDING, 0, 1),  # long-context stack: one head after another
    (1, 65536, 32, 32, 4096, FULL, 0, 1),
    (1, 4096, 32, 32, 4096, SLIDING, 61440, 1),  # a later chunk: every window full
    (1, 4096, 32, 32, 4096, FULL, 61440, 1),
    (1, 2048, 32, 32, 700, SLIDING, 0, 1),
    (1, 2048, 32, 8, 700, SLIDING, 0, 1),
    (1, 8192, 4, 4, 4096, FULL, 0, 2),        # head shard: the key-split instance
    (1, 300, 4, 4, 64, SLIDING, 0, 2),
    (1, 130, 64, 64, 64, SLIDING, 0, 2),
    (2, 700, 10, 2, 200, SLIDING, 0, 1),
    (3, 2100, 2, 1, 256, SLIDING, 0, 1),
]


def _random_cases(n=40, seed=5):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        G = rng.choice([1, 2, 4, 8, 16])
        H = G * rng.choice([1, 2, 5, 8])
        out.append((rng.choice([1, 2, 3]), rng.randint(1, 5000), H, G, rng.choice([1, 100, 4096, 1 << 30]),
                    rng.choice([SLIDING, FULL]), rng.choice([0, 0, 1000, 70000]), rng.choice([1, 2])))
    return out


def _full_window_first(T, window, pos_offset, layer_type, H, G):
    """Blocks whose sliding windows are full (kept head after head first on a
    layer with one query head per key/value head)."""
    nq = -(-T // BQ)
    if layer_type != SLIDING or H != G:
        return 0
    first = max(0, -(-(window - 1 - pos_offset) // BQ))
    return 0 if first >= nq else nq - first


@pytest.mark.parametrize("case", CASES + _random_cases(), ids=str)
def test_every_block_once_and_longest_first(case):
    B, T, H, G, window, lt, P, splits = case
    work = A.olmo3_probe_prefill_order(B, T, H, G, window, lt, P, splits).numpy()
    nq = -(-T // BQ)
    n = nq * H * B * splits
    assert work.shape == (n, 4)
    # a bijection onto (sequence, head, query block, split)
    key = ((work[:, 0] * H + work[:, 1]) * nq + work[:, 2]) * splits + work[:, 3]
    assert (work[:, 0] >= 0).all() and (work[:, 0] < B).all()
    assert (work[:, 1] >= 0).all() and (work[:, 1] < H).all()
    assert (work[:, 2] >= 0).all() and (work[:, 2] < nq).all()
    assert (work[:, 3] >= 0).all() and (work[:, 3] < splits).all()
    assert np.array_equal(np.sort(key), np.arange(n))
    # dispatch order: XCD by XCD (workgroups x, x + 8, ...), as the order is
    # laid out, when the grid splits evenly over the XCDs
    order = (np.concatenate([np.arange(x, n, 8) for x in range(8)]) if n % 8 == 0
             else np.arange(n))
    if splits > 1:  # the two splits of a block are neighbours in that order
        w = work[order]
        assert (w[0::2, :3] == w[1::2, :3]).all()
        assert (w[0::2, 3] == 0).all() and (w[1::2, 3] == 1).all()
    BH = B * H
    if BH % 8:
        return
    xcd = np.arange(n) % 8
    pair = work[:, 0] * H + work[:, 1]
    for p in np.unique(pair):  # every (sequence, head) on one XCD ...
        assert np.unique(xcd[pair == p]).size == 1
    k = BH // 8  # ... and XCD x holds pairs x k .. x k + k - 1
    assert ((pair // k) == xcd).all()
    interleaved = nq * BH <= 8192
    n_even = _full_window_first(T, window, P, lt, H, G) if interleaved else nq
    for x in range(8):
        qb = work[xcd == x, 2][::splits]   # the XCD's blocks in dispatch order
        pr = pair[xcd == x][::splits]
        head = k * n_even
        # first the full-window blocks (or, in large grids, every block) pair
        # after pair, each pair's longest first ...
        for p in np.unique(pr[:head]):
            seq = qb[:head][pr[:head] == p]
            assert (np.diff(seq) < 0).all(), (x, p)
        assert (qb[:head] >= nq - n_even).all()
        # ... then the rest longest first over all the XCD's pairs
        assert (np.diff(qb[head:]) <= 0).all(), x


def test_probe_rejects_bad_arguments():
    L = A.lib()
    buf = (A.ctypes.c_int32 * 16)()
    assert L.olmo3_probe_prefill_order(1, 128, 4, 4, 64, SLIDING, 0, 3, buf, 16) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_order(1, 128, 4, 4, 64, SLIDING, 0, 1, buf, 15) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_order(1, 128, 4, 3, 64, SLIDING, 0, 1, buf, 16) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_order(1, 128, 4, 4, 64, 7, 0, 1, buf, 16) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_order(1, 128, 4, 4, 64, SLIDING, 0, 1, None, 16) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_order(1, 128, 4, 4, 64, SLIDING, 0, 1, buf, 16) == A.OK
