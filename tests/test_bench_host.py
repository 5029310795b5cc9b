"""Host-side logic of bench.py, without a GPU: the algorithmic work it
divides by (checked against the oracle's explicit masks and cache
accounting), the refusal of more than one GPU, and the guard that drops a
recorded traffic figure once its kernel's sources change."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("T,window", [(1, 4), (5, 2), (64, 16), (300, 64), (257, 1000), (4096, 4096)])
def test_prefill_pairs_count_the_mask(T, window):
    assert bench.prefill_pairs(T, window, True) == int(O.sliding_window_mask(T, window).sum())
    assert bench.prefill_pairs(T, window, False) == int(O.causal_mask(T).sum())


def test_prefill_flops_at_the_7b_config():
    # 4 * d * H per allowed pair: 4.1235e11 (sliding) and 5.4982e11 (full) at T = 8192
    assert bench.prefill_flops(8192, 32, 128, 4096, True) == 412350414848
    assert bench.prefill_flops(8192, 32, 128, 4096, False) == 549822922752


def test_decode_bytes_match_the_cache_accounting():
    kinds = O.layer_types(32)
    L, G, d = 65536, 32, 128
    per_seq = sum(bench.decode_kv_bytes(1, G, d, bench.decode_rows(L - 1, 4096, k == O.SLIDING))
                  for k in kinds)
    assert per_seq // L == O.kv_bytes_per_token(kinds, G, d, 4096, L) == 155648
    assert bench.decode_kv_bytes(32, 32, 128, 65536) == 34359738368
    assert bench.decode_kv_bytes(32, 32, 128, 65536, elem=1) == 34359738368 // 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_recorded_traffic_needs_unchanged_sources(monkeypatch):
    key = ("7b/decode_full", "decode_split_kernel")
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key, dict(bytes=123, sources="0" * 16))
    assert bench.measured_traffic(*key) is None
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key,
                        dict(bytes=123, sources=bench.sources_digest("decode_split_kernel")))
    assert bench.measured_traffic(*key) == 123
    assert bench.measured_traffic("7b/no such group", "decode_split_kernel") is None


def test_every_recorded_traffic_figure_is_current():
    """A figure whose kernel's sources changed since it was measured is
    reported null; the table keeps only current ones."""
    for (group, kernel), entry in bench.MEASURED_TRAFFIC.items():
        assert bench.sources_digest(kernel) == entry["sources"], (group, kernel)


def test_prologue_bytes():
    # 7B sliding prefill at T = 8192: read q, k, v (3 x 64 MiB), write rotated q
    # (64 MiB), the ring's 4096 kept rows of k and v (2 x 32 MiB) and the
    # rotated-key copy (64 MiB)
    mib = 1 << 20
    assert bench.prefill_prologue_bytes(1, 8192, 32, 32, 128, True) == (3 * 64 + 64 + 64 + 64) * mib
    assert bench.prefill_prologue_bytes(1, 8192, 32, 32, 128, False) == (3 * 64 + 64 + 128) * mib
    assert bench.decode_prologue_bytes(32, 32, 32, 128) == 32 * (96 + 32 + 64) * 128 * 2


def test_workload_list_is_parsed(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "7b,32b"])
    assert bench.parse().workloads == ["7b", "32b"]
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().workloads == ["7b", "32b", "long"]
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "7b,nope"])
    with pytest.raises(SystemExit):
        bench.parse()


def test_decode_kernel_label():
    assert bench.decode_kernel(32, 32, False) == "decode_split_kernel"
    assert bench.decode_kernel(40, 8, False) == "decode_mfma_kernel"
    assert bench.decode_kernel(40, 8, True) == "decode_split_kernel"
    assert bench.decode_kernel(32, 32, True) == "decode_split_kernel"


def test_chunk_pairs_brute_force():
    """Allowed pairs of a chunk at an offset: the closed form against a count
    over the chunk's queries."""
    for P, T, w in [(0, 100, 64), (10, 100, 64), (60, 10, 64), (3, 5, 4), (61440, 4096, 4096),
                    (4000, 200, 4096)]:
        for sliding in (True, False):
            want = sum(min(t + 1, w) if sliding else t + 1 for t in range(P, P + T))
            assert bench.chunk_pairs(P, T, w, sliding) == want
    # offset 0 agrees with the whole-prefill count
    assert bench.chunk_pairs(0, 8192, 4096, True) == bench.prefill_pairs(8192, 4096, True)
    assert bench.chunk_pairs(0, 8192, 4096, False) == bench.prefill_pairs(8192, 4096, False)
