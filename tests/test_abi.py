"""The C-ABI library on the CPU: it loads, exports every symbol its header
declares, and rejects every invalid argument with its status code before
anything reaches the device.  No compute call is made here: invalid calls
use stand-in pointer values that are never dereferenced."""

import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "olmo3_attn.h")

A = pytest.importorskip("global_hybrid_causal_amd.attn")

if not os.path.exists(A.LIB_PATH):
    pytest.skip("libolmo3attn.so not built", allow_module_level=True)


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(olmo3_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = header_symbols()
    assert len(syms) >= 9
    L = ctypes.CDLL(A.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), f"{s} declared in the header but not exported"
    assert sorted(A.EXPORTS) == syms


def test_header_binding_and_library_versions_agree():
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "olmo3_attn.h")).read()
    header = int(re.search(r"#define OLMO3_ABI_VERSION (\d+)", text).group(1))
    assert header == A.ABI_VERSION == A.olmo3_abi_version()


def test_abi_version():
    assert A.olmo3_abi_version() == A.ABI_VERSION == 11


def test_layer_type_matches_oracle_bit_exact():
    for n in range(1, 80):
        want = [O.layer_type_code(k) for k in O.layer_types(n)]
        assert [A.olmo3_layer_type(i, n) for i in range(n)] == want
    assert A.olmo3_layer_type(-1, 4) == -1
    assert A.olmo3_layer_type(4, 4) == -1
    assert A.olmo3_layer_type(0, 0) == -1


def test_status_strings():
    for s in range(6):
        assert A.status_string(s)
    assert A.status_string(99) == "unknown status"


def test_workspace_bytes_split_partials():
    """Full layers with fewer than 512 query blocks x heads x sequences, and
    sliding layers with at most 256, reserve two partial states (d + 2
    floats) per query row and head; larger grids none."""
    ws = A.olmo3_workspace_bytes
    q = 8192 * 4 * 128 * 2  # rotated queries, H = 4
    assert ws(A.MODE_PREFILL, 1, 8192, 4, 4, 128, 1, 0, 8192) >= q + 8192 * 4 * 2 * 130 * 4
    assert ws(A.MODE_PREFILL, 1, 8192, 8, 8, 128, 1, 0, 8192) < 2 * (2 * q)   # 512 blocks: none
    assert ws(A.MODE_PREFILL, 1, 8192, 8, 8, 128, 1, 0, 8192) >= 2 * q
    assert ws(A.MODE_PREFILL, 1, 64, 2, 1, 16, 1, 1, 64) == 64 * 2 * 16 * 4  # fp32 path: none
    # sliding layers split only while the doubled grid fits one round (<= 256 blocks)
    q5, k1 = 8192 * 5 * 128 * 2, 8192 * 1 * 128 * 2
    assert ws(A.MODE_PREFILL, 1, 8192, 5, 1, 128, 0, 0, 4096) == q5 + k1   # 320 blocks
    assert ws(A.MODE_PREFILL, 1, 8192, 5, 1, 128, 1, 0, 8192) > q5          # full layer splits
    assert ws(A.MODE_PREFILL, 1, 8192, 4, 4, 128, 0, 0, 4096) > 2 * q       # 256 blocks: splits


def test_workspace_bytes():
    ws = A.olmo3_workspace_bytes
    assert ws(A.MODE_PREFILL, 1, 8192, 32, 32, 128, 0, 0, 4096) >= 2 * 8192 * 4096 * 2
    assert ws(A.MODE_PREFILL, 1, 8192, 32, 32, 128, 1, 0, 8192) >= 8192 * 4096 * 2
    # sliding prefill also stages rotated keys
    assert ws(A.MODE_PREFILL, 1, 100, 4, 2, 128, 0, 0, 64) > ws(A.MODE_PREFILL, 1, 100, 4, 2, 128, 1, 0, 100)
    assert ws(A.MODE_DECODE, 32, 1, 32, 32, 128, 1, 0, 65536) > 32 * 32 * 128 * 2
    assert ws(A.MODE_PREFILL, 0, 8, 2, 1, 16, 0, 1, 16) == 0
    assert ws(A.MODE_PREFILL, 1, 8, 3, 2, 16, 0, 1, 16) == 0
    assert ws(A.MODE_DECODE, 1, 1, 2, 1, 16, 0, 1, 0) == 0
    assert ws(7, 1, 8, 2, 1, 16, 0, 1, 16) == 0


# ---- invalid arguments -------------------------------------------------
BASE = 1 << 44
SPACING = 1 << 38  # stand-in buffers far apart, 256-byte aligned


def fake(i):
    return BASE + i * SPACING


GOOD = dict(B=2, T=64, H=4, G=2, d=128, window=16, layer_type=0, eps=1e-6, pos_offset=0,
            dtype=0, cap=16)


def prefill_call(**kw):
    a = dict(GOOD)
    ptrs = {n: fake(i) for i, n in enumerate(
        ["q_pre", "k_pre", "v", "q_gain", "k_gain", "k_cache", "v_cache", "out", "workspace"])}
    ws_bytes = 1 << 34
    rope = A.Rope(theta=500000.0)
    for k in list(kw):
        if k in ptrs:
            ptrs[k] = kw.pop(k)
    if "rope" in kw:
        rope = kw.pop("rope")
    ws_bytes = kw.pop("ws_bytes", ws_bytes)
    a.update(kw)
    r = ctypes.byref(rope.to_c()) if rope is not None else None
    return A.lib().olmo3_attn_prefill(
        a["B"], a["T"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"],
        a["pos_offset"], a["dtype"], ptrs["q_pre"], ptrs["k_pre"], ptrs["v"], ptrs["q_gain"],
        ptrs["k_gain"], ptrs["k_cache"], ptrs["v_cache"], a["cap"], ptrs["out"], ptrs["workspace"],
        ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), A.ERR_INVALID_ARG),
    (dict(T=0), A.ERR_INVALID_ARG),
    (dict(H=3), A.ERR_INVALID_ARG),          # H % G != 0
    (dict(G=0), A.ERR_INVALID_ARG),
    (dict(d=127), A.ERR_INVALID_ARG),
    (dict(d=48), A.ERR_UNSUPPORTED),
    (dict(d=256), A.ERR_UNSUPPORTED),
    (dict(window=0), A.ERR_INVALID_ARG),
    (dict(layer_type=2), A.ERR_INVALID_ARG),
    (dict(dtype=3), A.ERR_INVALID_ARG),
    (dict(eps=-1.0), A.ERR_INVALID_ARG),
    (dict(eps=float("nan")), A.ERR_INVALID_ARG),
    (dict(pos_offset=-1), A.ERR_INVALID_ARG),
    (dict(rope=None), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=0.0)), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=1e4, yarn=True, factor=0.5)), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=1e4, yarn=True, beta_fast=1.0, beta_slow=32.0)), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=1e4, yarn=True, beta_fast=32.0, beta_slow=0.0)), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=1.0, yarn=True, factor=8.0)), A.ERR_INVALID_ARG),
    (dict(rope=A.Rope(theta=1e4, yarn=True, factor=float("inf"))), A.ERR_INVALID_ARG),
    (dict(q_pre=0), A.ERR_INVALID_ARG),
    (dict(out=0), A.ERR_INVALID_ARG),
    (dict(q_pre=fake(0) + 8), A.ERR_INVALID_ARG),   # misaligned
    (dict(out=fake(0) + 4096), A.ERR_INVALID_ARG),  # out overlaps q_pre
    (dict(v_cache=fake(5) + 256), A.ERR_INVALID_ARG),  # caches overlap
    (dict(workspace=fake(7)), A.ERR_INVALID_ARG),   # workspace overlaps out
    (dict(cap=17), A.ERR_CAPACITY),           # ring must equal window
    (dict(layer_type=1, cap=63), A.ERR_CAPACITY),   # linear cache shorter than T
    (dict(workspace=0), A.ERR_WORKSPACE),
    (dict(ws_bytes=100), A.ERR_WORKSPACE),
    (dict(layer_type=1, cap=100, pos_offset=40), A.ERR_CAPACITY),  # chunk past a linear cache
    (dict(pos_offset=(1 << 30) - 63), A.ERR_UNSUPPORTED),  # positions past 2^30
    (dict(H=40 * 8, G=8), A.ERR_UNSUPPORTED),  # too many heads for one wavefront's norm
    (dict(layer_type=1, cap=1 << 45), A.ERR_UNSUPPORTED),  # cache past 2^50 bytes
    (dict(layer_type=1, cap=(1 << 62) + 1), A.ERR_UNSUPPORTED),  # byte size would wrap 64 bits
])
def test_prefill_rejects(kw, status):
    assert prefill_call(**kw) == status


def decode_call(**kw):
    a = dict(GOOD, pos=100)
    a.pop("T")
    a.update(kw)
    ptrs = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=500000.0).to_c())
    return A.lib().olmo3_attn_decode(
        a["B"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"], a["pos"],
        a["dtype"], *ptrs[:7], a["cap"], ptrs[7], ptrs[8], a.get("ws_bytes", 1 << 34), None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=-1), A.ERR_INVALID_ARG),
    (dict(cap=15), A.ERR_CAPACITY),
    (dict(layer_type=1, cap=100), A.ERR_CAPACITY),  # needs pos + 1 slots
    (dict(ws_bytes=16), A.ERR_WORKSPACE),
    (dict(H=5, G=2), A.ERR_INVALID_ARG),
    (dict(layer_type=1, cap=(1 << 62) + 1), A.ERR_UNSUPPORTED),  # byte size would wrap 64 bits
])
def test_decode_rejects(kw, status):
    assert decode_call(**kw) == status


def decode_noalloc_call(**kw):
    a = dict(GOOD, pos=100)
    a.pop("T")
    a.update(kw)
    ptrs = [fake(i) for i in range(8)]
    for i, n in enumerate(["q_pre", "k_pre", "v", "q_gain", "k_gain", "k_cache", "v_cache", "out"]):
        if n in kw:
            ptrs[i] = kw[n]
    r = ctypes.byref(A.Rope(theta=500000.0).to_c())
    return A.lib().olmo3_attn_decode_noalloc(
        a["B"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"], a["pos"],
        a["dtype"], *ptrs[:7], a["cap"], ptrs[7], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=-1), A.ERR_INVALID_ARG),
    (dict(H=5, G=2), A.ERR_INVALID_ARG),
    (dict(dtype=2), A.ERR_INVALID_ARG),             # e4m3 caches have their own entry points
    (dict(q_pre=0), A.ERR_INVALID_ARG),
    (dict(out=fake(7) + 8), A.ERR_INVALID_ARG),     # misaligned
    (dict(cap=15), A.ERR_CAPACITY),
    (dict(layer_type=1, cap=100), A.ERR_CAPACITY),  # needs pos + 1 slots
    # more scratch than the library holds: 1024 sequences x 64 heads of a
    # 2^17-slot linear cache need about 51 MiB of partial states
    (dict(B=1024, H=64, G=8, layer_type=1, cap=1 << 17, pos=(1 << 17) - 1), A.ERR_WORKSPACE),
])
def test_decode_noalloc_rejects_before_the_device(kw, status):
    """Every argument error, and a call needing more than the scratch array,
    returns its status before the device is touched (no GPU here)."""
    assert decode_noalloc_call(**kw) == status


def test_decode_noalloc_scratch_bound_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define OLMO3_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == A.NOALLOC_SCRATCH_BYTES
    B, H, G, d, cap = 1024, 64, 8, 128, 1 << 17
    assert A.olmo3_workspace_bytes(A.MODE_DECODE, B, 1, H, G, d, 1, A.DTYPE_BF16, cap) > \
        A.NOALLOC_SCRATCH_BYTES
    # the 7B and 32B decode batches fit
    for H, G in ((32, 32), (40, 8)):
        assert A.olmo3_workspace_bytes(A.MODE_DECODE, 32, 1, H, G, d, 1, A.DTYPE_BF16, 65536) <= \
            A.NOALLOC_SCRATCH_BYTES


def append_call(**kw):
    a = dict(B=2, T=8, G=2, d=64, window=16, layer_type=1, eps=1e-6, pos=0, dtype=0, cap=8)
    a.update(kw)
    p = [fake(i) for i in range(5)]
    if "k_cache" in kw:
        p[3] = kw["k_cache"]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_kv_append(a["B"], a["T"], a["G"], a["d"], a["window"], a["layer_type"],
                                   r, a["eps"], a["pos"], a["dtype"], *p, a["cap"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cap=7), A.ERR_CAPACITY),
    (dict(pos=1), A.ERR_CAPACITY),
    (dict(layer_type=0, cap=8), A.ERR_CAPACITY),
    (dict(k_cache=fake(0)), A.ERR_INVALID_ARG),  # cache overlaps an input
    (dict(d=24), A.ERR_UNSUPPORTED),
    (dict(cap=(1 << 62) + 1), A.ERR_UNSUPPORTED),  # byte size would wrap 64 bits
])
def test_append_rejects(kw, status):
    assert append_call(**kw) == status


def test_probe_rejects():
    L = A.lib()
    assert L.olmo3_probe_prefill_visits(0, 0, 4, 0, 1, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_visits(5, -1, 4, 0, 1, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_prefill_visits(5000, 0, 4, 0, 1, fake(0), None) == A.ERR_UNSUPPORTED
    assert L.olmo3_probe_prefill_visits(100, 8100, 4, 0, 1, fake(0), None) == A.ERR_UNSUPPORTED
    for bad in (0, 3, 4):
        assert L.olmo3_probe_prefill_visits(5, 0, 4, 0, bad, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_decode_reads(1, 1, 1, 64, 4, 0, 0, 3, 4, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_decode_reads(1, 3, 2, 128, 4, 0, 0, 3, 4, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_decode_reads(1, 2, 1, 128, 4, 0, 1, 3, 4, fake(0), None) == A.ERR_INVALID_ARG
    assert L.olmo3_probe_decode_reads(1, 1, 1, 128, 4, 1, 0, 3, (1 << 62) + 1, fake(0),
                                      None) == A.ERR_UNSUPPORTED
    assert L.olmo3_probe_decode_reads(1, 1, 1, 128, 4, 0, 0, 3, 5, fake(0), None) == A.ERR_CAPACITY


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 4, 32, dtype=torch.bfloat16)
    c = torch.zeros(1, 1, 4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.olmo3_kv_append(x, x, torch.zeros(32, dtype=torch.bfloat16), c, c.clone(), window=4,
                          layer_type=0, rope=A.Rope())


def test_phases_reject_bad_bits():
    L = A.lib()
    r = ctypes.byref(A.Rope().to_c())
    p = [fake(i) for i in range(9)]
    for ph in (0, 8, -1):
        assert L.olmo3_attn_prefill_phases(ph, 1, 8, 2, 1, 128, 4, 0, r, 1e-6, 0, 0, *p[:7], 4, p[7], p[8],
                                           1 << 30, None) == A.ERR_INVALID_ARG
        assert L.olmo3_attn_decode_phases(ph, 1, 2, 1, 128, 4, 0, r, 1e-6, 3, 0, *p[:7], 4, p[7], p[8],
                                          1 << 30, None) == A.ERR_INVALID_ARG


def ragged_prefill_call(**kw):
    a = dict(B=3, N=64, max_len=40, max_end=100, H=4, G=2, d=128, window=16, layer_type=0,
             eps=1e-6, dtype=0, cap=16, cu=fake(9), pos=fake(10))
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_prefill_ragged(
        a["B"], a["N"], a["max_len"], a["max_end"], a["H"], a["G"], a["d"], a["window"],
        a["layer_type"], r, a["eps"], a["cu"], a["pos"], a["dtype"], *p[:7], a["cap"], p[7], p[8],
        1 << 34, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), A.ERR_INVALID_ARG),
    (dict(N=0), A.ERR_INVALID_ARG),
    (dict(max_len=0), A.ERR_INVALID_ARG),
    (dict(max_len=65), A.ERR_INVALID_ARG),        # longer than all rows
    (dict(max_end=39), A.ERR_INVALID_ARG),        # shorter than the longest sequence
    (dict(cu=0), A.ERR_INVALID_ARG),
    (dict(cu=fake(9) + 2), A.ERR_INVALID_ARG),    # misaligned device array
    (dict(pos=fake(10) + 1), A.ERR_INVALID_ARG),
    (dict(cap=17), A.ERR_CAPACITY),               # ring must equal window
    (dict(layer_type=1, cap=99), A.ERR_CAPACITY),  # linear cache shorter than max_end
    (dict(max_end=(1 << 30) + 1), A.ERR_UNSUPPORTED),
    (dict(H=3), A.ERR_INVALID_ARG),
])
def test_ragged_prefill_rejects(kw, status):
    assert ragged_prefill_call(**kw) == status


def ragged_decode_call(**kw):
    a = dict(B=3, H=4, G=2, d=128, window=16, layer_type=0, eps=1e-6, pos=fake(10), max_pos=50,
             dtype=0, cap=16)
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_decode_ragged(
        a["B"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"], a["pos"],
        a["max_pos"], a["dtype"], *p[:7], a["cap"], p[7], p[8], 1 << 34, None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=0), A.ERR_INVALID_ARG),
    (dict(pos=fake(10) + 2), A.ERR_INVALID_ARG),
    (dict(max_pos=-1), A.ERR_INVALID_ARG),
    (dict(max_pos=1 << 31), A.ERR_INVALID_ARG),
    (dict(layer_type=1, cap=50), A.ERR_CAPACITY),  # needs max_pos + 1 slots
    (dict(B=0), A.ERR_INVALID_ARG),
])
def test_ragged_decode_rejects(kw, status):
    assert ragged_decode_call(**kw) == status


def e4m3_decode_call(**kw):
    a = dict(B=2, H=4, G=2, d=128, window=16, layer_type=0, eps=1e-6, pos=20, cap=16,
             ks=0.5, vs=0.5)
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_decode_e4m3(
        a["B"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"], a["pos"],
        *p[:7], a["ks"], a["vs"], a["cap"], p[7], p[8], 1 << 34, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0.0), A.ERR_INVALID_ARG),
    (dict(vs=-1.0), A.ERR_INVALID_ARG),
    (dict(ks=float("inf")), A.ERR_INVALID_ARG),
    (dict(vs=float("nan")), A.ERR_INVALID_ARG),
    (dict(ks=1e-45), A.ERR_INVALID_ARG),          # 1/scale overflows
    (dict(d=64), A.ERR_UNSUPPORTED),              # split kernel only
    (dict(H=18, G=2), A.ERR_UNSUPPORTED),         # 9 query heads per key/value head
    (dict(cap=15), A.ERR_CAPACITY),
    (dict(pos=-1), A.ERR_INVALID_ARG),
])
def test_e4m3_decode_rejects(kw, status):
    assert e4m3_decode_call(**kw) == status


def test_e4m3_workspace_adds_rotated_keys_on_full_layers():
    L = A.lib()
    plain = L.olmo3_workspace_bytes(0, 1, 100, 4, 2, 128, 1, A.DTYPE_BF16, 100)
    e4m3 = L.olmo3_workspace_bytes(0, 1, 100, 4, 2, 128, 1, A.DTYPE_BF16_E4M3, 100)
    assert e4m3 - plain >= 100 * 2 * 128 * 2
    # a first chunk (capacity 0): the same as bf16 on a sliding layer
    assert L.olmo3_workspace_bytes(0, 1, 100, 4, 2, 128, 0, A.DTYPE_BF16_E4M3, 0) == \
        L.olmo3_workspace_bytes(0, 1, 100, 4, 2, 128, 0, A.DTYPE_BF16, 16)


def test_e4m3_workspace_adds_cache_copy_for_later_chunks():
    # room for a bf16 copy of every key and value row of the cache
    L = A.lib()
    for lt, cap in ((0, 16), (1, 300)):
        first = L.olmo3_workspace_bytes(0, 3, 100, 4, 2, 128, lt, A.DTYPE_BF16_E4M3, 0)
        later = L.olmo3_workspace_bytes(0, 3, 100, 4, 2, 128, lt, A.DTYPE_BF16_E4M3, cap)
        assert later - first == 2 * 3 * 2 * cap * 128 * 2


def e4m3_prefill_call(ws_bytes=1 << 34, **kw):
    a = dict(B=1, T=8, H=4, G=2, d=128, window=16, layer_type=1, eps=1e-6, pos=40, cap=64,
             ks=0.5, vs=0.5)
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_prefill_e4m3(
        a["B"], a["T"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"],
        a["pos"], *p[:7], a["ks"], a["vs"], a["cap"], p[7], p[8], ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=-1), A.ERR_INVALID_ARG),
    (dict(ks=0.0), A.ERR_INVALID_ARG),
    (dict(cap=47), A.ERR_CAPACITY),               # positions 40 .. 47 need 48 slots
    (dict(layer_type=0, cap=15), A.ERR_CAPACITY),  # ring size != window
    (dict(pos=(1 << 30) - 7), A.ERR_CAPACITY),
    (dict(d=20), A.ERR_UNSUPPORTED),
])
def test_e4m3_prefill_rejects(kw, status):
    assert e4m3_prefill_call(**kw) == status


@pytest.mark.parametrize("lt,rows", [(1, 40), (0, 16)])
def test_e4m3_prefill_later_chunk_needs_the_copy(lt, rows):
    # a chunk at pos_offset 40 reads its prefix from a bf16 copy and never
    # splits its keys: it needs its rotated queries (8 x 4 x 128 bf16) and
    # keys (8 x 2 x 128), each region 256-byte aligned, plus the copy of 40
    # linear rows, or of the 16-slot ring, of keys and of values
    L = A.lib()
    first = L.olmo3_workspace_bytes(0, 1, 8, 4, 2, 128, lt, A.DTYPE_BF16_E4M3, 0)
    need = 8 * 4 * 128 * 2 + 8 * 2 * 128 * 2 + 2 * 2 * rows * 128 * 2
    assert first > 8 * 4 * 128 * 2 + 8 * 2 * 128 * 2   # the first chunk may split: its states
    cap = 64 if lt == 1 else 16
    assert e4m3_prefill_call(ws_bytes=need - 1, layer_type=lt, cap=cap) == A.ERR_WORKSPACE


def ragged_e4m3_call(**kw):
    a = dict(B=2, H=4, G=2, d=128, window=16, layer_type=0, eps=1e-6, pos=fake(10), max_pos=20,
             cap=16, ks=0.5, vs=0.5)
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_decode_ragged_e4m3(
        a["B"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r, a["eps"], a["pos"],
        a["max_pos"], *p[:7], a["ks"], a["vs"], a["cap"], p[7], p[8], 1 << 34, None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=0), A.ERR_INVALID_ARG),              # null positions
    (dict(pos=fake(10) + 2), A.ERR_INVALID_ARG),   # misaligned positions
    (dict(max_pos=-1), A.ERR_INVALID_ARG),
    (dict(ks=0.0), A.ERR_INVALID_ARG),
    (dict(vs=float("inf")), A.ERR_INVALID_ARG),
    (dict(d=64), A.ERR_UNSUPPORTED),               # split kernels only
    (dict(layer_type=1, cap=20), A.ERR_CAPACITY),  # needs max_pos + 1 slots
    (dict(cap=15), A.ERR_CAPACITY),                # ring size != window
])
def test_ragged_decode_e4m3_rejects(kw, status):
    assert ragged_e4m3_call(**kw) == status


def ragged_prefill_e4m3_call(**kw):
    a = dict(B=2, n=40, max_len=30, H=4, G=2, d=128, window=16, layer_type=0, eps=1e-6,
             cu=fake(10), cap=16, ks=0.5, vs=0.5)
    a.update(kw)
    p = [fake(i) for i in range(9)]
    r = ctypes.byref(A.Rope(theta=1e4).to_c())
    return A.lib().olmo3_attn_prefill_ragged_e4m3(
        a["B"], a["n"], a["max_len"], a["H"], a["G"], a["d"], a["window"], a["layer_type"], r,
        a["eps"], a["cu"], *p[:7], a["ks"], a["vs"], a["cap"], p[7], p[8], 1 << 34, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=0), A.ERR_INVALID_ARG),               # null cu_seqlens
    (dict(cu=fake(10) + 2), A.ERR_INVALID_ARG),    # misaligned cu_seqlens
    (dict(max_len=41), A.ERR_INVALID_ARG),         # longer than all rows
    (dict(B=0), A.ERR_INVALID_ARG),
    (dict(ks=-1.0), A.ERR_INVALID_ARG),
    (dict(cap=15), A.ERR_CAPACITY),                # ring size != window
    (dict(layer_type=1, cap=29), A.ERR_CAPACITY),  # a linear cache needs max_len slots
    (dict(d=20), A.ERR_UNSUPPORTED),
])
def test_ragged_prefill_e4m3_rejects(kw, status):
    assert ragged_prefill_e4m3_call(**kw) == status
