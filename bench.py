#!/usr/bin/env python3
"""Throughput of the OLMo 3 per-layer attention path on one MI355X.

One step runs the whole path once per layer kind:
  prefill of T new tokens (QK-norm + RoPE + cache append, then attention), on
  a sliding layer and on a full (YaRN) layer, and
  decode of one token per sequence against a pre-filled cache (append, then
  split-KV attention and merge), on a sliding (ring) and a full layer.
Workloads (synthetic, seeded, shaped like the OLMo 3 configurations):
  7b   (default) prefill B=1, T=8192, H=G=32, d=128, window 4096;
       decode B=32 at cache length 65,536 (new token at position 65,535)
  32b  prefill B=1, T=8192, H=40, G=8; decode B=64 at cache length 32,768
  long 32-layer attention-only stack (24 sliding, 8 full YaRN), B=1,
       T=65,536, 7B head shapes, prefill only
  decode-stack  the same 32-layer stack decoding one token per sequence,
       B=16 at cache length 65,536: KV bytes read per step and per token of
       context (the per-layer-type cache of the page "Olmo 3 7B")
  chunked  7B prefill of a 4,096-token chunk at position 61,440 onto a
       filled cache (full layer: 61,440 cached positions; sliding: the ring)
  7b-e4m3  7B decode (B=32 at 65,536) against e4m3 caches (1-byte codes)
  decode-stack-e4m3  the decode stack against e4m3 caches

Printed: one JSON line.  `value` is prefill TFLOP/s (algorithmic FLOPs of the
allowed query/key pairs over the whole prefill call time); decode KV GB/s is
in "decode" (and is `value` for the decode-only stack workload).  Each kernel is bracketed by HIP events on the stream it is
launched on (the stage-by-stage entry points), giving the per-kernel
rooflines; a decode call's merge stage shares its attention stage's events
(at these batch sizes each (sequence, key/value head) is one workgroup of the
split kernel, which writes the output itself, and no merge kernel runs).  The CPU oracle is timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM peak), 7B & 32B shapes"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WINDOW = 4096
THETA = 500000.0


# HBM bytes per launch of the timed kernels (7B and 32B layer workloads), from
# two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by what the same counter reads for a 1 GiB
# device-to-device copy on the same GPU (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).
# An entry holds only while the kernel's sources hash to `sources`; otherwise
# the figure is reported null.
KERNEL_SOURCES = {
    "prefill_d128_kernel": ["prefill.hip", "tiles.h", "common.h", "kernels.h"],
    "decode_split_kernel": ["attn.hip", "tiles.h", "common.h", "kernels.h"],
    "decode_mfma_kernel": ["attn.hip", "tiles.h", "common.h", "kernels.h"],
}


def decode_kernel(H: int, G: int, e4m3: bool) -> str:
    """The split kernel the library runs: the grouped MFMA one for bf16
    caches with H/G >= 2, else the per-row one."""
    return "decode_mfma_kernel" if not e4m3 and H // G >= 2 else "decode_split_kernel"


MEASURED_TRAFFIC = {
    ("olmo3-7b-layer", "prefill_sliding_l0"): dict(bytes=695532543, sources="3bc9cbd506cb2b68"),
    ("olmo3-7b-layer", "prefill_full_l3"): dict(bytes=301389061, sources="3bc9cbd506cb2b68"),
    ("olmo3-7b-layer", "decode_sliding"): dict(bytes=2148100278, sources="1bb78d08d293ba50"),
    ("olmo3-7b-layer", "decode_full"): dict(bytes=34359469838, sources="1bb78d08d293ba50"),
    ("olmo3-32b-layer", "prefill_sliding_l0"): dict(bytes=321227602, sources="3bc9cbd506cb2b68"),
    ("olmo3-32b-layer", "prefill_full_l3"): dict(bytes=320242780, sources="3bc9cbd506cb2b68"),
    ("olmo3-32b-layer", "decode_sliding"): dict(bytes=1079199164, sources="1bb78d08d293ba50"),
    ("olmo3-32b-layer", "decode_full"): dict(bytes=8621331768, sources="1bb78d08d293ba50"),
}


def sources_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "global_hybrid_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, segment: str, kernel: str):
    entry = MEASURED_TRAFFIC.get((workload, segment))
    if entry is None or kernel not in KERNEL_SOURCES or sources_digest(kernel) != entry["sources"]:
        return None
    return entry["bytes"]


def prefill_pairs(T: int, window: int, sliding: bool) -> int:
    """Allowed (query, key) pairs: sum over t of min(t+1, window), or T(T+1)/2."""
    if not sliding or window >= T:
        return T * (T + 1) // 2
    return window * (window + 1) // 2 + (T - window) * window


def chunk_pairs(P: int, T: int, window: int, sliding: bool) -> int:
    """Allowed pairs of queries at positions P .. P+T-1 over keys 0 .. P+T-1:
    sum over t of min(t+1, window) (sliding) or t+1 (full)."""
    if not sliding:
        return T * P + T * (T + 1) // 2
    grow = max(0, min(P + T, window) - P)  # queries with t + 1 <= window
    return sum(P + j + 1 for j in range(grow)) + (T - grow) * window


def prefill_flops(T, H, d, window, sliding, B=1, P=0) -> int:
    if P:
        return 4 * d * H * chunk_pairs(P, T, window, sliding) * B
    return 4 * d * H * prefill_pairs(T, window, sliding) * B


def decode_rows(pos, window, sliding) -> int:
    return min(pos + 1, window) if sliding else pos + 1


def decode_kv_bytes(B, G, d, n, elem=2) -> int:
    return B * G * n * d * 2 * elem


WORKLOADS = {
    "7b": dict(name="olmo3-7b-layer", prefill=dict(B=1, T=8192, H=32, G=32),
               decode=dict(B=32, H=32, G=32, L=65536)),
    "32b": dict(name="olmo3-32b-layer", prefill=dict(B=1, T=8192, H=40, G=8),
                decode=dict(B=64, H=40, G=8, L=32768)),
    "long": dict(name="olmo3-7b-long-context-stack", prefill=dict(B=1, T=65536, H=32, G=32, layers=32),
                 decode=None),
    "decode-stack": dict(name="olmo3-7b-decode-stack", prefill=None,
                         decode=dict(B=16, H=32, G=32, L=65536, layers=32)),
    "chunked": dict(name="olmo3-7b-chunked-prefill",
                    prefill=dict(B=1, T=4096, H=32, G=32, pos_offset=61440), decode=None),
    "7b-e4m3": dict(name="olmo3-7b-decode-e4m3", prefill=None,
                    decode=dict(B=32, H=32, G=32, L=65536, e4m3=True)),
    "decode-stack-e4m3": dict(name="olmo3-7b-decode-stack-e4m3", prefill=None,
                              decode=dict(B=16, H=32, G=32, L=65536, layers=32, e4m3=True)),
    # one GPU's share when a layer's heads are spread over 8 GPUs (4 of the
    # 7B's 32 key/value heads; 1 of the 32B's 8 with its 5 query heads); the
    # QK-norm statistic then covers the local heads only, where a sharded
    # model would add the other GPUs' sums of squares (an all-reduce of one
    # value per token), so these time the kernels, not the whole layer
    "7b-shard": dict(name="olmo3-7b-head-shard-of-8", prefill=dict(B=1, T=8192, H=4, G=4),
                     decode=dict(B=32, H=4, G=4, L=65536)),
    "32b-shard": dict(name="olmo3-32b-head-shard-of-8", prefill=dict(B=1, T=8192, H=5, G=1),
                      decode=dict(B=64, H=5, G=1, L=32768)),
}
E4M3_SCALES = (1.0 / 16, 1.0 / 16)  # k_scale, v_scale of the e4m3 workload
N_LAYERS_7B = 32
NAIVE_BYTES_PER_TOKEN_7B = N_LAYERS_7B * 32 * 128 * 2 * 2  # every layer full: 524,288


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="7b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline (0 disables it)")
    ap.add_argument("--segments", default="",
                    help="comma-separated subset of prefill_sliding, prefill_full, decode_sliding, "
                         "decode_full (for profiling runs; default: all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three times "
                         "(reference for HBM byte counters) and exit")
    return ap.parse_args()


def copy_calibration(nbytes: int) -> None:
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from global_hybrid_causal_amd import attn as A
    from global_hybrid_causal_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    wanted = set(filter(None, args.segments.split(",")))

    def keep(kind, sliding):
        return not wanted or f"{kind}_{'sliding' if sliding else 'full'}" in wanted
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A.lib()  # fail loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    d = 128
    bf16 = torch.bfloat16
    rope = A.Rope(theta=THETA, yarn=True, factor=8.0, orig_ctx=8192)
    segments = []  # (name, kind, callable(phases), phase list, work, work unit)

    # ---- prefill layers
    pf = wl["prefill"] or dict(B=0, T=0, H=0, G=0)
    B, T, H, G = pf["B"], pf["T"], pf["H"], pf["G"]
    n_layers = pf.get("layers", 0)
    layer_list = ([(ell, A.olmo3_layer_type(ell, n_layers)) for ell in range(n_layers)]
                  if n_layers else [(0, 0), (3, 1)]) if wl["prefill"] else []
    print(f"[bench] workload {wl['name']}: preparing {len(layer_list)} prefill layer(s)", file=sys.stderr,
          flush=True)
    seed_base = 5 if n_layers else (2 if args.workload == "7b" else 4)
    for ell, lt in layer_list:
        sliding = lt == 0
        if not keep("prefill", sliding):
            continue
        x = synth.layer_inputs(seed_base + (ell if n_layers else 0), ell, B, T, H, G, d,
                               device=dev, dtype=bf16)
        P = pf.get("pos_offset", 0)
        cap = WINDOW if sliding else P + T
        if P:
            # a cache already holding positions 0 .. P-1 (the ring: the last
            # WINDOW of them); each call rewrites the chunk's slots (on the
            # ring, the slots its later calls read as the prefix: the values
            # change from the second call on, the work does not)
            kc, vc = synth.cache_fill(7, ell, B, G, cap, d, device=dev, dtype=bf16)
        else:
            kc = torch.zeros((B, G, cap, d), dtype=bf16, device=dev)
            vc = torch.zeros_like(kc)
        out = torch.empty_like(x["q_pre"])
        ws = A.workspace(A.MODE_PREFILL, B, T, H, G, d, lt, bf16, cap, dev)
        r = rope if not sliding else A.Rope(theta=THETA)

        def run(phases, x=x, kc=kc, vc=vc, out=out, ws=ws, lt=lt, r=r, P=P):
            A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc, vc,
                                 out, ws, window=WINDOW, layer_type=lt, rope=r, pos_offset=P,
                                 phases=phases)

        segments.append(dict(name=f"prefill_{'sliding' if sliding else 'full'}_l{ell}", kind="prefill",
                             sliding=sliding, run=run, phases=[A.PHASE_PROLOGUE, A.PHASE_ATTENTION],
                             work=prefill_flops(T, H, d, WINDOW, sliding, B, P)))

    # ---- decode layers
    dc = wl["decode"]
    if dc:
        Bd, Hd, Gd, L = dc["B"], dc["H"], dc["G"], dc["L"]
        pos = L - 1  # the cache holds positions 0 .. L-2; the new token is the L-th
        n_dec_layers = dc.get("layers", 0)
        dec_layers = ([(ell, A.olmo3_layer_type(ell, n_dec_layers)) for ell in range(n_dec_layers)]
                      if n_dec_layers else [(0, 0), (3, 1)])
        dseed = 6 if n_dec_layers else (3 if args.workload == "7b" else 4)
        for ell, lt in dec_layers:
            sliding = lt == 0
            if not keep("decode", sliding):
                continue
            cap = WINDOW if sliding else L
            print(f"[bench] filling {'ring' if sliding else 'linear'} decode cache of layer {ell} "
                  f"[{Bd}, {Gd}, {cap}, {d}] x2", file=sys.stderr, flush=True)
            e4m3 = dc.get("e4m3", False)
            if e4m3:
                kc, vc = synth.e4m3_cache_fill(dseed, (ell if n_dec_layers else 100 + lt), Bd, Gd,
                                               cap, d, device=dev)
            else:
                kc, vc = synth.cache_fill(dseed, (ell if n_dec_layers else 100 + lt), Bd, Gd, cap, d,
                                          device=dev, dtype=bf16)
            x = synth.layer_inputs(dseed, (100 + ell if n_dec_layers else 200 + lt), Bd, 1, Hd, Gd, d,
                                   device=dev, dtype=bf16)
            q = x["q_pre"][:, 0].contiguous()
            k = x["k_pre"][:, 0].contiguous()
            v = x["v"][:, 0].contiguous()
            out = torch.empty_like(q)
            ws = A.workspace(A.MODE_DECODE, Bd, 1, Hd, Gd, d, lt,
                             A.DTYPE_BF16_E4M3 if e4m3 else bf16, cap, dev)
            r = rope if not sliding else A.Rope(theta=THETA)

            def run(phases, q=q, k=k, v=v, x=x, kc=kc, vc=vc, out=out, ws=ws, lt=lt, r=r, pos=pos,
                    e4m3=e4m3):
                if e4m3:
                    A.olmo3_attn_decode_e4m3(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws,
                                             k_scale=E4M3_SCALES[0], v_scale=E4M3_SCALES[1],
                                             window=WINDOW, layer_type=lt, rope=r, pos=pos,
                                             phases=phases)
                else:
                    A.olmo3_attn_decode(q, k, v, x["q_gain"], x["k_gain"], kc, vc, out, ws,
                                        window=WINDOW, layer_type=lt, rope=r, pos=pos, phases=phases)

            n = decode_rows(pos, WINDOW, sliding)
            name = f"decode_{'sliding' if sliding else 'full'}" + (f"_l{ell}" if n_dec_layers else "")
            segments.append(dict(name=name, kind="decode", sliding=sliding, run=run,
                                 # the merge (a kernel only when a key range is split,
                                 # which these batch sizes never need) shares the
                                 # attention stage's events: one event pair fewer
                                 phases=[A.PHASE_PROLOGUE, A.PHASE_ATTENTION | A.PHASE_MERGE],
                                 work=decode_kv_bytes(Bd, Gd, d, n, elem=1 if e4m3 else 2),
                                 rows=n))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(record):
        for seg in segments:
            if record:
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(seg["phases"]) + 1)]
                evs[0].record(stream)
                for i, ph in enumerate(seg["phases"]):
                    seg["run"](ph)
                    evs[i + 1].record(stream)
                seg.setdefault("events", []).append(evs)
            else:
                seg["run"](A.PHASES_ALL if seg["kind"] == "decode" else
                           A.PHASE_PROLOGUE | A.PHASE_ATTENTION)

    print(f"[bench] warmup {args.warmup} step(s)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} step(s)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- per-kernel and per-call times (ms), averaged over the timed steps
    dcfg = wl["decode"] or {}
    kernel_names = {("prefill", 0): "qknorm_rope_append_kernel", ("prefill", 1): "prefill_d128_kernel",
                    ("decode", 0): "decode_prologue_kernel",
                    ("decode", 1): decode_kernel(dcfg.get("H", 1), dcfg.get("G", 1),
                                                 bool(dcfg.get("e4m3")))}
    for seg in segments:
        per_phase = [[evs[i].elapsed_time(evs[i + 1]) for evs in seg["events"]]
                     for i in range(len(seg["phases"]))]
        seg["phase_ms"] = [sum(p) / len(p) for p in per_phase]
        seg["call_ms"] = sum(seg["phase_ms"])
    ms_per_step = wall * 1e3 / args.steps

    pre = [s for s in segments if s["kind"] == "prefill"]
    dec = [s for s in segments if s["kind"] == "decode"]
    prefill_tflops = (sum(s["work"] for s in pre) / (sum(s["call_ms"] for s in pre) * 1e-3) / 1e12
                      if pre else 0.0)

    def roof(seg, phase_idx):
        ms = seg["phase_ms"][phase_idx]
        if seg["kind"] == "prefill":
            ach = seg["work"] / (ms * 1e-3) / 1e12
            kernel = kernel_names[("prefill", phase_idx)]
            return dict(kernel=kernel, segment=seg["name"], bound="mfma",
                        achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(ach / PEAK_BF16_TFLOPS, 4),
                        traffic=measured_traffic(wl["name"], seg["name"], kernel), avg_ms=round(ms, 4))
        ach = seg["work"] / (ms * 1e-3) / 1e9
        kernel = kernel_names[("decode", phase_idx)]
        return dict(kernel=kernel, segment=seg["name"], bound="hbm",
                    achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(ach / PEAK_HBM_GBS, 4),
                    traffic=measured_traffic(wl["name"], seg["name"], kernel), avg_ms=round(ms, 4))

    rooflines = [roof(s, 1) for s in segments]
    dominant = max(zip(segments, rooflines), key=lambda sr: sr[0]["phase_ms"][1])[1]

    dec_gbs = (sum(s["work"] for s in dec) / (sum(s["call_ms"] for s in dec) * 1e-3) / 1e9
               if dec else 0.0)
    result = {
        "metric": METRIC,
        "value": round(prefill_tflops, 2) if pre else round(dec_gbs, 1),
        "unit": "TFLOP/s" if pre else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["name"],
                   "prefill": (dict(pf, d=d, window=WINDOW, theta=THETA, yarn_full="factor 8, orig 8192")
                               if pre else None),
                   "decode": (dict(dc, d=d, window=WINDOW, pos=dc["L"] - 1) if dc else None),
                   "parallelism": "single GPU"},
        "prefill": {"tflops": round(prefill_tflops, 2),
                    "frac_of_peak": round(prefill_tflops / PEAK_BF16_TFLOPS, 4),
                    "calls": {s["name"]: {"call_ms": round(s["call_ms"], 4),
                                          "tflops": round(s["work"] / (s["call_ms"] * 1e-3) / 1e12, 2),
                                          "flop": s["work"]} for s in pre}},
        "roofline": dominant,
        "rooflines": rooflines,
    }
    if dec:
        gbs = dec_gbs
        result["decode"] = {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                            "calls": {s["name"]: {"call_ms": round(s["call_ms"], 4),
                                                  "gbs": round(s["work"] / (s["call_ms"] * 1e-3) / 1e9, 1),
                                                  "kv_bytes": s["work"], "rows": s["rows"]}
                                      for s in dec}}
    if dc and dc.get("layers") and len(dec) == dc["layers"]:
        # per decode step of the stack: every layer reads its whole cache once
        kv_step = sum(s["work"] for s in dec)
        step_ms = sum(s["call_ms"] for s in dec)
        result["stack"] = {
            "layers": dc["layers"], "sliding": sum(s["sliding"] for s in dec),
            "kv_bytes_per_step": kv_step, "step_ms": round(step_ms, 4),
            "tokens_per_s": round(dc["B"] / (step_ms * 1e-3), 1),
            "kv_bytes_per_token_of_context": kv_step // (dc["B"] * dc["L"]),
            "naive_bytes_per_token_of_context": NAIVE_BYTES_PER_TOKEN_7B // (2 if dc.get("e4m3") else 1),
        }
    if args.cpu_seconds > 0 and (pre or dec) and not (wl["prefill"] or {}).get("pos_offset"):
        print(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        result["cpu_baseline"] = (cpu_baseline(args, wl, segments, dev) if pre else
                                  cpu_baseline_decode(args, wl))
    if dc and dec:
        result["decode"]["tokens_per_s"] = round(
            dc["B"] / (sum(s["call_ms"] for s in dec) * 1e-3), 1)
        result["decode"]["cache_dtype"] = "e4m3" if dc.get("e4m3") else "bf16"
    print(json.dumps(result), flush=True)


def cpu_baseline(args, wl, segments, dev):
    """The oracle, as it stands, on a bounded sample of the prefill workload:
    blocks of 32 query rows of the sliding layer (all heads, the keys those
    rows can see), spread over the sequence, until the time budget is spent.
    FLOPs are counted like the GPU's (allowed pairs only)."""
    import numpy as np
    import torch

    import oracle as O

    threads = _blas_threads()
    from global_hybrid_causal_amd import synth

    pf = wl["prefill"]
    B, T, H, G, d = 1, pf["T"], pf["H"], pf["G"], 128
    seed = 5 if pf.get("layers") else (2 if args.workload == "7b" else 4)
    x = synth.layer_inputs(seed, 0, B, T, H, G, d, device=dev, dtype=torch.bfloat16)
    hx = {k: v.detach().to("cpu", torch.float64).numpy() for k, v in x.items()}
    rope = O.RopeParams(theta=THETA)
    rng = np.random.default_rng(0)
    rows_per_block = 32
    flops = 0
    blocks = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.cpu_seconds:
        t_start = int(rng.integers(0, T - rows_per_block + 1))
        rows = np.arange(t_start, t_start + rows_per_block)
        k_lo = max(0, t_start - WINDOW + 1)
        keys = np.arange(k_lo, t_start + rows_per_block)
        O.attention_rows_ref(hx["q_pre"][0, rows], rows, hx["k_pre"][0, keys],
                             hx["v"][0, keys].reshape(len(keys), G, d), keys, hx["q_gain"],
                             hx["k_gain"], H=H, G=G, d=d, kv_heads=range(G), kind=O.SLIDING,
                             window=WINDOW, rope=rope)
        flops += 4 * d * H * int(np.minimum(rows + 1, WINDOW).sum())
        blocks += 1
    elapsed = time.perf_counter() - t0
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{blocks} blocks of {rows_per_block} query rows x {H} heads of the "
                      f"{wl['name']} sliding prefill (T={T}, window {WINDOW}), fp64 NumPy, "
                      f"{elapsed:.1f} s"}


def cpu_baseline_decode(args, wl):
    """The oracle's decode on a bounded sample of the decode workload: one
    (sequence, key/value head) of a full layer at the workload's cache length
    per call, seeded cache rows of the same shape, until the time budget is
    spent.  Bytes are counted like the GPU's (the K and V rows read, bf16)."""
    import numpy as np
    import torch

    import oracle as O
    from global_hybrid_causal_amd import synth

    threads = _blas_threads()
    dc = wl["decode"]
    H, G, L, d = dc["H"], dc["G"], dc["L"], 128
    pos = L - 1
    group = H // G
    e4m3 = dc.get("e4m3", False)
    rope = O.RopeParams(theta=THETA, yarn=True, factor=8.0, orig_ctx=8192)
    if e4m3:  # the codes' values, as the oracle's e4m3 cache holds them
        table = O.e4m3_values()
        ck = table[synth.e4m3_codes((1, L, d), 7, 0, synth.CACHE_K).numpy()] * E4M3_SCALES[0]
        cv = table[synth.e4m3_codes((1, L, d), 7, 0, synth.CACHE_V).numpy()] * E4M3_SCALES[1]
    else:
        ck = synth.normal((1, L, d), 7, 0, synth.CACHE_K).to(torch.float64).numpy()
        cv = synth.normal((1, L, d), 7, 0, synth.CACHE_V).to(torch.float64).numpy()
    tags = O.ring_positions(O.FULL, WINDOW, L, pos)
    x = synth.layer_inputs(7, 0, 1, 1, H, G, d, dtype=torch.float32)
    hx = {k: v.to(torch.float64).numpy() for k, v in x.items()}
    calls, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.cpu_seconds:
        O.decode_rows_ref(hx["q_pre"][0, 0], hx["k_pre"][0, 0], hx["v"][0, 0], hx["q_gain"],
                          hx["k_gain"], ck, cv, tags, H=H, G=G, d=d, kv_heads=[0], kind=O.FULL,
                          window=WINDOW, rope=rope, pos=pos)
        calls += 1
    elapsed = time.perf_counter() - t0
    nbytes = calls * L * d * 2 * (1 if e4m3 else 2)
    return {"value": round(nbytes / elapsed / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{calls} decode calls of one sequence x one key/value head ({group} query "
                      f"head{'s' if group > 1 else ''}) of a full layer at cache length {L}, fp64 "
                      f"NumPy, {elapsed:.1f} s"}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()
                    if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        return len(os.sched_getaffinity(0))


if __name__ == "__main__":
    main()
