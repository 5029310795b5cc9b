#!/usr/bin/env python3
"""Throughput of the OLMo 3 per-layer attention path on one MI355X.

One step runs every workload named by --workload once, each call stage by
stage (prologue: QK-norm + RoPE + cache append; then attention):
  7b   prefill B=1, T=8192, H=G=32, d=128 on a sliding layer (window 4096)
       and on a full (YaRN) layer; decode B=32 at cache length 65,536 (new
       token at position 65,535) on a sliding (ring) and a full layer
  32b  the same with H=40, G=8; decode B=64 at cache length 32,768
  long 32-layer attention-only stack (24 sliding, 8 full YaRN), B=1,
       T=65,536, 7B head shapes, prefill only
The default is all three ("7b,32b,long").  Other workloads, one at a time or
in a list:
  decode-stack  the 32-layer stack decoding one token per sequence, B=16 at
       cache length 65,536: KV bytes read per step and per token of context
       (the per-layer-type cache of the page "Olmo 3 7B")
  chunked  7B prefill of a 4,096-token chunk at position 61,440 onto a
       filled cache (full layer: 61,440 cached positions; sliding: the ring)
  7b-e4m3  7B decode (B=32 at 65,536) against e4m3 caches (1-byte codes)
  32b-e4m3  32B decode (B=64 at 32,768) against e4m3 caches
  decode-stack-e4m3  the decode stack against e4m3 caches
  7b-shard, 32b-shard  one GPU's share of an 8-way head split of a layer

Printed: one JSON line.  `value` is prefill TFLOP/s (algorithmic FLOPs of the
allowed query/key pairs over the whole call time, prologue included) over the
prefill calls of the 7B and 32B layers when either is run (else over every
prefill call, else decode KV GB/s); per-workload blocks give each call.  The
timed steps run twice.  First stage by stage: each kernel is bracketed by HIP
events on the stream it is launched on (the stage-by-stage entry points),
giving the per-kernel rooflines; a decode call's merge stage shares its
attention stage's events (at these batch sizes each (sequence, key/value
head) is one workgroup of the split kernel, which writes the output itself,
and no merge kernel runs).  Then call by call, one pair of events around each
whole call: the call times, `value` and ms_per_step.  The CPU oracle is timed
on a bounded sample of the 7B layer shape.
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


# HBM bytes per launch of the timed kernels, from two rocprofv3 --pmc runs of
# this script's default step (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by what the same counter reads for a 1 GiB device-to-device
# copy on the same GPU (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Keyed by (roofline group, kernel); a group of several launches (the
# long stack's layers of one kind) holds the mean per launch.  An entry holds
# only while the kernel's sources hash to `sources`; otherwise the figure is
# reported null.
KERNEL_SOURCES = {
    "prefill_d128_kernel": ["prefill.hip", "tiles.h", "common.h", "kernels.h"],
    "decode_split_kernel": ["attn.hip", "tiles.h", "common.h", "kernels.h"],
    "decode_mfma_kernel": ["attn.hip", "tiles.h", "common.h", "kernels.h"],
    "qknorm_rope_append_kernel": ["prologue.hip", "common.h", "kernels.h"],
    "decode_prologue_kernel": ["prologue.hip", "common.h", "kernels.h"],
}


def decode_kernel(H: int, G: int, e4m3: bool) -> str:
    """The split kernel the library runs: the grouped MFMA one for bf16
    caches with H/G >= 2, else the per-row one."""
    return "decode_mfma_kernel" if not e4m3 and H // G >= 2 else "decode_split_kernel"


MEASURED_TRAFFIC = {
    ("7b/prefill_sliding_l0", "qknorm_rope_append_kernel"): dict(bytes=369829721, sources="698d00bb50ad00da"),
    ("7b/prefill_sliding_l0", "prefill_d128_kernel"): dict(bytes=550013977, sources="ca4d3856a3738d99"),
    ("7b/prefill_full_l3", "qknorm_rope_append_kernel"): dict(bytes=403382729, sources="698d00bb50ad00da"),
    ("7b/prefill_full_l3", "prefill_d128_kernel"): dict(bytes=568240730, sources="ca4d3856a3738d99"),
    ("7b/decode_sliding", "decode_prologue_kernel"): dict(bytes=1895197, sources="698d00bb50ad00da"),
    ("7b/decode_sliding", "decode_split_kernel"): dict(bytes=2148037911, sources="4b67bc8a681e176b"),
    ("7b/decode_full", "decode_prologue_kernel"): dict(bytes=1910972, sources="698d00bb50ad00da"),
    ("7b/decode_full", "decode_split_kernel"): dict(bytes=34359278327, sources="4b67bc8a681e176b"),
    ("32b/prefill_sliding_l0", "qknorm_rope_append_kernel"): dict(bytes=227165550, sources="698d00bb50ad00da"),
    ("32b/prefill_sliding_l0", "prefill_d128_kernel"): dict(bytes=253362563, sources="ca4d3856a3738d99"),
    ("32b/prefill_full_l3", "qknorm_rope_append_kernel"): dict(bytes=235553795, sources="698d00bb50ad00da"),
    ("32b/prefill_full_l3", "prefill_d128_kernel"): dict(bytes=266877244, sources="ca4d3856a3738d99"),
    ("32b/decode_sliding", "decode_prologue_kernel"): dict(bytes=2113562, sources="698d00bb50ad00da"),
    ("32b/decode_sliding", "decode_mfma_kernel"): dict(bytes=1079346818, sources="4b67bc8a681e176b"),
    ("32b/decode_full", "decode_prologue_kernel"): dict(bytes=2116858, sources="698d00bb50ad00da"),
    ("32b/decode_full", "decode_mfma_kernel"): dict(bytes=8624507172, sources="4b67bc8a681e176b"),
    ("long/prefill_sliding", "qknorm_rope_append_kernel"): dict(bytes=2249100419, sources="698d00bb50ad00da"),
    ("long/prefill_sliding", "prefill_d128_kernel"): dict(bytes=20187753857, sources="ca4d3856a3738d99"),
    ("long/prefill_full", "qknorm_rope_append_kernel"): dict(bytes=3222470100, sources="698d00bb50ad00da"),
    ("long/prefill_full", "prefill_d128_kernel"): dict(bytes=6537490627, sources="ca4d3856a3738d99"),
    # mean per launch over the four 7B and 32B layer launches (the `roofline` group)
    ("32b+7b prefill calls", "prefill_d128_kernel"): dict(bytes=409623628, sources="ca4d3856a3738d99"),
}


def sources_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "global_hybrid_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(group: str, kernel: str):
    entry = MEASURED_TRAFFIC.get((group, kernel))
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


def prefill_prologue_bytes(B, T, H, G, d, sliding, window=4096, es=2) -> int:
    """Algorithmic HBM bytes of the prefill prologue at position 0: it reads
    the projected q, k and v rows and writes the rotated queries, the cache
    rows it keeps (the last `window` positions on a ring) and, on a sliding
    layer, a rotated copy of every key for the attention."""
    kept = min(T, window) if sliding else T
    return (B * T * (H + 2 * G) * d * es + B * T * H * d * es + B * kept * 2 * G * d * es
            + (B * T * G * d * es if sliding else 0))


def decode_prologue_bytes(B, H, G, d, cache_elem=2, es=2) -> int:
    """Reads one token's q, k, v per sequence; writes its rotated query and
    its key and value to one cache slot."""
    return B * (H + 2 * G) * d * es + B * H * d * es + B * 2 * G * d * cache_elem


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
    "32b-e4m3": dict(name="olmo3-32b-decode-e4m3", prefill=None,
                     decode=dict(B=64, H=40, G=8, L=32768, e4m3=True)),
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


HEADLINE = ("7b", "32b")  # `value` and `roofline` cover these workloads' prefill calls


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="7b,32b,long",
                    help="comma-separated list of " + ", ".join(sorted(WORKLOADS)))
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU time budget of the oracle baseline (0 disables it)")
    ap.add_argument("--segments", default="",
                    help="comma-separated subset of prefill_sliding, prefill_full, decode_sliding, "
                         "decode_full (for profiling runs; default: all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three times "
                         "(reference for HBM byte counters) and exit")
    args = ap.parse_args()
    args.workloads = [w for w in args.workload.split(",") if w]
    bad = [w for w in args.workloads if w not in WORKLOADS]
    if bad or not args.workloads:
        ap.error(f"unknown workload(s) {bad}; choose from {sorted(WORKLOADS)}")
    return args


def copy_calibration(nbytes: int) -> None:
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)


def build_segments(key, wanted, dev, A, synth, torch):
    """The calls of workload `key`, in step order: dicts with the workload,
    the call's name, its roofline group, a run(phases) closure, the stages
    timed separately and, per stage, the kernel and its algorithmic work."""
    wl = WORKLOADS[key]
    d = 128
    bf16 = torch.bfloat16
    rope = A.Rope(theta=THETA, yarn=True, factor=8.0, orig_ctx=8192)
    segments = []

    def keep(kind, sliding):
        return not wanted or f"{kind}_{'sliding' if sliding else 'full'}" in wanted

    pf = wl["prefill"]
    if pf:
        B, T, H, G = pf["B"], pf["T"], pf["H"], pf["G"]
        n_layers = pf.get("layers", 0)
        layer_list = ([(ell, A.olmo3_layer_type(ell, n_layers)) for ell in range(n_layers)]
                      if n_layers else [(0, 0), (3, 1)])
        print(f"[bench] {wl['name']}: preparing {len(layer_list)} prefill layer(s)", file=sys.stderr,
              flush=True)
        seed_base = 5 if n_layers else (2 if key == "7b" else 4)
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
                A.olmo3_attn_prefill(x["q_pre"], x["k_pre"], x["v"], x["q_gain"], x["k_gain"], kc,
                                     vc, out, ws, window=WINDOW, layer_type=lt, rope=r,
                                     pos_offset=P, phases=phases)

            kind = "sliding" if sliding else "full"
            flops = prefill_flops(T, H, d, WINDOW, sliding, B, P)
            segments.append(dict(
                wl=key, wl_name=wl["name"], name=f"prefill_{kind}_l{ell}", kind="prefill",
                group=f"{key}/prefill_{kind}" + ("" if n_layers else f"_l{ell}"), sliding=sliding,
                run=run, phases=[A.PHASE_PROLOGUE, A.PHASE_ATTENTION],
                kernels=["qknorm_rope_append_kernel", "prefill_d128_kernel"],
                # the prologue's bytes are stated for calls at position 0 only
                stage_work=[prefill_prologue_bytes(B, T, H, G, d, sliding) if not P else None, flops],
                stage_bound=["hbm", "mfma"], work=flops))

    dc = wl["decode"]
    if dc:
        Bd, Hd, Gd, L = dc["B"], dc["H"], dc["G"], dc["L"]
        pos = L - 1  # the cache holds positions 0 .. L-2; the new token is the L-th
        n_dec_layers = dc.get("layers", 0)
        dec_layers = ([(ell, A.olmo3_layer_type(ell, n_dec_layers)) for ell in range(n_dec_layers)]
                      if n_dec_layers else [(0, 0), (3, 1)])
        dseed = 6 if n_dec_layers else (3 if key == "7b" else 4)
        e4m3 = dc.get("e4m3", False)
        for ell, lt in dec_layers:
            sliding = lt == 0
            if not keep("decode", sliding):
                continue
            cap = WINDOW if sliding else L
            print(f"[bench] {wl['name']}: filling {'ring' if sliding else 'linear'} decode cache of "
                  f"layer {ell} [{Bd}, {Gd}, {cap}, {d}] x2", file=sys.stderr, flush=True)
            if e4m3:
                kc, vc = synth.e4m3_cache_fill(dseed, (ell if n_dec_layers else 100 + lt), Bd, Gd,
                                               cap, d, device=dev)
            else:
                kc, vc = synth.cache_fill(dseed, (ell if n_dec_layers else 100 + lt), Bd, Gd, cap,
                                          d, device=dev, dtype=bf16)
            x = synth.layer_inputs(dseed, (100 + ell if n_dec_layers else 200 + lt), Bd, 1, Hd, Gd,
                                   d, device=dev, dtype=bf16)
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
            kind = "sliding" if sliding else "full"
            name = f"decode_{kind}" + (f"_l{ell}" if n_dec_layers else "")
            kv = decode_kv_bytes(Bd, Gd, d, n, elem=1 if e4m3 else 2)
            segments.append(dict(
                wl=key, wl_name=wl["name"], name=name, kind="decode",
                group=f"{key}/decode_{kind}", sliding=sliding, run=run,
                # the merge (a kernel only when a key range is split, which
                # these batch sizes never need) shares the attention stage's
                # events: one event pair fewer
                phases=[A.PHASE_PROLOGUE, A.PHASE_ATTENTION | A.PHASE_MERGE],
                kernels=["decode_prologue_kernel", decode_kernel(Hd, Gd, e4m3)],
                stage_work=[decode_prologue_bytes(Bd, Hd, Gd, d, 1 if e4m3 else 2), kv],
                stage_bound=["hbm", "hbm"], work=kv, rows=n))
    return segments


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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A.lib()  # fail loudly if the HIP library is missing
    segments = []
    for key in args.workloads:
        segments += build_segments(key, wanted, dev, A, synth, torch)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    whole = {"prefill": A.PHASE_PROLOGUE | A.PHASE_ATTENTION, "decode": A.PHASES_ALL}

    def step(mode):
        """mode None: untimed; "stages": every stage of every call between its
        own events; "calls": every call whole, between one pair of events."""
        for seg in segments:
            if mode == "stages":
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(seg["phases"]) + 1)]
                evs[0].record(stream)
                for i, ph in enumerate(seg["phases"]):
                    seg["run"](ph)
                    evs[i + 1].record(stream)
                seg.setdefault("events", []).append(evs)
            elif mode == "calls":
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                evs[0].record(stream)
                seg["run"](whole[seg["kind"]])
                evs[1].record(stream)
                seg.setdefault("call_events", []).append(evs)
            else:
                seg["run"](whole[seg["kind"]])

    print(f"[bench] warmup {args.warmup} step(s)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    # the timed steps, twice: stage by stage for the per-kernel figures, then
    # call by call (no events between a call's kernels) for the call times,
    # `value` and ms_per_step
    print(f"[bench] timing {args.steps} step(s), stage by stage", file=sys.stderr, flush=True)
    for _ in range(args.steps):
        step("stages")
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} step(s), call by call", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step("calls")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- per-stage and per-call times (ms), averaged over the timed steps
    for seg in segments:
        per_phase = [[evs[i].elapsed_time(evs[i + 1]) for evs in seg["events"]]
                     for i in range(len(seg["phases"]))]
        seg["phase_ms"] = [sum(p) / len(p) for p in per_phase]
        calls = [e0.elapsed_time(e1) for e0, e1 in seg["call_events"]]
        seg["call_ms"] = sum(calls) / len(calls)
    ms_per_step = wall * 1e3 / args.steps

    def tflops(segs):
        return sum(s["work"] for s in segs) / (sum(s["call_ms"] for s in segs) * 1e-3) / 1e12

    def gbs(segs):
        return sum(s["work"] for s in segs) / (sum(s["call_ms"] for s in segs) * 1e-3) / 1e9

    def roof(segs, stage, label):
        """Roofline of one kernel over the launches of `segs` at `stage`:
        algorithmic work per launch / mean launch time."""
        ms = sum(s["phase_ms"][stage] for s in segs) / len(segs)
        work = sum(s["stage_work"][stage] for s in segs) / len(segs)
        kernel, bound = segs[0]["kernels"][stage], segs[0]["stage_bound"][stage]
        mfma = bound == "mfma"
        ach = work / (ms * 1e-3) / (1e12 if mfma else 1e9)
        peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS
        return dict(kernel=kernel, segment=label, launches_per_step=len(segs), bound=bound,
                    achieved=round(ach, 2), peak=peak, unit="TFLOP/s" if mfma else "GB/s",
                    frac=round(ach / peak, 4), traffic=measured_traffic(label, kernel),
                    avg_ms=round(ms, 4))

    groups = {}
    for seg in segments:
        groups.setdefault(seg["group"], []).append(seg)
    rooflines = []
    for label, segs in groups.items():
        for stage in (1, 0):
            if all(s["stage_work"][stage] for s in segs):
                rooflines.append(roof(segs, stage, label))

    pre = [s for s in segments if s["kind"] == "prefill"]
    dec = [s for s in segments if s["kind"] == "decode"]
    head = [s for s in pre if s["wl"] in HEADLINE] or pre
    if head:
        dominant = roof(head, 1, "+".join(sorted({s["wl"] for s in head})) + " prefill calls")
        value, unit = tflops(head), "TFLOP/s"
    else:
        dominant = max(rooflines, key=lambda r: r["avg_ms"] * r["launches_per_step"])
        value, unit = gbs(dec), "GB/s"

    by_wl = {}
    for key in args.workloads:
        wl = WORKLOADS[key]
        wp = [s for s in pre if s["wl"] == key]
        wd = [s for s in dec if s["wl"] == key]
        block = {"name": wl["name"]}
        if wp:
            pf = wl["prefill"]
            block["prefill"] = {
                "config": dict(pf, d=128, window=WINDOW, theta=THETA, yarn_full="factor 8, orig 8192"),
                "tflops": round(tflops(wp), 2), "frac_of_peak": round(tflops(wp) / PEAK_BF16_TFLOPS, 4),
                "attention_tflops": round(sum(s["work"] for s in wp) /
                                          (sum(s["phase_ms"][1] for s in wp) * 1e-3) / 1e12, 2),
                "calls_ms": round(sum(s["call_ms"] for s in wp), 4)}
            if not pf.get("layers"):
                block["prefill"]["calls"] = {
                    s["name"]: {"call_ms": round(s["call_ms"], 4),
                                "tflops": round(s["work"] / (s["call_ms"] * 1e-3) / 1e12, 2),
                                "flop": s["work"]} for s in wp}
            else:
                block["prefill"]["layers"] = pf["layers"]
                block["prefill"]["sliding_layers"] = sum(s["sliding"] for s in wp)
        if wd:
            dc = wl["decode"]
            block["decode"] = {
                "config": dict(dc, d=128, window=WINDOW, pos=dc["L"] - 1),
                "gbs": round(gbs(wd), 1), "frac_of_peak": round(gbs(wd) / PEAK_HBM_GBS, 4),
                "tokens_per_s": round(dc["B"] / (sum(s["call_ms"] for s in wd) * 1e-3), 1),
                "cache_dtype": "e4m3" if dc.get("e4m3") else "bf16"}
            if not dc.get("layers"):
                block["decode"]["calls"] = {
                    s["name"]: {"call_ms": round(s["call_ms"], 4),
                                "gbs": round(s["work"] / (s["call_ms"] * 1e-3) / 1e9, 1),
                                "kv_bytes": s["work"], "rows": s["rows"]} for s in wd}
            elif len(wd) == dc["layers"]:
                # per decode step of the stack: every layer reads its whole cache once
                kv_step = sum(s["work"] for s in wd)
                step_ms = sum(s["call_ms"] for s in wd)
                block["decode"]["stack"] = {
                    "layers": dc["layers"], "sliding": sum(s["sliding"] for s in wd),
                    "kv_bytes_per_step": kv_step, "step_ms": round(step_ms, 4),
                    "kv_bytes_per_token_of_context": kv_step // (dc["B"] * dc["L"]),
                    "naive_bytes_per_token_of_context":
                        NAIVE_BYTES_PER_TOKEN_7B // (2 if dc.get("e4m3") else 1)}
        by_wl[key] = block

    names = [WORKLOADS[k]["name"] for k in args.workloads]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": " + ".join(names), "workloads": args.workloads,
                   "value_covers": ("prefill calls (prologue + attention) of " +
                                    " and ".join(sorted({s["wl_name"] for s in head}))
                                    if head else "decode calls"),
                   "parallelism": "single GPU"},
        "workloads": by_wl,
        "roofline": dominant,
        "rooflines": rooflines,
    }
    plain = [k for k in args.workloads if WORKLOADS[k]["prefill"] and
             not WORKLOADS[k]["prefill"].get("pos_offset")]
    if args.cpu_seconds > 0 and plain:
        print(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(args, dev, args.cpu_seconds)
    elif args.cpu_seconds > 0 and dec:
        result["cpu_baseline"] = cpu_baseline_decode(args, WORKLOADS[dec[0]["wl"]])
    print(json.dumps(result), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover - informational only
        pass
    return "unknown"


def cpu_baseline(args, dev, seconds):
    """The oracle, as it stands (fp64 NumPy), on a bounded sample of the 7B
    layer prefill: blocks of 32 query rows (all heads, the keys those rows
    can see) at random places of the sequence, half the budget on a sliding
    and half on a full layer.  FLOPs are counted like the GPU's (allowed
    pairs only).  The rates extrapolate to whole calls and to the long stack
    (24 sliding + 8 full layers at T = 65,536), labelled as extrapolated."""
    import numpy as np
    import torch

    import oracle as O
    from global_hybrid_causal_amd import synth

    threads = _blas_threads()
    B, T, H, G, d = 1, 8192, 32, 32, 128
    x = synth.layer_inputs(2, 0, B, T, H, G, d, device=dev, dtype=torch.bfloat16)
    hx = {k: v.detach().to("cpu", torch.float64).numpy() for k, v in x.items()}
    rng = np.random.default_rng(0)
    rows_per_block = 32
    rates, blocks, spent, done = {}, {}, 0.0, 0
    for kind, rope in ((O.SLIDING, O.RopeParams(theta=THETA)),
                       (O.FULL, O.RopeParams(theta=THETA, yarn=True, factor=8.0, orig_ctx=8192))):
        flops, n, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds / 2:
            t_start = int(rng.integers(0, T - rows_per_block + 1))
            rows = np.arange(t_start, t_start + rows_per_block)
            k_lo = max(0, t_start - WINDOW + 1) if kind == O.SLIDING else 0
            keys = np.arange(k_lo, t_start + rows_per_block)
            O.attention_rows_ref(hx["q_pre"][0, rows], rows, hx["k_pre"][0, keys],
                                 hx["v"][0, keys].reshape(len(keys), G, d), keys, hx["q_gain"],
                                 hx["k_gain"], H=H, G=G, d=d, kv_heads=range(G), kind=kind,
                                 window=WINDOW, rope=rope)
            allowed = np.minimum(rows + 1, WINDOW) if kind == O.SLIDING else rows + 1
            flops += 4 * d * H * int(allowed.sum())
            n += 1
        elapsed = time.perf_counter() - t0
        rates[kind] = flops / elapsed
        blocks[kind] = n
        spent += elapsed
        done += flops
    total = sum(blocks.values())
    value = done / spent
    f_s, f_f = prefill_flops(T, H, d, WINDOW, True), prefill_flops(T, H, d, WINDOW, False)
    long_T = WORKLOADS["long"]["prefill"]["T"]
    long_s = (24 * prefill_flops(long_T, H, d, WINDOW, True) / rates[O.SLIDING] +
              8 * prefill_flops(long_T, H, d, WINDOW, False) / rates[O.FULL])
    return {"value": round(value / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "cpu_model": _cpu_model(), "precision": "fp64 (NumPy, BLAS matmuls)", "kind": "oracle",
            "sample": f"{total} blocks of {rows_per_block} query rows x {H} heads of the 7B layer "
                      f"prefill (T={T}, window {WINDOW}): {blocks[O.SLIDING]} sliding, "
                      f"{blocks[O.FULL]} full (YaRN), {spent:.1f} s in all",
            "tflops_sliding": round(rates[O.SLIDING] / 1e12, 6),
            "tflops_full": round(rates[O.FULL] / 1e12, 6),
            "extrapolated_s": {"7b_prefill_sliding_call": round(f_s / rates[O.SLIDING], 1),
                               "7b_prefill_full_call": round(f_f / rates[O.FULL], 1),
                               "long_stack_prefill_32_layers": round(long_s, 1)}}


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
            "cpu_model": _cpu_model(), "precision": "fp64 (NumPy)", "kind": "oracle",
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
