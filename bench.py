#!/usr/bin/env python3
"""Benchmark of the TTT-layer forward on one MI355X; prints ONE JSON line.

One step = one forward of every layer variant of the library, each at its reference shape:
  * full-batch TTT-Linear, H-ViT^3-T stage 1: B=64, N=3136 (56x56), 2 heads x 32, bf16
  * bidirectional chunked scan, Vision-TTT at 1280x1280 / 16-px patches: B=8, N=6400, 3 x 64, b=64
  * causal TTT-Linear language layer: B=2, N=16384, 12 x 64, b=16
  * causal TTT-MLP language layer: B=4, N=8192, 12 x 64, hidden 256, b=16
Inputs are synthetic (seeded i.i.d. Gaussians of those shapes) and resident in HBM before the
timed region. The four layers' inputs (584 MB) exceed the 256 MB Infinity Cache, so every layer
starts with its inputs evicted by the other three. Within a step the TTT-MLP layer, whose 48
sequential chains occupy 48 CUs, runs on a second stream beside the other three layers (--serial:
all four one after another on one stream).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--serial]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SUITE = ["hvit3t_stage1_fullbatch", "vittt_bidir_1280", "ttt_linear_causal_16k", "ttt_mlp_causal_8k"]
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
# Kernel sources and the build script (compiler flags) of each layer, for the traffic-counter
# freshness check: a change to any of them makes the stored counters stale.
_BUILD = "test_sequence_layers_amd/build.py"
KERNEL_SOURCES = {
    "fullbatch": ["test_sequence_layers_amd/csrc/fullbatch.hip", "test_sequence_layers_amd/csrc/device.hpp", _BUILD],
    "bidir": ["test_sequence_layers_amd/csrc/chunked.hip", "test_sequence_layers_amd/csrc/device.hpp", _BUILD],
    "causal": ["test_sequence_layers_amd/csrc/chunked.hip", "test_sequence_layers_amd/csrc/device.hpp", _BUILD],
    "mlp": ["test_sequence_layers_amd/csrc/mlp.hip", "test_sequence_layers_amd/csrc/device.hpp", _BUILD],
}


def alg_flops(wl) -> float:
    """Algorithmic flops of one layer forward (per token and head: full-batch 6d^2, bidirectional
    12d^2, causal TTT-Linear 6d^2 + 4bd, TTT-MLP 14 d Dh + 4b(d + Dh))."""
    d, b = wl.D, wl.chunk
    per = {"fullbatch": 6 * d * d, "bidir": 12 * d * d, "causal": 6 * d * d + 4 * b * d,
           "mlp": 14 * d * wl.Dh + 4 * b * (d + wl.Dh)}[wl.op]
    return float(per) * wl.tokens * wl.H


def source_hash(op: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[op]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(op: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{op}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_hash(op):
        return None
    return rec.get("traffic_bytes_per_launch")


def to_device(x, torch):
    import numpy as np

    def cv(a):
        if x.wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = {"q": cv(x.q), "k": cv(x.k), "v": cv(x.v)}
    if x.wl.op == "mlp":
        d["w1"] = torch.from_numpy(x.w1).cuda()
        d["w2"] = torch.from_numpy(x.w2).cuda()
    else:
        d["w0"] = torch.from_numpy(x.w0).cuda()
    d["o"] = torch.empty_like(d["q"])
    return d


def make_call(T, wl, d, torch):
    op = {"fullbatch": T.TTT_OP_FULLBATCH, "causal": T.TTT_OP_CAUSAL, "bidir": T.TTT_OP_BIDIR,
          "mlp": T.TTT_OP_MLP}[wl.op]
    need = T.ttt_workspace_size(op, T.TTT_BF16, wl.B, wl.H, wl.N, wl.D, wl.Dh, wl.chunk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if wl.op == "fullbatch":
        return lambda: T.ttt_forward_fullbatch(d["q"], d["k"], d["v"], d["w0"], wl.eta, o=d["o"], workspace=ws)
    if wl.op == "causal":
        return lambda: T.ttt_forward_chunked_causal(d["q"], d["k"], d["v"], d["w0"], wl.chunk, wl.eta, o=d["o"],
                                                    workspace=ws)
    if wl.op == "bidir":
        return lambda: T.ttt_forward_chunked_bidir(d["q"], d["k"], d["v"], d["w0"], wl.chunk, wl.eta, o=d["o"],
                                                   workspace=ws)
    return lambda: T.ttt_mlp_forward(d["q"], d["k"], d["v"], d["w1"], d["w2"], wl.chunk, wl.eta, o=d["o"],
                                     workspace=ws)


def cpu_baseline(inputs) -> dict:
    """The fp64 oracle, single-threaded, on a bounded sample of every layer (a subset of the
    independent (batch, head) pairs), scaled to the whole suite step."""
    from threadpoolctl import threadpool_limits

    from oracle import ttt_oracle as O

    samples = {"hvit3t_stage1_fullbatch": (64, 2), "vittt_bidir_1280": (8, 3), "ttt_linear_causal_16k": (2, 12),
               "ttt_mlp_causal_8k": (1, 12)}  # (batches, heads) of each layer that the oracle runs (about 10 s)
    total_s = 0.0
    desc = []
    with threadpool_limits(limits=1):
        for name in SUITE:
            x = inputs[name]
            wl = x.wl
            nb, nh = samples[name]
            sl = (slice(0, nb), slice(None), slice(0, nh))
            q, k, v = x.q64[sl], x.k64[sl], x.v64[sl]
            t0 = time.perf_counter()
            if wl.op == "fullbatch":
                O.fullbatch(q, k, v, x.w0[:nh], wl.eta)
            elif wl.op == "bidir":
                O.chunked_bidir(q, k, v, x.w0[:nh], wl.eta, wl.chunk)
            elif wl.op == "causal":
                O.chunked_causal(q, k, v, x.w0[:nh], wl.eta, wl.chunk)
            else:
                O.mlp_causal(q, k, v, x.w1[:nh], x.w2[:nh], wl.eta, wl.chunk)
            dt = time.perf_counter() - t0
            scale = (wl.B * wl.H) / (nb * nh)
            total_s += dt * scale
            desc.append(f"{name}: {nb}x{nh} of {wl.B}x{wl.H} (batch x head) pairs in {dt:.2f} s")
    tokens = sum(inputs[n].wl.tokens for n in SUITE)
    return {"value": tokens / total_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "fp64 numpy oracle, one thread; " + "; ".join(desc) +
                      "; each layer's time scaled by its (batch, head) count"}


def copy_calibration(torch, reps: int = 5) -> None:
    """A plain copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings."""
    n = 1 << 28  # 256 Mi floats = 1 GiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}))


def counter_means(path: str) -> dict:
    """Mean Counter_Value (KiB) per kernel name of a rocprofv3 --pmc counter_collection.csv."""
    import csv

    acc = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(pmc_dir: str) -> int:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic_<op>.json (HBM bytes per
    layer launch). Expects <pmc_dir>/pmc_<layer>_<COUNTER>/run_counter_collection.csv for every
    suite layer and pmc_copy_<COUNTER> from `--copy-calibration`; each counter is scaled by
    (bytes the 1 GiB copy moved) / (what the counter read for that copy)."""
    from test_sequence_layers_amd import synth

    def csv_path(tag, counter):
        return os.path.join(pmc_dir, f"pmc_{tag}_{counter}", "run_counter_collection.csv")

    scale = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [v for k, v in counter_means(csv_path("copy", counter)).items() if "copyBuffer" in k]
        scale[counter] = (1 << 30) / (copy[0] * 1024.0)
    for name in SUITE:
        wl = synth.WORKLOADS[name]
        kernels = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            for k, kib in counter_means(csv_path(name, counter)).items():
                if "ttt::" in k or "_ZN3ttt" in k:
                    kernels.setdefault(k, {})[counter] = kib * 1024.0 * scale[counter]
        total = sum(v.get("FETCH_SIZE", 0.0) + v.get("WRITE_SIZE", 0.0) for v in kernels.values())
        rec = {"layer": name, "op": wl.op, "traffic_bytes_per_launch": total,
               "algorithmic_bytes_per_launch": wl.io_bytes, "counter_scale": scale,
               "per_kernel_bytes": kernels, "source_sha256": source_hash(wl.op)}
        with open(os.path.join(ROOT, "profiles", f"traffic_{wl.op}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{name}: {total / 1e6:.2f} MB per launch (algorithmic {wl.io_bytes / 1e6:.2f} MB)")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true", help="run the layers of a step one after another on one stream")
    ap.add_argument("--layers", default=",".join(SUITE), help="comma-separated subset of the suite (profiling)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--write-traffic", metavar="PMC_DIR", help="write profiles/traffic_<op>.json from counter runs")
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(args.write_traffic)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); every (batch, head) "
              "pair is independent, so N GPUs would each run this step on their own shard.", file=sys.stderr)
        return 2

    import torch

    import test_sequence_layers_amd as T
    from test_sequence_layers_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    T.load_library()  # fails loudly when the HIP library is missing
    if args.copy_calibration:
        copy_calibration(torch)
        return 0

    layers = [n for n in args.layers.split(",") if n]
    inputs = {n: synth.make_inputs(synth.WORKLOADS[n]) for n in layers}
    dev = {n: to_device(inputs[n], torch) for n in layers}
    calls = {n: make_call(T, inputs[n].wl, dev[n], torch) for n in layers}
    stream = torch.cuda.current_stream()
    # The TTT-MLP layer is one workgroup per (batch, head) chain: 48 chains hold 48 of the 256 CUs for
    # its whole run and leave the rest idle. The layers share no data, so a step runs the MLP on a
    # second stream (default priority) beside the other layers. Steps never overlap: each stream's
    # work of a step starts only after the other stream has finished its work of the previous step.
    side = torch.cuda.Stream() if "ttt_mlp_causal_8k" in layers and len(layers) > 1 and not args.serial else None
    layer_stream = {n: (side if side is not None and n == "ttt_mlp_causal_8k" else stream) for n in layers}
    order = sorted(layers, key=lambda n: layer_stream[n] is stream)  # the side-stream launch first
    main_done = torch.cuda.Event()
    side_done = [torch.cuda.Event()]  # the side stream's last recorded event

    def step(marks=None, layer=None):
        if side is not None:
            stream.wait_event(side_done[0])  # both as last recorded: the previous step's work on each stream
            side.wait_event(main_done)
        for n in order:
            st = layer_stream[n]
            with torch.cuda.stream(st):
                if marks is not None and n == layer:
                    marks[0].record(st)
                calls[n]()
                if marks is not None and n == layer:
                    marks[1].record(st)
        if side is not None:
            if marks is not None and layer_stream[layer] is side:
                side_done[0] = marks[1]  # the timing event after the side stream's layer also marks its end
            else:
                side_done[0] = torch.cuda.Event()
                side_done[0].record(side)
            main_done.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-layer times: each layer alone, `reps` back-to-back calls between one pair of events (the
    # events' own cost amortised over the calls). A short spin kernel first lets the host queue
    # the calls ahead of the GPU, so that launch overhead on the host does not show in the time.
    reps = max(args.steps, 10)
    layer_ms = {}
    for n in layers:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        calls[n]()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(1_000_000)
        e0.record(stream)
        for _ in range(reps):
            calls[n]()
        e1.record(stream)
        torch.cuda.synchronize()
        layer_ms[n] = e0.elapsed_time(e1) / reps
    dom = max(layers, key=lambda n: layer_ms[n])

    # Timed region: whole steps; one pair of events per step brackets the dominant layer's launch,
    # for its live average duration (the roofline entry).
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i], dom)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps

    ms_per_step = elapsed * 1000.0 / args.steps
    tokens = sum(inputs[n].wl.tokens for n in layers)
    per_layer = {}
    for n in layers:
        wl = inputs[n].wl
        s = layer_ms[n] / 1000.0
        per_layer[n] = {
            "op": wl.op, "B": wl.B, "N": wl.N, "H": wl.H, "D": wl.D, "chunk": wl.chunk, "Dh": wl.Dh,
            "ms": round(layer_ms[n], 5), "tokens_per_s": wl.tokens / s,
            "alg_GBs": wl.io_bytes / s / 1e9, "hbm_frac": wl.io_bytes / s / 1e9 / PEAK_HBM_GBS,
            "alg_TFLOPs": alg_flops(wl) / s / 1e12, "mfma_frac": alg_flops(wl) / s / 1e12 / PEAK_BF16_TFLOPS,
        }
    wl = inputs[dom].wl
    s = dom_ms / 1000.0
    if wl.op == "mlp":
        ach = alg_flops(wl) / s / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS}
    else:
        ach = wl.io_bytes / s / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    roof["traffic"] = load_traffic(wl.op)
    roof["kernel_layer"] = dom
    roof["launch_ms"] = round(dom_ms, 5)

    out = {
        "metric": "TTT-layer fwd tokens/sec at N=3136/6400/16384; % of HBM-BW roofline",
        "value": tokens / (ms_per_step / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ttt_layer_suite", "layers": layers, "tokens_per_step": tokens,
                   "parallelism": "single GPU",
                   "schedule": "serial" if side is None else "TTT-MLP on a second stream beside the other layers"},
        "roofline": roof,
        "per_layer": per_layer,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
