#!/usr/bin/env python3
"""Benchmark of the TTT-layer forward on one MI355X; prints ONE JSON line.

One step = one forward of every layer variant of the library, each at its reference shape:
  * full-batch TTT-Linear, H-ViT^3-T stage 1: B=64, N=3136 (56x56), 2 heads x 32, bf16
  * bidirectional chunked scan, Vision-TTT at 1280x1280 / 16-px patches: B=8, N=6400, 3 x 64, b=64
  * causal TTT-Linear language layer: B=2, N=16384, 12 x 64, b=16
  * causal TTT-MLP language layer: B=4, N=8192, 12 x 64, hidden 256, b=16
The metric's N = 3136 / 6400 / 16384 are the first three (`metric_layers` in the output: their cold
per-layer tokens/s and fraction of the 8 TB/s HBM peak). Per-layer figures are timed with each
layer alone and its inputs rotated over copies totalling more than 1 GiB, so that every call
reads them from HBM (cold); the warm figures (same inputs back to back) are reported beside them.
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SUITE = ["hvit3t_stage1_fullbatch", "vittt_bidir_1280", "ttt_linear_causal_16k", "ttt_mlp_causal_8k"]
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 1200 * 2 ** 20   # cold per-layer timing: input copies rotated over more than this
SPIN_CYCLES = 25_000_000        # GPU spin before a timed sequence of calls, so the host queues them all
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


# CPU baseline sample: per layer, the (batch, head) slices the oracle runs, as tasks of
# (batches, heads); each task's time is scaled by the layer's pair count over the pairs sampled
# from that layer.
CPU_SAMPLE = {
    "hvit3t_stage1_fullbatch": [(8, 2)] * 2,   # 16 of 64 batches
    "vittt_bidir_1280": [(1, 3)] * 2,          # 2 of 8 batches
    "ttt_linear_causal_16k": [(1, 1)] * 4,     # 4 of 24 (batch, head) pairs
    "ttt_mlp_causal_8k": [(1, 1)] * 8,         # 8 of 48 (batch, head) pairs
}


def _oracle_task(args):
    """One oracle call on a (batch, head) slice, single-threaded; returns its duration (s)."""
    from threadpoolctl import threadpool_limits

    from oracle import ttt_oracle as O

    op, eta, chunk, q, k, v, states = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if op == "fullbatch":
            O.fullbatch(q, k, v, states[0], eta)
        elif op == "bidir":
            O.chunked_bidir(q, k, v, states[0], eta, chunk)
        elif op == "causal":
            O.chunked_causal(q, k, v, states[0], eta, chunk)
        else:
            O.mlp_causal(q, k, v, states[0], states[1], eta, chunk)
        return time.perf_counter() - t0


def cpu_workers() -> int:
    """Host cores for the oracle: OMP_NUM_THREADS (the host threads this process may use) or the core count, at most
    16 (a host's share per GPU)."""
    n = int(os.environ.get("OMP_NUM_THREADS") or 0) or (os.cpu_count() or 1)
    return max(1, min(16, n, os.cpu_count() or 1))


def cpu_baseline(inputs, runs: int = 3) -> dict:
    """The fp64 oracle as it stands, on the host's cores: a bounded sample of (batch, head) slices of
    every layer (CPU_SAMPLE), one single-threaded task per slice, spread over a pool of worker
    processes. Each run's time for the whole suite step is the sum over tasks of (task time x the
    layer's pairs / the pairs sampled from that layer), divided by the worker count (the slices are independent, so
    the full step would keep every core busy). One warm-up run, then the median of `runs`."""
    import multiprocessing as mp
    import statistics
    from concurrent.futures import ProcessPoolExecutor

    tasks, scales, desc = [], [], []
    for name in SUITE:
        if name not in inputs:
            continue
        x = inputs[name]
        wl = x.wl
        hb = 0
        n_pairs = sum(nb * nh for nb, nh in CPU_SAMPLE[name])
        for nb, nh in CPU_SAMPLE[name]:
            # consecutive tasks take consecutive heads, then the next batches
            b0, h0 = (hb // wl.H) * nb % wl.B, hb % wl.H
            hb += nh
            sl = (slice(b0, b0 + nb), slice(None), slice(h0, h0 + nh))
            st = (x.w1[h0:h0 + nh], x.w2[h0:h0 + nh]) if wl.op == "mlp" else (x.w0[h0:h0 + nh],)
            tasks.append((wl.op, wl.eta, wl.chunk, np.ascontiguousarray(x.q64[sl]), np.ascontiguousarray(x.k64[sl]),
                          np.ascontiguousarray(x.v64[sl]), st))
            scales.append(wl.B * wl.H / n_pairs)
        desc.append(f"{name}: {n_pairs} of {wl.B * wl.H} (batch, head) pairs")
    cores = cpu_workers()
    ests, walls = [], []
    with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn")) as ex:
        for run in range(runs + 1):
            t0 = time.perf_counter()
            durs = list(ex.map(_oracle_task, tasks))
            walls.append(time.perf_counter() - t0)
            ests.append(sum(d * sc for d, sc in zip(durs, scales)) / cores)
    step_s = statistics.median(ests[1:])
    tokens = sum(inputs[n].wl.tokens for n in SUITE if n in inputs)
    return {"value": tokens / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 numpy oracle, {cores} worker processes of one thread each; "
                       + "; ".join(desc) + f"; {len(tasks)} single-threaded tasks per run, each task's time "
                       f"scaled by its layer's pair count over the pairs sampled from it, the sum divided by "
                       f"{cores}; one warm-up run, then the "
                       f"median of {runs} (suite step {step_s:.2f} s; sample wall times "
                       + ", ".join(f"{w:.2f}" for w in walls[1:]) + " s)")}


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


def extra_legs(T, torch, inputs, dev, time_rotated) -> dict:
    """Legs outside the suite step, each timed like the layers (cold, inputs rotated over > 1 GiB):
      * dwconv_kv_vittt_1280: the Vision-TTT Conv2d preprocessing, a depth-wise 3x3 convolution of
        K and of V over the 80 x 80 token grid (8 images, C = 3 x 64), bf16;
      * vittt_bidir_1280_with_dwconv: that preprocessing followed by the bidirectional scan;
      * vittt_bidir2d_1280: the raster- plus column-order bidirectional scans of the 80 x 80 grid
        (algorithmic bytes: q, k, v read and o written once);
      * fullbatch_backward_hvit3t_stage1: the full-batch layer's backward pass (dQ, dK, dV, dW0) at
        the H-ViT^3-T stage-1 shape, bf16;
      * block_epilogue_hvit3t_stage1: the ViT^3 block epilogue over that layer's 200,704 tokens
        (C = C_out = 64), bf16;
      * causal_backward_16k, bidir_backward_vittt_1280: the backward passes (dQ, dK, dV, dW0) of the
        causal TTT-Linear layer (2 x 16384 x 12 x 64, b = 16) and of the Vision-TTT bidirectional
        scan (8 x 6400 x 3 x 64, b = 64), bf16;
      * design-space variants: 4 full-batch epochs at the H-ViT^3-T stage-1 shape, the Vision-TTT scan
        with b = 16, and a 4x wider inner MLP (Dh = 1024) at a reduced shape;
      * vit3s_fullbatch: the ViT^3-S-shaped full-batch layer (64 images x 196 tokens, 6 heads of 64,
        bf16), which runs as one launch (one workgroup per (image, head))."""
    from test_sequence_layers_amd import synth

    out = {}
    vw = synth.WORKLOADS["vit3s_fullbatch"]
    dv3 = to_device(synth.make_inputs(vw), torch)
    cold, warm, nsets = time_rotated(lambda d: make_call(T, vw, d, torch), dv3, vw.io_bytes)
    sec = cold / 1000.0
    out["vit3s_fullbatch"] = {
        "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": vw.tokens / sec, "alg_bytes": vw.io_bytes,
        "alg_GBs": vw.io_bytes / sec / 1e9, "hbm_frac": vw.io_bytes / sec / 1e9 / PEAK_HBM_GBS,
        "hbm_frac_warm": vw.io_bytes / (warm / 1000.0) / 1e9 / PEAK_HBM_GBS,
        "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB)"}
    del dv3
    name = "vittt_bidir_1280"
    if name not in inputs:
        return out
    wl = inputs[name].wl
    Hi = Wi = 80
    C = wl.H * wl.D
    rs = np.random.default_rng(4242)
    wk, wv = [torch.from_numpy((rs.standard_normal((C, 3, 3)) / 3.0).astype(np.float32)).cuda() for _ in range(2)]
    bk, bv = [torch.from_numpy((rs.standard_normal(C) * 0.05).astype(np.float32)).cuda() for _ in range(2)]
    need = T.ttt_workspace_size(T.TTT_OP_BIDIR, T.TTT_BF16, wl.B, wl.H, wl.N, wl.D, 0, wl.chunk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    kc, vc = torch.empty_like(dev[name]["k"]), torch.empty_like(dev[name]["v"])

    def conv(d):
        return lambda: (T.ttt_dwconv3x3(d["k"], wk, bk, height=Hi, width=Wi, y=kc),
                        T.ttt_dwconv3x3(d["v"], wv, bv, height=Hi, width=Wi, y=vc))

    def chain(d):
        def run():
            conv(d)()
            T.ttt_forward_chunked_bidir(d["q"], kc, vc, d["w0"], wl.chunk, wl.eta, o=d["o"], workspace=ws)
        return run

    conv_bytes = 4 * wl.B * wl.N * C * 2          # read K and V, write both convolved
    fb = "hvit3t_stage1_fullbatch"
    if fb in inputs:  # the full-batch layer's backward pass at the H-ViT^3-T stage-1 shape
        fw = inputs[fb].wl
        rs2 = np.random.default_rng(4343)
        d_o = torch.from_numpy((rs2.standard_normal((fw.B, fw.N, fw.H, fw.D)) / np.sqrt(fw.D)).astype(np.float32)
                               ).cuda().to(torch.bfloat16)
        need_b = T.ttt_workspace_size(T.TTT_OP_FULLBATCH_BWD, T.TTT_BF16, fw.B, fw.H, fw.N, fw.D)
        wsb = torch.empty(need_b, dtype=torch.uint8, device="cuda")
        grads = [torch.empty_like(dev[fb]["q"]) for _ in range(3)]
        dw0 = torch.empty((fw.B, fw.H, fw.D, fw.D), dtype=torch.float32, device="cuda")

        def bwd(d):
            return lambda: T.ttt_backward_fullbatch(d["q"], d["k"], d["v"], d["w0"], d_o, fw.eta, d_q=grads[0],
                                                    d_k=grads[1], d_v=grads[2], d_w0=dw0, workspace=wsb)

        # the ViT^3 block epilogue at this width: [O * sigmoid(G), X] Wo^T + b over the layer's tokens
        Mt, Ct = fw.B * fw.N, fw.H * fw.D
        ep_in = {key: torch.from_numpy((rs2.standard_normal((Mt, Ct)) * 0.3).astype(np.float32)).cuda()
                 .to(torch.bfloat16) for key in ("q", "k", "v")}
        wpj = torch.from_numpy((rs2.standard_normal((Ct, 2 * Ct)) / np.sqrt(2 * Ct)).astype(np.float32)).cuda() \
            .to(torch.bfloat16)
        bpj = torch.zeros(Ct, dtype=torch.float32, device="cuda")
        yep = torch.empty((Mt, Ct), dtype=torch.bfloat16, device="cuda")

        def epi(d):
            return lambda: T.ttt_block_epilogue(d["q"], d["k"], d["v"], wpj, bpj, y=yep)

        nbe = 4 * Mt * Ct * 2                      # read O, G, X; write y
        cold, warm, nsets = time_rotated(epi, ep_in, nbe)
        sec = cold / 1000.0
        out["block_epilogue_hvit3t_stage1"] = {
            "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": Mt / sec, "alg_bytes": nbe,
            "alg_GBs": nbe / sec / 1e9, "hbm_frac": nbe / sec / 1e9 / PEAK_HBM_GBS,
            "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB); M = {Mt} tokens, C = C_out = {Ct}"}
        nb = 7 * fw.B * fw.N * fw.H * fw.D * 2    # read q, k, v, dO; write dq, dk, dv
        cold, warm, nsets = time_rotated(bwd, dev[fb], nb)
        sec = cold / 1000.0
        out["fullbatch_backward_hvit3t_stage1"] = {
            "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": fw.tokens / sec, "alg_bytes": nb,
            "alg_GBs": nb / sec / 1e9, "hbm_frac": nb / sec / 1e9 / PEAK_HBM_GBS,
            "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB); dO fixed"}
    # backward passes of the chunked layers at their full sizes (dO fixed, inputs rotated)
    for lname, leg, op, fn in (("ttt_linear_causal_16k", "causal_backward_16k", T.TTT_OP_CAUSAL_BWD,
                                T.ttt_backward_chunked_causal),
                               ("vittt_bidir_1280", "bidir_backward_vittt_1280", T.TTT_OP_BIDIR_BWD,
                                T.ttt_backward_chunked_bidir)):
        if lname not in inputs:
            continue
        cw = inputs[lname].wl
        rs3 = np.random.default_rng(4444)
        d_oc = torch.from_numpy((rs3.standard_normal((cw.B, cw.N, cw.H, cw.D)) / np.sqrt(cw.D)).astype(np.float32)
                                ).cuda().to(torch.bfloat16)
        wsc = torch.empty(max(T.ttt_workspace_size(op, T.TTT_BF16, cw.B, cw.H, cw.N, cw.D, 0, cw.chunk), 1),
                          dtype=torch.uint8, device="cuda")
        gc = [torch.empty_like(dev[lname]["q"]) for _ in range(3)]
        dw0c = torch.empty((cw.B, cw.H, cw.D, cw.D), dtype=torch.float32, device="cuda")

        def cbwd(d, cw=cw, fn=fn, d_oc=d_oc, wsc=wsc, gc=gc, dw0c=dw0c):
            return lambda: fn(d["q"], d["k"], d["v"], d["w0"], d_oc, cw.chunk, cw.eta, d_q=gc[0], d_k=gc[1],
                              d_v=gc[2], d_w0=dw0c, workspace=wsc)

        nbc = 7 * cw.B * cw.N * cw.H * cw.D * 2   # read q, k, v, dO; write dq, dk, dv
        cold, warm, nsets = time_rotated(cbwd, dev[lname], nbc)
        sec = cold / 1000.0
        out[leg] = {"ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": cw.tokens / sec,
                    "alg_bytes": nbc, "alg_GBs": nbc / sec / 1e9, "hbm_frac": nbc / sec / 1e9 / PEAK_HBM_GBS,
                    "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB); dO fixed"}
    need2 = T.ttt_workspace_size(T.TTT_OP_BIDIR2D, T.TTT_BF16, wl.B, wl.H, wl.N, wl.D, 0, wl.chunk)
    ws2 = torch.empty(need2, dtype=torch.uint8, device="cuda")

    def scan2d(d):
        return lambda: T.ttt_forward_chunked_bidir2d(d["q"], d["k"], d["v"], d["w0"], wl.chunk, Hi, Wi, wl.eta,
                                                     o=d["o"], workspace=ws2)

    for leg, make, nbytes in (("dwconv_kv_vittt_1280", conv, conv_bytes),
                              ("vittt_bidir_1280_with_dwconv", chain, conv_bytes + wl.io_bytes),
                              ("vittt_bidir2d_1280", scan2d, wl.io_bytes)):
        cold, warm, nsets = time_rotated(make, dev[name], nbytes)
        s = cold / 1000.0
        out[leg] = {"ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": wl.tokens / s,
                    "alg_bytes": nbytes, "alg_GBs": nbytes / s / 1e9, "hbm_frac": nbytes / s / 1e9 / PEAK_HBM_GBS,
                    "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB)"}
    # design-space variants (ViT^3 review, design-space study; Vision-TTT's b = 16)
    if fb in inputs:  # 4 full-batch epochs at the H-ViT^3-T stage-1 shape
        fw = inputs[fb].wl
        wse = torch.empty(max(T.ttt_workspace_size(T.TTT_OP_FULLBATCH, T.TTT_BF16, fw.B, fw.H, fw.N, fw.D), 1),
                          dtype=torch.uint8, device="cuda")

        def ep4(d, fw=fw, wse=wse):
            return lambda: T.ttt_forward_fullbatch_epochs(d["q"], d["k"], d["v"], d["w0"], 4, fw.eta, o=d["o"],
                                                          workspace=wse)

        cold, warm, nsets = time_rotated(ep4, dev[fb], fw.io_bytes)
        sec = cold / 1000.0
        out["fullbatch_4_epochs_hvit3t_stage1"] = {
            "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": fw.tokens / sec,
            "alg_bytes": fw.io_bytes, "alg_GBs": fw.io_bytes / sec / 1e9,
            "hbm_frac": fw.io_bytes / sec / 1e9 / PEAK_HBM_GBS,
            "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB); 4 epochs over one pass of K and V"}
    # the Vision-TTT scan with b = 16 (its summary's mini-batch size), same tensors as the b = 64 layer
    ws16 = torch.empty(max(T.ttt_workspace_size(T.TTT_OP_BIDIR, T.TTT_BF16, wl.B, wl.H, wl.N, wl.D, 0, 16), 1),
                       dtype=torch.uint8, device="cuda")

    def bidir16(d):
        return lambda: T.ttt_forward_chunked_bidir(d["q"], d["k"], d["v"], d["w0"], 16, wl.eta, o=d["o"],
                                                   workspace=ws16)

    cold, warm, nsets = time_rotated(bidir16, dev[name], wl.io_bytes)
    sec = cold / 1000.0
    out["vittt_bidir_1280_b16"] = {
        "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": wl.tokens / sec,
        "alg_bytes": wl.io_bytes, "alg_GBs": wl.io_bytes / sec / 1e9, "hbm_frac": wl.io_bytes / sec / 1e9 / PEAK_HBM_GBS,
        "timing": f"cold: inputs rotated over {nsets} copies (> 1 GiB); mini-batches of 16 tokens"}
    # a wider inner MLP (Dh = 1024, 4 x the suite's) at a reduced shape (the matrix-core kernel whose fp32
    # state lives in the workspace)
    mw = synth.WORKLOADS["ttt_mlp_causal_8k"].with_(B=1, N=1024, H=12, Dh=1024, seed=4545)
    xm = synth.make_inputs(mw)
    dm = to_device(xm, torch)
    wsm = torch.empty(T.ttt_workspace_size(T.TTT_OP_MLP, T.TTT_BF16, mw.B, mw.H, mw.N, mw.D, mw.Dh, mw.chunk),
                      dtype=torch.uint8, device="cuda")

    def mlpw(d):
        return lambda: T.ttt_mlp_forward(d["q"], d["k"], d["v"], d["w1"], d["w2"], mw.chunk, mw.eta, o=d["o"],
                                         workspace=wsm)

    # compute-bound (6 MB of I/O against 12 GFLOP): two input sets alternate instead of a 1 GiB rotation
    cold, warm, nsets = time_rotated(mlpw, dm, ROTATE_BYTES)
    sec = cold / 1000.0
    flops = alg_flops(mw)
    out["ttt_mlp_wide_dh1024_1x1024x12"] = {
        "ms": round(cold, 5), "ms_warm": round(warm, 5), "tokens_per_s": mw.tokens / sec,
        "alg_TFLOPs": flops / sec / 1e12, "mfma_frac": flops / sec / 1e12 / PEAK_BF16_TFLOPS,
        "timing": f"{nsets} input sets alternating; B = 1, N = 1024, 12 heads of 64, Dh = 1024, b = 16 "
                  "(matrix-core kernel with the fp32 state in the workspace)"}
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true", help="run the layers of a step one after another on one stream")
    ap.add_argument("--layers", default=",".join(SUITE), help="comma-separated subset of the suite (profiling)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-extra-legs", action="store_true", help="skip the legs outside the suite step")
    ap.add_argument("--per-layer-only", action="store_true",
                    help="only the per-layer cold and warm timings, one JSON line per layer (profiling)")
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

    # Per-layer times, each layer alone, many calls between one pair of events on the stream the
    # kernels run on (the events' own cost amortised over the calls); a spin kernel first lets the
    # host queue all the calls ahead of the GPU, so that host time per call does not show.
    #  * cold: the calls rotate over copies of the layer's inputs and outputs totalling more than
    #    1 GiB, so each call finds its inputs evicted from the 256 MB Infinity Cache;
    #  * warm: back-to-back calls on one set of inputs (they fit in the Infinity Cache).
    def time_rotated(make, d0, io_bytes):
        """(cold ms, warm ms, input sets) of the calls make(d) builds, d rotating over copies of d0."""
        nsets = max(2, -(-ROTATE_BYTES // io_bytes))
        sets = [d0] + [{key: (t.clone() if key in ("q", "k", "v") else (torch.empty_like(t) if key == "o" else t))
                        for key, t in d0.items()} for _ in range(nsets - 1)]
        rcalls = [make(d) for d in sets]
        res = {}
        for label, seq in (("cold", [rcalls[i % nsets] for i in range(max(args.steps, 3 * nsets))]),
                           ("warm", [rcalls[0]] * max(args.steps, 10))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for c in rcalls:
                c()
            if hasattr(torch.cuda, "_sleep"):  # (about 10 ms: the binding takes ~20 us of host time a call)
                torch.cuda._sleep(SPIN_CYCLES)
            e0.record(stream)
            for c in seq:
                c()
            e1.record(stream)
            torch.cuda.synchronize()
            res[label] = e0.elapsed_time(e1) / len(seq)
        return res["cold"], res["warm"], nsets

    layer_ms, layer_ms_warm, rot_sets = {}, {}, {}
    for n in layers:
        wl = inputs[n].wl
        layer_ms[n], layer_ms_warm[n], rot_sets[n] = time_rotated(
            lambda d, wl=wl: make_call(T, wl, d, torch), dev[n], wl.io_bytes)
    if args.per_layer_only:
        for n in layers:
            print(json.dumps({"layer": n, "ms_cold": layer_ms[n], "ms_warm": layer_ms_warm[n],
                              "rotated_input_sets": rot_sets[n]}))
        return 0
    dom = max(layers, key=lambda n: layer_ms[n])

    # Timed region: whole steps; one pair of events per step brackets the dominant layer's launch,
    # for its live average duration (the roofline entry). The warm-up steps are repeated right before
    # it, after the per-layer timing. The legs outside the step are measured after it: run before
    # it, they left the step about 4 % slower (the TTT-MLP launch 0.90 instead of 0.87 ms, the same
    # in back-to-back runs, so not a clock or temperature effect).
    for _ in range(args.warmup):
        step()
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i], dom)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps

    ms_per_step = elapsed * 1000.0 / args.steps
    extra = {} if args.no_extra_legs else extra_legs(T, torch, inputs, dev, time_rotated)
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
            "timing": f"cold: inputs rotated over {rot_sets[n]} copies (> 1 GiB)",
            "ms_warm": round(layer_ms_warm[n], 5),
            "hbm_frac_warm": wl.io_bytes / (layer_ms_warm[n] / 1000.0) / 1e9 / PEAK_HBM_GBS,
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
        "extra_legs": extra,
        "metric_layers": {str(inputs[n].wl.N): {"layer": n, "tokens_per_s": per_layer[n]["tokens_per_s"],
                                                 "hbm_frac": per_layer[n]["hbm_frac"]}
                          for n in ("hvit3t_stage1_fullbatch", "vittt_bidir_1280", "ttt_linear_causal_16k")
                          if n in per_layer},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
