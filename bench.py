#!/usr/bin/env python3
"""Benchmark of the activation-sparse gated FFN forward pass on one MI355X.

A step is one sparse FFN forward pass (gate GEMM + selection + TwELL pack +
routing, fused sparse up/down, dense backup) over one batch of synthetic
tokens, on one FFN layer. Steps rotate over `--layers` distinct copies of the
layer's weights so that successive steps read different HBM addresses and the
256 MB last-level cache cannot serve them (a model has many such layers).

Prints one JSON line: tokens/s per FFN layer (value), the effective HBM rate
on the weight bytes the method touches, the own dense FFN on the same inputs
(speedup), the roofline of the dominant kernel measured with HIP events, and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_BF16_TFLOPS = 2500.0     # dense bf16 matrix cores
WORKLOADS = {
    "c2": "decode-relu-bf16-2048x8192",
    "c3": "lopa-relu-thresh-bf16-4096x14336-r512",
    "c4": "wina-silu-topk-bf16-4096x11008",
    "c5": "prefill-hybrid-relu-bf16-2048x8192",
    "c6": "input-wina-gate-bf16-2048x8192",
    "c7": "lopa-input-wina-bf16-4096x14336-r512",
    "gsi": "gsi-linear-bf16-4096x14336-k256",
    "moe": "moe-lopa-relu-thresh-bf16-8x4096x14336-r512-top2",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--m", type=int, default=None, help="tokens per step (default: the decode batch)")
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--graph", action="store_true", help="replay the steps from a HIP graph")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (full-gate workloads: c2, c5) after one forward pass")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="profiling mode: run this many sparse steps and one 256 MiB device copy "
                         "(counter calibration), print nothing else")
    return ap.parse_args()


def note(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash() -> str:
    """Hash of every kernel source: stored counter readings apply only to the
    kernels they were taken on."""
    d = os.path.join(ROOT, "activation_sparse_gated_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from synth import make_workload
    import activation_sparse_gated_amd as asg

    asg.load()          # fail loudly without the built library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cid = args.workload
    if cid == "gsi":
        return bench_gsi(args, dev)
    if cid == "moe":
        return bench_moe(args, dev)
    if args.backward:
        return bench_backward(args, dev)
    m = args.m if args.m is not None else {"c2": 1, "c3": 1, "c4": 1, "c5": 4096, "c6": 1, "c7": 1}[cid]
    t_gen = time.time()
    wl = make_workload(cid, m, 0)
    t_gen = time.time() - t_gen
    note(f"inputs {cid} m={m} generated in {t_gen:.1f}s")

    def dev_bf16(a):
        return torch.from_numpy(wl.storage(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {k: (dev_bf16(getattr(wl, k)) if getattr(wl, k) is not None else None)
            for k in ("w_gate", "u", "v", "w_up", "w_down")}
    x = dev_bf16(wl.x)
    bias = torch.from_numpy(wl.bias.astype(np.float32)).to(dev) if wl.bias is not None else None
    tau = torch.from_numpy(wl.tau.astype(np.float32)).to(dev) if wl.tau is not None else None
    sel_kw = dict(bias=bias, tau=tau, k=wl.k)

    layers = []
    for li in range(args.layers):
        w = {k: (v.clone() if v is not None else None) for k, v in base.items()}
        ffn = asg.SparseFFN(d_model=wl.d, d_ff=wl.f, rank=wl.rank, dtype="bf16", act=wl.act, sel=wl.sel,
                            tile_w=wl.T, ell_w=wl.E, max_m=m, w_gate=w["w_gate"], u=w["u"], v=w["v"],
                            w_up=w["w_up"], w_down=w["w_down"], wdown_out_major=True, in_keep=wl.in_keep)
        layers.append((ffn, ffn.new_pack(m), ffn.new_output(m), ffn.new_output(m)))
    torch.cuda.synchronize()

    def sparse_step(i):
        ffn, pack, y, _ = layers[i % len(layers)]
        ffn.forward(x, pack=pack, y=y, **sel_kw)

    def dense_step(i):
        ffn, _, _, yd = layers[i % len(layers)]
        ffn.dense_forward(x, bias=bias, tau=tau, y=yd)

    def timed(step, n, warm, graph=False):
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        if graph:
            s = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(len(layers)):
                    step(i)
            reps = max(1, n // len(layers))
            n = reps * len(layers)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n, n
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            step(warm + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, n

    if args.profile_steps:
        for i in range(args.profile_steps):
            sparse_step(i)
        torch.cuda.synchronize()
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": f"{WORKLOADS[cid]} m={m}",
                          "copy_bytes": src.numel()}))
        return

    def per_step(step, n):
        """Per-step durations (us) from an event pair around each step (a
        separate pass: the events add a little time to every step)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            step(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return {"p10": round(float(np.percentile(us, 10)), 3), "p50": round(float(np.median(us)), 3),
                "p90": round(float(np.percentile(us, 90)), 3), "steps": n}

    # ---- timed region: the sparse forward pass (value) ----
    ms_sparse, steps = timed(sparse_step, args.steps, args.warmup, graph=args.graph)
    note(f"sparse step {ms_sparse * 1e3:.2f} us")
    ms_dense, _ = timed(dense_step, max(20, args.steps // 4), 5, graph=args.graph)
    note(f"dense step {ms_dense * 1e3:.2f} us")
    dist_sparse = per_step(sparse_step, args.steps)
    dist_dense = per_step(dense_step, max(20, args.steps // 4))

    # ---- touched bytes of one step (from the pack the step wrote) ----
    ffn0, pack0, y0, _ = layers[0]
    ffn0.forward(x, pack=pack0, y=y0, **sel_kw)
    torch.cuda.synchronize()
    cnt = pack0.cnt[:m].cpu().numpy()
    route = pack0.route[:m].cpu().numpy().astype(bool)
    idx = pack0.idx[:m].cpu().numpy().view(np.uint16)
    T, E, d, F, r = wl.T, wl.E, wl.d, wl.f, wl.rank
    ntiles = F // T
    active = set()
    entries = 0
    for t in range(m):
        if route[t]:
            continue
        for j in range(ntiles):
            c = int(min(cnt[t, j], E))
            entries += c
            for s in range(c):
                active.add(j * T + int(idx[t, j, s]))
    n_union = len(active)
    gate_bytes = (F * r + r * d) * 2 if r else F * d * 2
    gate_bytes_dense = gate_bytes
    if wl.in_keep:
        # input-side gate: only the kept channels' rows of the input-major W_gate
        # (or V), plus x and the column norms the selection reads
        gate_bytes = (F * r * 2 + wl.in_keep * r * 2 if r else wl.in_keep * F * 2) + m * d * 2 + d * 4
    if wl.sel == "topk":
        gate_bytes = 2 * F * d * 2
        row_bytes = d * 2
    else:
        row_bytes = 2 * d * 2
    pack_bytes = m * ntiles * (4 + E * 4)
    touched = gate_bytes + n_union * row_bytes + 2 * m * d * 2 + 2 * pack_bytes
    n_dense = int(route.sum())
    # the own dense FFN reads every weight once: gate (or U and V), W_up, W_down, x, y
    dense_bytes = (F * r + r * d) * 2 + 2 * F * d * 2 + 2 * m * d * 2 if r else 3 * F * d * 2 + 2 * m * d * 2
    if n_dense:
        touched += 3 * F * d * 2

    # ---- per-kernel durations with HIP events on the library's stream ----
    for ffn, *_ in layers:
        ffn.timing_enable(True, capacity=args.steps + 8)
    for i in range(args.steps):
        sparse_step(i)
    torch.cuda.synchronize()
    kernels = {}
    for kind in ("lowrank_v", "gate", "up", "topk", "updown", "reduce", "fallback"):
        n_tot, ms_tot = 0, 0.0
        for ffn, *_ in layers:
            n, ms = ffn.timing_read(kind)
            n_tot += n
            ms_tot += ms
        if n_tot:
            kernels[kind] = {"launches": n_tot, "avg_us": 1e3 * ms_tot / n_tot}
    for ffn, *_ in layers:
        ffn.timing_enable(False)

    # algorithmic bytes per launch of each kernel
    # algorithmic bytes per launch: each weight byte a kernel must read once,
    # its inputs and its outputs (partial rows and lists are not counted)
    path = ffn0.forward_path(m)
    gate_alg = (F * r * 2 + m * r * 4 if r else F * d * 2 + m * d * 2) + pack_bytes + m * 9
    urow = n_union * d * 2                       # up rows (or down rows) of the union neurons
    alg = {
        "lowrank_v": r * d * 2 + m * d * 2 + m * r * 4,
        "gate": gate_alg,
        "updown": entries * row_bytes + m * d * 2 + m * d * 2 + pack_bytes,
        "topk": m * F * 8 + pack_bytes,
        "reduce": m * d * 2,
    }
    if path == "decode-chunk":
        alg["gate"] = gate_alg + urow
        alg["updown"] = urow + m * d * 2
    elif path == "decode-part":
        alg["gate"] = gate_alg + 2 * urow
        alg["updown"] = m * d * 2
    elif path == "decode-split":
        alg["up"] = urow + m * d * 2
        alg["updown"] = urow + m * d * 2
    elif path == "general" and "up" in kernels:                 # prefill: XCD-sliced up, then down
        alg["up"] = entries * d * 2 + m * d * 2
        alg["updown"] = entries * d * 2 + m * d * 2
    elif path == "general":
        # HBM minimum of the sparse pass: each union neuron's up and down rows
        # once (the per-entry re-reads are cache traffic)
        alg["updown"] = n_union * row_bytes + m * d * 2 + m * d * 2 + pack_bytes
    elif path == "masked-dense":
        # the dense products with the selection applied to every neuron: each
        # weight byte once, the gate values [m x F] written and read, h [m x F]
        alg["gate"] = F * r * 2 + m * r * 4 + m * F * 4              # U t (low rank)
        alg["up"] = (F * d * 2 if r else 2 * F * d * 2) + m * d * 2 + m * F * (4 + 2)
        alg["updown"] = F * d * 2 + m * F * 2 + m * d * 2
    elif path == "topk-masked-dense":
        alg["updown"] = F * d * 2 + m * F * 2 + m * d * 2      # all of W_down, the masked h rows, y
    if wl.sel == "topk":
        alg["gate"] = 2 * F * d * 2 + m * d * 2 + 2 * m * F * 4
    if wl.in_keep:
        # input-side gate: the kept rows of W_gate^T (or V^T) in the channel-group
        # stream, reported under the first-stage kind; the gate kind is the
        # selection and pack (full gate) or U t (low rank)
        alg["lowrank_v"] = wl.in_keep * (r if r else F) * 2 + m * d * 2 + d * 4
        alg["gate"] = (F * r * 2 + m * r * 4 if r else 0) + pack_bytes + m * 9
    dom = max((k for k in kernels if k in alg), key=lambda k: kernels[k]["avg_us"])
    achieved = alg[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tinfo = json.load(fh).get(f"{cid}-m{m}", {}).get(dom)
        if tinfo and tinfo.get("source_sha") == src_hash():
            traffic = tinfo.get("bytes_per_launch")
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": int(alg[dom]), "avg_us": round(kernels[dom]["avg_us"], 3)}
    if m >= 128 and dom == "gate":
        # prefill: the gate GEMM is a dense contraction on matrix cores
        flops = 2.0 * m * F * (r if r else d) + (2.0 * m * r * d if r else 0.0)
        tf = flops / (kernels[dom]["avg_us"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(tf, 1), "peak": MFMA_PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "flops_per_launch": int(flops), "avg_us": round(kernels[dom]["avg_us"], 3)}

    # ---- CPU oracle on a bounded sample of the same workload ----
    # (all the host threads BLAS uses here, then one thread; the oracle is
    # plain NumPy fp64, untuned)
    cpu = cpu1 = None
    host = {}
    if not args.no_cpu:
        from oracle import ffn_oracle as O
        from threadpoolctl import threadpool_info, threadpool_limits
        try:
            host["nproc"] = len(os.sched_getaffinity(0))
        except Exception:
            host["nproc"] = os.cpu_count()
        host["cpu_count"] = os.cpu_count()
        try:
            with open("/proc/cpuinfo") as fh:
                host["cpu_model"] = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
        except Exception:
            host["cpu_model"] = None

        def oracle_rate(seconds):
            t0 = time.time()
            reps = 0
            while time.time() - t0 < seconds or reps == 0:
                O.forward(wl)
                reps += 1
            el = time.time() - t0
            return reps, el

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        reps, el = oracle_rate(args.cpu_seconds)
        cpu = {"value": round(reps * m / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} full oracle forward passes of the {m}-token batch ({el:.1f} s)",
               "nproc": host["nproc"], "cpu_model": host["cpu_model"]}
        with threadpool_limits(limits=1):
            reps1, el1 = oracle_rate(args.cpu_seconds)
        cpu1 = {"value": round(reps1 * m / el1, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{reps1} full oracle forward passes of the {m}-token batch ({el1:.1f} s), one thread"}

    tok_s = m * 1e3 / ms_sparse
    out = {
        "metric": "sparse-FFN tokens/sec + effective HBM GB/s at 90% sparsity, d=4096 (1 GPU)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_sparse, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOADS[cid]} m={m}", "d_model": d, "d_ff": F, "rank": r, "m": m,
                   "tile_w": T, "ell_w": E, "active_neurons": n_union, "routed_tokens": n_dense,
                   "layers_rotated": len(layers),
                   "hip_graph": bool(args.graph), "kernel_path": path},
        "effective_hbm_GBps": round(touched / (ms_sparse * 1e-3) / 1e9, 1),
        "gate_bytes": int(gate_bytes),
        "gate_bytes_saved": int(gate_bytes_dense - gate_bytes) if wl.in_keep else 0,
        "in_keep": int(wl.in_keep),
        "touched_bytes": int(touched),
        "dense_ms_per_step": round(ms_dense, 5),
        "dense_effective_hbm_GBps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(ms_dense / ms_sparse, 3),
        "step_us_dist": dist_sparse,
        "dense_step_us_dist": dist_dense,
        "kernels_us": {k: round(v["avg_us"], 3) for k, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out))


def bench_backward(args, dev):
    """Backward pass of one FFN layer (Sparser/Faster/Lighter page, "Hybrid
    應對非均勻稀疏": training with the compact format and a dense backup):
    a step is one ffn_sparse_backward call (dx and the three fp32 weight
    gradients) for the batch, after one forward pass wrote the pack; steps
    rotate over `--layers` copies of the weights."""
    import numpy as np
    import torch

    import activation_sparse_gated_amd as asg
    from synth import draw_dy, make_workload

    cid = args.workload
    if cid not in ("c2", "c5"):
        raise SystemExit("--backward: full-gate workloads c2 and c5 only")
    m = args.m if args.m is not None else {"c2": 16, "c5": 4096}[cid]
    t_gen = time.time()
    wl = make_workload(cid, m, 0)
    dyh = draw_dy(wl, 1)
    t_gen = time.time() - t_gen
    note(f"inputs {cid} m={m} generated in {t_gen:.1f}s")

    def dev_bf16(a):
        return torch.from_numpy(wl.storage(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {k: dev_bf16(getattr(wl, k)) for k in ("w_gate", "w_up", "w_down")}
    x, dy = dev_bf16(wl.x), dev_bf16(dyh)
    bias = torch.from_numpy(wl.bias.astype(np.float32)).to(dev)
    nl = max(1, min(args.layers, 4))
    layers = []
    for li in range(nl):
        w = {k: (v if li == 0 else v.clone()) for k, v in base.items()}
        ffn = asg.SparseFFN(d_model=wl.d, d_ff=wl.f, rank=0, dtype="bf16", act=wl.act, sel=wl.sel, tile_w=wl.T,
                            ell_w=wl.E, max_m=m, w_gate=w["w_gate"], w_up=w["w_up"], w_down=w["w_down"],
                            wdown_out_major=True)
        pack = ffn.new_pack(m)
        ffn.forward(x, pack=pack, bias=bias)
        grads = [torch.zeros((wl.f, wl.d), dtype=torch.float32, device=dev) for _ in range(3)]
        layers.append((ffn, pack, grads))
    import ctypes
    lib = asg.load()
    wsb = lib.ffn_sparse_backward_workspace_bytes(ctypes.byref(layers[0][0].cfg), m)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    dx = torch.empty((m, wl.d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i):
        ffn, pack, (gg, gu, gd) = layers[i % nl]
        ffn.backward(x, dy, pack, bias=bias, dx=dx, dw_gate=gg, dw_up=gu, dw_down_nm=gd, workspace=ws)

    if args.profile_steps:
        for i in range(args.profile_steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": f"{WORKLOADS[cid]} m={m} backward"}))
        return

    steps = max(5, min(args.steps, 40 if m > 256 else args.steps))
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    note(f"backward step {ms * 1e3:.2f} us")
    e0.record()
    for i in range(steps):
        ffn, pack, _ = layers[i % nl]
        ffn.forward(x, pack=pack, bias=bias)
    e1.record()
    torch.cuda.synchronize()
    ms_fwd = e0.elapsed_time(e1) / steps

    for ffn, *_ in layers:
        ffn.timing_enable(True, capacity=4 * steps + 8)   # up to four dx launches a step
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    kernels = {}
    for kind in ("bw_gate", "bw_neuron", "bw_dx"):
        n_tot, ms_tot = 0, 0.0
        for ffn, *_ in layers:
            n, t = ffn.timing_read(kind)
            n_tot += n
            ms_tot += t
        if n_tot:
            kernels[kind] = {"launches": n_tot, "avg_us": 1e3 * ms_tot / n_tot, "step_us": 1e3 * ms_tot / steps}
    for ffn, *_ in layers:
        ffn.timing_enable(False)
    fwd = None
    from oracle import ffn_oracle as O
    fwd = O.forward(wl)
    mask = fwd["mask"]
    pairs = int(mask.sum())
    n_act = int(mask.any(axis=0).sum())
    d, F = wl.d, wl.f
    # HBM bytes the neuron kernel cannot avoid: each active neuron's W_up and
    # W_down rows, its three fp32 gradient rows read and written, x and dy once,
    # and du, dz of every pair
    alg = {"bw_neuron": n_act * (2 * d * 2 + 3 * d * 8) + 2 * m * d * 2 + pairs * 8,
           "bw_dx": n_act * 2 * d * 2 + pairs * 8 + m * d * 2,
           "bw_gate": F * d * 2 + int(fwd["n_dense"]) * (d * 2 + F * 4)}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    achieved = alg[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "alg_bytes_per_launch": int(alg[dom]),
                "avg_us": round(kernels[dom]["avg_us"], 3)}
    cpu = None
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        t0 = time.time()
        reps = 0
        while time.time() - t0 < args.cpu_seconds or reps == 0:
            O.backward(wl, dyh, fwd)
            reps += 1
        el = time.time() - t0
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": round(reps * m / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} oracle backward passes of the {m}-token batch ({el:.1f} s)"}
    out = {
        "metric": "sparse-FFN backward tokens/sec (dx + fp32 weight gradients), one layer (1 GPU)",
        "value": round(m * 1e3 / ms, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 3,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOADS[cid]} m={m} backward", "d_model": d, "d_ff": F, "m": m,
                   "active_pairs": pairs, "active_neurons": n_act, "routed_tokens": int(fwd["n_dense"]),
                   "layers_rotated": nl},
        "forward_ms_per_step": round(ms_fwd, 5),
        # per step: from 512 bf16 tokens the dx role is four launches (two
        # weight transposes, the (du | dz) rows, the matrix-core GEMM)
        "kernels_us": {k: round(v["step_us"], 3) for k, v in kernels.items()},
        "launches_per_step": {k: round(v["launches"] / steps, 2) for k, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out))


def bench_moe(args, dev):
    """A mixture-of-experts layer of 8 LoPA-gated experts of the LoPA shape
    (d = 4096, d_ff = 14336, rank 512, 90% sparsity), top-2 routing: a step is
    one layer call over the batch (gather, the chosen experts' sparse forward
    passes, weighted combination); the baseline runs the same layer with the
    experts' dense forward passes. Steps rotate over `--layers` copies of the
    expert set and four routed batches, so the touched weights do not stay in
    the last-level cache."""
    import numpy as np
    import torch

    import activation_sparse_gated_amd as asg
    from synth.moe import make_moe_config

    m = args.m if args.m is not None else 1
    nb = 4
    t_gen = time.time()
    mw = make_moe_config("moe", m=m * nb, seed=0)
    t_gen = time.time() - t_gen
    note(f"inputs moe m={m} x {nb} batches generated in {t_gen:.1f}s")
    e0 = mw.experts[0]

    def dev_bf16(a):
        return torch.from_numpy(e0.storage(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = [{k: dev_bf16(getattr(wl, k)) for k in ("u", "v", "w_up", "w_down")} for wl in mw.experts]
    n_sets = max(1, min(args.layers, 3))
    sets = []
    for li in range(n_sets):
        ffns = []
        for e, wl in enumerate(mw.experts):
            w = {k: (v if li == 0 else v.clone()) for k, v in base[e].items()}
            ffns.append(asg.SparseFFN(d_model=wl.d, d_ff=wl.f, rank=wl.rank, dtype="bf16", act=wl.act, sel=wl.sel,
                                      tile_w=wl.T, ell_w=wl.E, max_m=m, u=w["u"], v=w["v"], w_up=w["w_up"],
                                      w_down=w["w_down"], wdown_out_major=True))
        sets.append(ffns)
    x_all = dev_bf16(mw.x)
    tau_all = torch.from_numpy(mw.tau.astype(np.float32)).to(dev)
    batches = [(x_all[b * m:(b + 1) * m], mw.expert_ids[b * m:(b + 1) * m].copy(),
                mw.weights[b * m:(b + 1) * m].copy(), tau_all[b * m:(b + 1) * m].contiguous()) for b in range(nb)]
    lib = asg.load()
    import ctypes
    wsb = lib.ffn_sparse_moe_workspace_bytes(ctypes.byref(sets[0][0].cfg), m, mw.topk)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    y = torch.empty((m, mw.d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    combos = [(li, b) for li in range(n_sets) for b in range(nb)]

    def step(i, dense=False):
        li, b = combos[i % len(combos)]
        xb, ids, wts, tb = batches[b]
        asg.moe_forward(sets[li], xb, ids, wts, tau=tb, y=y, workspace=ws, dense=dense)

    if args.profile_steps:
        for i in range(args.profile_steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": f"{WORKLOADS['moe']} m={m}"}))
        return

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(warm + i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms = timed(step, args.steps, args.warmup)
    note(f"moe step {ms * 1e3:.2f} us")
    ms_dense = timed(lambda i: step(i, dense=True), max(20, args.steps // 4), 5)
    note(f"dense moe step {ms_dense * 1e3:.2f} us")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    dist = {"p10": round(float(np.percentile(us, 10)), 3), "p50": round(float(np.median(us)), 3),
            "p90": round(float(np.percentile(us, 90)), 3), "steps": args.steps}

    # per-kernel durations of the experts' kernels (HIP events on the stream)
    for ffns in sets:
        for f in ffns:
            f.timing_enable(True, capacity=2 * args.steps + 8)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kernels = {}
    for kind in ("lowrank_v", "gate", "up", "updown", "reduce", "fallback"):
        n_tot, ms_tot = 0, 0.0
        for ffns in sets:
            for f in ffns:
                n, t = f.timing_read(kind)
                n_tot += n
                ms_tot += t
        if n_tot:
            kernels[kind] = {"launches": n_tot, "avg_us": 1e3 * ms_tot / n_tot}
    for ffns in sets:
        for f in ffns:
            f.timing_enable(False)
    d, F, r, T, E = e0.d, e0.f, e0.rank, e0.T, e0.E
    k_act = e0.k
    pairs = m * mw.topk
    # touched bytes per step: each active expert's gate (U, V) once, its tokens'
    # active up and down rows (union per expert), x gathered, y combined
    ids0 = batches[0][1]
    active_experts = len(set(ids0.ravel().tolist()))
    touched = active_experts * (F * r + r * d) * 2 + pairs * k_act * 2 * d * 2 + 3 * pairs * d * 2 + m * d * 2
    dense_bytes = active_experts * ((F * r + r * d) * 2 + 2 * F * d * 2) + 3 * pairs * d * 2 + m * d * 2
    roofline = None
    if m == 1 and "gate" in kernels:
        ntiles = F // T
        pack_bytes = ntiles * (4 + E * 4)
        alg = F * r * 2 + r * 4 + pack_bytes + 9 + 2 * k_act * d * 2      # partial-row gate kernel of one expert
        achieved = alg / (kernels["gate"]["avg_us"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": "gate", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "alg_bytes_per_launch": int(alg), "avg_us": round(kernels["gate"]["avg_us"], 3)}
    cpu = None
    if not args.no_cpu:
        from oracle import ffn_oracle as O
        from threadpoolctl import threadpool_info
        t0 = time.time()
        reps = 0
        while time.time() - t0 < args.cpu_seconds or reps == 0:
            O.moe_forward(mw)
            reps += 1
        el = time.time() - t0
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": round(reps * mw.m / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} oracle passes of the layer over {mw.m} tokens ({el:.1f} s)"}
    out = {
        "metric": "MoE layer (8 LoPA-gated experts, top-2) tokens/sec + effective HBM GB/s, d=4096 (1 GPU)",
        "value": round(m * 1e3 / ms, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOADS['moe']} m={m}", "experts": mw.n_experts, "topk": mw.topk,
                   "d_model": d, "d_ff": F, "rank": r, "m": m, "active_experts_batch0": active_experts,
                   "expert_sets_rotated": n_sets, "batches_rotated": nb},
        # one token: exact; several: rows shared by an expert's tokens are
        # counted once per token (an upper bound)
        "effective_hbm_GBps": round(touched / (ms * 1e-3) / 1e9, 1) if m == 1 else None,
        "touched_bytes": int(touched) if m == 1 else None,
        "touched_bytes_upper": int(touched),
        "dense_ms_per_step": round(ms_dense, 5),
        "dense_effective_hbm_GBps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(ms_dense / ms, 3),
        "step_us_dist": dist,
        "kernels_us": {kk: round(v["avg_us"], 3) for kk, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out))


def bench_gsi(args, dev):
    """The gated subspace linear map ("Gated Subspace Inference for
    Transformer Acceleration", sections 2.1-2.2) on the LoPA FFN's up
    projection, d = 4096 -> 14336, k = 256, eps = 0.10: a step is one gated
    forward call over the batch (projection, residual gate, image or full
    product); the baseline is y = W x on the same tokens."""
    import numpy as np
    import torch

    import activation_sparse_gated_amd as asg
    from synth.gsi import make_gsi_config

    m = args.m if args.m is not None else 1
    t_gen = time.time()
    wl = make_gsi_config("gsi", m=m, seed=0)
    t_gen = time.time() - t_gen
    note(f"inputs gsi m={m} generated in {t_gen:.1f}s")

    def dev_bf16(a):
        from synth import bf16_bits
        return torch.from_numpy(bf16_bits(np.ascontiguousarray(a)).view(np.int16)).view(torch.bfloat16).to(dev)

    w0, v0 = dev_bf16(wl.w), dev_bf16(wl.vk)
    x = dev_bf16(wl.x)
    layers = []
    for _ in range(args.layers):
        lin = asg.GsiLinear(w0.clone(), v0.clone(), max_m=m)
        bufs = (lin.new_output(m), torch.empty(max(m, 1), dtype=torch.float32, device=dev),
                torch.empty(max(m, 1), dtype=torch.int32, device=dev), torch.empty(4, dtype=torch.int32, device=dev),
                lin.new_output(m))
        layers.append((lin, bufs))
    torch.cuda.synchronize()

    def step(i):
        lin, (y, rho, sl, ns, _) = layers[i % len(layers)]
        lin.forward(x, wl.eps, y=y, rho=rho, slow_list=sl, n_slow=ns)

    def dense_step(i):
        lin, (_, _, _, _, yd) = layers[i % len(layers)]
        lin.dense_forward(x, y=yd)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(warm + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    if args.profile_steps:
        for i in range(args.profile_steps):
            step(i)
        torch.cuda.synchronize()
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": f"{WORKLOADS['gsi']} m={m}",
                          "copy_bytes": src.numel()}))
        return

    ms = timed(step, args.steps, args.warmup)
    note(f"gsi step {ms * 1e3:.2f} us")
    ms_dense = timed(dense_step, max(20, args.steps // 4), 5)
    note(f"dense step {ms_dense * 1e3:.2f} us")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    dist = {"p10": round(float(np.percentile(us, 10)), 3), "p50": round(float(np.median(us)), 3),
            "p90": round(float(np.percentile(us, 90)), 3), "steps": args.steps}

    lin0, (y0, rho0, sl0, ns0, _) = layers[0]
    step(0)
    torch.cuda.synchronize()
    n_slow = int(ns0[0])
    d, dout, k = wl.d, wl.d_out, wl.k
    alg = {
        "proj": k * d * 2 + m * d * 2 + m * k * 4,
        "resid": d * k * 2 + m * d * 2 + m * k * 4,
        "out": (dout * k * 2 if n_slow < m else 0) + (dout * d * 2 + m * d * 2 if n_slow else 0)
        + m * k * 4 + m * dout * 2,
    }
    touched = 2 * k * d * 2 + (dout * k * 2 if n_slow < m else 0) + (dout * d * 2 if n_slow else 0) \
        + m * d * 2 + m * dout * 2
    dense_bytes = dout * d * 2 + m * d * 2 + m * dout * 2

    for lin, _ in layers:
        lin.timing_enable(True, capacity=args.steps + 8)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kernels = {}
    for kind in ("proj", "resid", "out"):
        n_tot, ms_tot = 0, 0.0
        for lin, _ in layers:
            n, t = lin.timing_read(kind)
            n_tot += n
            ms_tot += t
        if n_tot:
            kernels[kind] = {"launches": n_tot, "avg_us": 1e3 * ms_tot / n_tot}
    for lin, _ in layers:
        lin.timing_enable(False)
    dom = max(kernels, key=lambda kk: kernels[kk]["avg_us"])
    achieved = alg[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tinfo = json.load(fh).get(f"gsi-m{m}", {}).get(dom)
        if tinfo and tinfo.get("source_sha") == src_hash():
            traffic = tinfo.get("bytes_per_launch")
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": int(alg[dom]), "avg_us": round(kernels[dom]["avg_us"], 3)}

    cpu = None
    if not args.no_cpu:
        from oracle import gsi_oracle as G
        from threadpoolctl import threadpool_info
        from synth import round_bf16
        img = round_bf16(G.image(wl.w, wl.vk))          # the cached image: set-up, not timed
        t0 = time.time()
        reps = 0
        while time.time() - t0 < args.cpu_seconds or reps == 0:
            G.forward(wl.w, img, wl.vk, wl.x, wl.eps)
            reps += 1
        el = time.time() - t0
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": round(reps * m / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} oracle gated forward passes of the {m}-token batch ({el:.1f} s), image precomputed"}

    out = {
        "metric": "gated-subspace linear tokens/sec + effective HBM GB/s, d=4096 -> 14336, k=256 (1 GPU)",
        "value": round(m * 1e3 / ms, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOADS['gsi']} m={m}", "d_in": d, "d_out": dout, "k": k, "m": m,
                   "eps": wl.eps, "slow_tokens": n_slow, "layers_rotated": len(layers)},
        "effective_hbm_GBps": round(touched / (ms * 1e-3) / 1e9, 1),
        "touched_bytes": int(touched),
        "weight_read_reduction": round(dense_bytes / touched, 2),
        "dense_ms_per_step": round(ms_dense, 5),
        "dense_effective_hbm_GBps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(ms_dense / ms, 3),
        "step_us_dist": dist,
        "kernels_us": {kk: round(v["avg_us"], 3) for kk, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
