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
WORKLOADS = {
    "c2": "decode-relu-bf16-2048x8192",
    "c3": "lopa-relu-thresh-bf16-4096x14336-r512",
    "c4": "wina-silu-topk-bf16-4096x11008",
    "c5": "prefill-hybrid-relu-bf16-2048x8192",
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
    m = args.m if args.m is not None else {"c2": 1, "c3": 1, "c4": 1, "c5": 4096}[cid]
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
                            w_up=w["w_up"], w_down=w["w_down"], wdown_out_major=True)
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

    # ---- timed region: the sparse forward pass (value) ----
    ms_sparse, steps = timed(sparse_step, args.steps, args.warmup, graph=args.graph)
    note(f"sparse step {ms_sparse * 1e3:.2f} us")
    ms_dense, _ = timed(dense_step, max(20, args.steps // 4), 5, graph=args.graph)
    note(f"dense step {ms_dense * 1e3:.2f} us")

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
    elif path == "topk-masked-dense":
        alg["updown"] = F * d * 2 + m * F * 2 + m * d * 2      # all of W_down, the masked h rows, y
    if wl.sel == "topk":
        alg["gate"] = 2 * F * d * 2 + m * d * 2 + 2 * m * F * 4
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

    # ---- CPU oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu:
        from oracle import ffn_oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count() or 1
        t0 = time.time()
        reps = 0
        while time.time() - t0 < args.cpu_seconds or reps == 0:
            O.forward(wl)
            reps += 1
        el = time.time() - t0
        cpu = {"value": round(reps * m / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} full oracle forward passes of the {m}-token batch ({el:.1f} s)"}

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
        "touched_bytes": int(touched),
        "dense_ms_per_step": round(ms_dense, 5),
        "dense_effective_hbm_GBps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(ms_dense / ms_sparse, 3),
        "kernels_us": {k: round(v["avg_us"], 3) for k, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
