"""Benchmark of the MI355X Muon step (one GPU).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload owner] [--mode bf16]
                    [--variant step|grouped|graph|master|phases|noalloc]

One "step" is one whole ``muon_step`` call (momentum + Nesterov input,
Frobenius normalization, 5 Newton-Schulz iterations, decay + apply) over the
workload's matrices, with every input already resident in HBM.  The default
workload is one GPU's owner share of a 32-layer, 4096-hidden model: 32 copies
of a Llama-style decoder layer's matrices (Wq 4096x4096, Wk/Wv 1024x4096,
Wo 4096x4096, gate/up 14336x4096, down 4096x14336), 224 matrices in flat
buffers, descriptors in a seeded random order, every update scattered into 8
shard slices; bfloat16 weights, float32 gradients and momentum, synthetic
seeded values.  The single layer's figures are reported next to it.

Variants (same workload): ``grouped`` runs muon_step_grouped with two optimizer
groups (attention and MLP matrices, different lr / weight decay / beta) read
from a device table; ``graph`` captures that grouped step in a HIP graph and
times graph replays; ``master`` keeps float32 master weights and refreshes a
bfloat16 model copy in the same step; ``phases`` runs the step as its three
separate entry points (muon_momentum, muon_orthogonalize, muon_apply), which
times the standalone momentum and apply kernels; ``noalloc`` runs
muon_step_noalloc (intermediates in the library's fixed per-GPU scratch array,
matrices in waves that fit it).

Prints one JSON line: matrices/s for the whole step, the Newton-Schulz
algorithmic TFLOP/s and its fraction of the bf16 dense MFMA peak (with the
dense-equivalent rate, counting full products, beside it), the roofline
of the dominant kernel (per-launch durations from HIP events recorded on the
launch stream during the timed region), and the CPU oracle timed on a bounded
sample of the same workload (for the owner share: of one layer, times 32).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wlm  # noqa: E402

METRIC = "Muon step matrices/s; Newton-Schulz TFLOPS as % of bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0


def ns_flops(r, c):
    """Algorithmic flops of one iteration, by stage (triangles for the symmetric ones)."""
    return {"a": r * (r + 1) * c, "b": r * r * (r + 1), "x": 2 * r * r * c}


def stage_flops(wl, ns_steps):
    tot = {"a": 0, "b": 0, "x": 0}
    for d in wl.descs:
        r, c = min(d.rows, d.cols), max(d.rows, d.cols)
        for k, v in ns_flops(r, c).items():
            tot[k] += v
    return tot  # per iteration (one launch per stage and tile size)


def dense_flops(wl):
    """Flops of one iteration counted as dense products (full A, A^2 and B X):
    4 r^2 c + 2 r^3 per matrix, reported beside the algorithmic count."""
    return sum(4 * r * r * c + 2 * r ** 3
               for r, c in ((min(d.rows, d.cols), max(d.rows, d.cols)) for d in wl.descs))


def elementwise_bytes(wl, mode):
    """Bytes each elementwise kernel must move, per step (per launch)."""
    n = wl.numel()
    wb = 2 if wl.param_dtype == "bf16" else 4
    xb = 2 if mode == "bf16" else 4
    return {"front_cast": 12 * n + xb * n,  # G, M read; M written; first iterate written
            "front": 16 * n,                # G read, M read + write, U write (float32)
            "cast": 4 * n + xb * n,         # U read, X0 written
            "sumsq_cast": 4 * n + xb * n,   # U read, first iterate written (muon_orthogonalize)
            "apply": 4 * n + 2 * wb * n}    # O read, W read + write


def kernel_source(kernel):
    """The source file that holds a kernel of the profile table."""
    if kernel.startswith("ns_"):
        return "k_ns_gemm.hip"
    if kernel in ("front", "apply", "sumsq"):
        return "k_elementwise.hip"
    return "k_norm_cast.hip"  # front_cast, sumsq_cast, norm, cast


def recorded_traffic(kernel, workload):
    """HBM bytes per launch (read + written) that profiler counters recorded for
    this kernel on this workload, if the kernel's source file is unchanged
    since; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    try:
        rec = json.load(open(path))
        f = kernel_source(kernel)
        src = os.path.join(ROOT, "newton_schulz_flat_amd", "csrc", f)
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["sources_sha256"][f]:
            return None
        b = rec["per_launch_bytes"][kernel]
        return b["read"] + b["written"]
    except (OSError, KeyError, ValueError):
        return None


def host_info():
    """CPU model, logical CPUs, and the BLAS library NumPy uses (with its threads)."""
    info = {"nproc": os.cpu_count() or 1, "cpu_model": "unknown", "blas": "unknown",
            "blas_threads": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        if blas:
            b = blas[0]
            info["blas"] = (f"{b.get('internal_api')} {b.get('version')} "
                            f"({b.get('threading_layer')}, {b.get('architecture')})")
            info["blas_threads"] = int(b.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return info


def _oracle_sample(wl, order, budget_s):
    """Oracle step times of wl's matrices in the given order until budget_s/2 is
    spent; returns (seconds, NS flops of the sample, labels)."""
    import numpy as np
    from oracle import muon_oracle as mo
    h = wlm.HYPER
    spent, sample_flops, picked = 0.0, 0.0, []
    for i in order:
        d = wl.descs[i]
        r, c = min(d.rows, d.cols), max(d.rows, d.cols)
        rng = np.random.default_rng([wlm.seed_of(wl.name, i, 0)])
        w = rng.standard_normal((d.rows, d.cols)) * wl.w_std
        g = rng.standard_normal((d.rows, d.cols)) * wl.g_std
        m = np.zeros_like(g)
        t0 = time.perf_counter()
        mo.step_matrix(w, g, m, lr=mo.as_f32_value(h["lr"]),
                       weight_decay=mo.as_f32_value(h["weight_decay"]),
                       beta=mo.as_f32_value(h["beta"]), nesterov=True, ns_steps=h["ns_steps"])
        spent += time.perf_counter() - t0
        sample_flops += sum(ns_flops(r, c).values()) * h["ns_steps"]
        picked.append(f"{wl.names[i]} {d.rows}x{d.cols}")
        if spent > budget_s / 2:
            break
    return spent, sample_flops, picked


def cpu_baseline(wl, budget_s=20.0):
    """The fp64 NumPy oracle's step time, on a bounded sample, scaled to the workload.

    The sample is the workload's own smallest matrices, scaled by Newton-Schulz
    flops.  For the owner share (32 copies of the llama layer) the sample is
    taken from the llama layer, scaled to the layer by flops, and the owner
    share's time is 32 times the layer's (extrapolated)."""
    info = host_info()
    h = wlm.HYPER
    base = wlm.make_workload("llama") if wl.name == "owner" else wl
    order = sorted(range(base.n), key=lambda i: base.descs[i].rows * base.descs[i].cols)
    spent, sample_flops, picked = _oracle_sample(base, order, budget_s)
    base_flops = sum(stage_flops(base, h["ns_steps"]).values()) * h["ns_steps"]
    est_base = spent * base_flops / sample_flops
    est = est_base * (wl.n // base.n if wl.name == "owner" else 1)
    out = {"value": wl.n / est, "unit": "matrices/s",
           "cores": info["blas_threads"] or info["nproc"], "kind": "oracle",
           "sample": (f"fp64 NumPy oracle step of {', '.join(picked)} ({spent:.1f} s), "
                      f"scaled by Newton-Schulz flops to all {base.n} matrices of the "
                      f"{'llama layer' if base is not wl else 'workload'}"
                      + (f", times {wl.n // base.n} layers" if base is not wl else "")),
           "seconds_per_step": est, "nproc": info["nproc"], "cpu_model": info["cpu_model"],
           "blas": info["blas"], "extrapolated": True}
    if base is not wl:
        out["llama_layer_seconds_per_step"] = est_base
    return out


def measure(workload, mode, variant, steps, warmup):
    """Runs warmup + steps whole steps of one workload; returns its figures."""
    import dataclasses

    import torch

    import newton_schulz_flat_amd as nsf
    h = wlm.HYPER
    wl = wlm.make_workload(workload)
    if variant == "master":
        wl = dataclasses.replace(wl, param_dtype="f32")
    params, grads, mom = wlm.make_tensors(wl, "cuda:0")
    descs = wl.descs
    if variant in ("grouped", "graph"):
        # attention matrices (q, k, v, o) in group 0, the rest (MLP) in group 1
        descs = [dataclasses.replace(d, group=0 if nm.split(".")[-1] in ("wq", "wk", "wv", "wo")
                                     else 1)
                 for d, nm in zip(wl.descs, wl.names)]
        table = nsf.group_table([(h["lr"], h["weight_decay"], h["beta"], True),
                                 (0.5 * h["lr"], 0.1, 0.9, True)], "cuda:0")
    elif variant == "master":
        table = nsf.group_table([(h["lr"], h["weight_decay"], h["beta"], True)], "cuda:0")
        model_copy = params.to(torch.bfloat16)
    elif variant == "phases":
        u = torch.empty_like(grads)
        o = torch.empty_like(grads)
    ws = torch.empty(0 if variant == "noalloc" else nsf.muon_workspace_bytes(descs, mode),
                     dtype=torch.uint8, device="cuda:0")

    def eager():
        if variant == "step":
            nsf.muon_step(params, grads, mom, descs, h["lr"], h["weight_decay"], h["beta"],
                          nesterov=h["nesterov"], ns_steps=h["ns_steps"], mode=mode, workspace=ws)
        elif variant == "noalloc":
            nsf.muon_step_noalloc(params, grads, mom, descs, h["lr"], h["weight_decay"],
                                  h["beta"], nesterov=h["nesterov"], ns_steps=h["ns_steps"],
                                  mode=mode)
        elif variant == "phases":
            nsf.muon_momentum(grads, mom, u, descs, h["beta"], h["nesterov"])
            nsf.muon_orthogonalize(u, o, descs, ns_steps=h["ns_steps"], mode=mode, workspace=ws)
            nsf.muon_apply(params, o, descs, h["lr"], h["weight_decay"])
        else:
            nsf.muon_step_grouped(params, grads, mom, descs, table, ns_steps=h["ns_steps"],
                                  mode=mode, workspace=ws,
                                  model_copy=model_copy if variant == "master" else None)

    step = eager
    if variant == "graph":
        eager()  # builds the plan outside capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager()
        torch.cuda.synchronize()
        step = graph.replay

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nsf.muon_profile_begin()   # replays of a graph are not bracketed: no kernel table
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    kernels = nsf.muon_profile_end()
    ms = ev0.elapsed_time(ev1) / steps

    fl = stage_flops(wl, h["ns_steps"])
    ns_alg = sum(fl.values()) * h["ns_steps"]
    ew = elementwise_bytes(wl, mode)
    ns_ms, ns_tflops, ns_dense, roof, per_kernel = None, None, None, None, {}
    if kernels:  # eager launches (graph replays carry no per-kernel events)
        ns_ms = sum(v[0] for k, v in kernels.items() if k.startswith("ns_")) / steps
        ns_tflops = ns_alg / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
        ns_dense = dense_flops(wl) * h["ns_steps"] / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
        # dominant kernel = largest total time; its algorithmic work per launch
        name, (tot_ms, launches) = max(kernels.items(), key=lambda kv: kv[1][0])
        avg_s = tot_ms / launches * 1e-3
        if name.startswith("ns_"):
            stage = name.split("_")[1]
            same = [k for k in kernels if k.startswith(f"ns_{stage}_")]
            if len(same) == 1:
                work = fl[stage]
            else:  # several tile sizes: attribute this stage's flops by measured time share
                work = fl[stage] * tot_ms / sum(kernels[k][0] for k in same)
            roof = {"kernel": name, "bound": "mfma", "achieved": work / avg_s / 1e12,
                    "peak": PEAK_TFLOPS[mode], "unit": "TFLOP/s",
                    "work_per_launch": work, "avg_launch_ms": avg_s * 1e3}
        else:
            work = ew.get(name, 0)
            roof = {"kernel": name, "bound": "hbm", "achieved": work / avg_s / 1e9,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "work_per_launch": work,
                    "avg_launch_ms": avg_s * 1e3}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = recorded_traffic(name, PROFILE_NAMES.get(wl.name, wl.name)) \
            if variant == "step" else None
        per_kernel = {k: {"ms_per_step": v[0] / steps, "launches_per_step": v[1] / steps}
                      for k, v in sorted(kernels.items())}
        for k in ("front_cast", "front", "cast", "sumsq_cast", "apply"):
            if k in kernels:
                per_kernel[k]["GB/s"] = ew[k] / (kernels[k][0] / kernels[k][1] * 1e-3) / 1e9
                per_kernel[k]["frac_hbm"] = per_kernel[k]["GB/s"] / PEAK_HBM_GBS
    del params, grads, mom, ws
    if variant == "phases":
        del u, o
    torch.cuda.empty_cache()
    return {"wl": wl, "ms": ms, "value": wl.n * 1e3 / ms, "ns_tflops": ns_tflops,
            "ns_dense_equivalent_tflops": ns_dense, "ns_ms": ns_ms, "roofline": roof,
            "kernels": per_kernel}


#: profiles/<name>_traffic.json of each workload
PROFILE_NAMES = {"llama": "llama_layer", "owner": "owner_share", "moe": "moe_set",
                 "batched": "batched_512"}
#: the workload names used in the JSON line
CONFIG_NAMES = {"llama": "llama-layer", "owner": "owner-share-32-layers", "moe": "moe-set",
                "batched": "batched-512", "single": "single-256x512"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="owner", choices=wlm.WORKLOADS)
    ap.add_argument("--mode", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--variant", default="step",
                    choices=["step", "grouped", "graph", "master", "phases", "noalloc"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-llama", action="store_true",
                    help="skip the extra llama-layer figures reported next to the owner share")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates the "
                         "HBM byte counters of a profiler run) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the Muon step here runs on one GPU; the multi-GPU owner-compute "
              "path (exchanges of update slices between ranks) is not implemented, so "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n}))
        return

    import newton_schulz_flat_amd as nsf
    if not os.path.exists(nsf.LIB_PATH):
        from newton_schulz_flat_amd import build
        build.build()
    nsf.load_library()
    torch.cuda.set_device(0)

    h = wlm.HYPER
    r = measure(args.workload, args.mode, args.variant, args.steps, args.warmup)
    wl = r["wl"]
    out = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mode == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES.get(wl.name, wl.name),
                   "matrices": wl.n, "elements": wl.numel(), "param_dtype": wl.param_dtype,
                   "gemm_mode": args.mode, "ns_steps": h["ns_steps"], "lr": h["lr"],
                   "weight_decay": h["weight_decay"], "beta": h["beta"], "nesterov": True,
                   "parallelism": "single-gpu", "variant": args.variant},
        "ns_tflops": r["ns_tflops"],
        "ns_frac_of_peak": None if r["ns_tflops"] is None
        else r["ns_tflops"] / PEAK_TFLOPS[args.mode],
        "ns_ms_per_step": r["ns_ms"],
        "ns_dense_equivalent_tflops": r["ns_dense_equivalent_tflops"],
        "roofline": r["roofline"],
        "kernels": r["kernels"],
    }
    if wl.name == "owner" and not args.no_llama:
        # one decoder layer (the owner share's building block) on its own
        lr_ = measure("llama", args.mode, args.variant, args.steps, args.warmup)
        out["llama_layer"] = {
            "value": lr_["value"], "unit": "matrices/s", "ms_per_step": lr_["ms"],
            "ns_tflops": lr_["ns_tflops"],
            "ns_frac_of_peak": None if lr_["ns_tflops"] is None
            else lr_["ns_tflops"] / PEAK_TFLOPS[args.mode],
            "roofline": lr_["roofline"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
