"""Benchmark: fused linear-cross-entropy forward + backward on one MI355X.

A step is one pass of the whole hot path over one batch: valid-token
compaction, forward (projection tiles + online LSE + merge + loss) and
backward (replay -> G, dH and dW GEMMs, db, finalize), on seeded synthetic
inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload packed] [--no-cpu-baseline]

Prints ONE JSON line.  Only one GPU is supported (--gpus N>1 exits).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s and TFLOP/s (% of bf16 MFMA peak)"
METRIC_FWD = "fused linear-CE forward-only loss tokens/s and TFLOP/s (% of bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix (published)
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=12)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="packed")
    p.add_argument("--mode", choices=("train", "forward", "shard"), default="train",
                   help="train: compaction + forward + backward; forward: compaction + forward-only loss; "
                        "shard: train with the vocabulary split into --shards shards run one after another")
    p.add_argument("--shards", type=int, default=8, help="vocabulary shards for --mode shard")
    p.add_argument("--filter-eps", type=float, default=None,
                   help="train with the gradient filter at this threshold (lce_backward_filtered)")
    p.add_argument("--filter-grads", choices=["dh", "both"], default="both",
                   help="which gradients the filter applies to")
    p.add_argument("--reduction", choices=("mean", "sum", "none"), default="mean",
                   help="mean: plain entries; sum (per-position weights, divisor N) / none: the _ex entries")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run 3 device-to-device copies of BYTES (scales HBM byte counters) and exit")
    return p.parse_args()


def copy_calibration(nbytes: int):
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": a.numel() * 4, "copies": 3}), flush=True)


def git_rev():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


# Algorithmic FLOPs per step (2*C*D*V per GEMM pass: the logits in the
# forward, their replay and the dH and dW products in the backward).  The
# library reports each launch's share; their sum must come to this.
def step_flops(C, D, V, mode="train"):
    return (2.0 if mode == "forward" else 8.0) * C * D * V


def kernel_bytes(C, N, D, V, esz, has_mask, has_bias):
    """Algorithmic HBM bytes per launch of the memory-bound kernels: the
    compaction (labels and mask read, indices written), the row gather, and
    the two finalisations.  The gather also fills per-position arrays, 4 bytes
    a position each: m and log s in the forward call, the inverse row map in
    the backward call (1.5 arrays a launch on average over a training step).
    k_dh_finalize reads at least one fp32 partial per supervised element (more
    when the library splits dH over several slots), so its figure is a lower
    bound."""
    cpad = -(-C // 256) * 256
    per_pos = 8 + (1 if has_mask else 0)
    out = {"k_cmp_one": N * per_pos + 4 * C, "k_cmp_count": N * per_pos, "k_cmp_scatter": N * per_pos + 4 * C,
           "k_gather": C * D * esz + cpad * D * esz + 6 * N,
           "k_dh_finalize": C * D * 4 + N * D * esz}
    if has_bias:
        out["k_db_finalize"] = (cpad // 256) * (-(-V // 256) * 256) * 4 + V * esz
    return out


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, from the committed
    counter profile profiles/<kernel>_<workload>_hbm_traffic.md, or None when
    there is none or the library sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    from lm_head_projection_amd.build import source_digest
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`")
            for key in ("source_sha256", "fetch_bytes_per_launch", "write_bytes_per_launch"):
                if line.startswith(key + ":"):
                    vals[key] = line.split(":", 1)[1].strip()
    if len(vals) != 3 or vals["source_sha256"] != source_digest():
        return None
    return {"fetch_bytes_per_launch": float(vals["fetch_bytes_per_launch"]),
            "write_bytes_per_launch": float(vals["write_bytes_per_launch"]),
            "path": os.path.relpath(path, ROOT)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_vendor():
    """The BLAS library NumPy calls (name, version, threads), as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"library": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "path": os.path.basename(i.get("filepath", ""))}
    except Exception:
        pass
    return None


def library_record():
    """Which HIP library ran: its path (relative to the repository), the
    SHA-256 of the file and of the sources it is built from."""
    from lm_head_projection_amd import _lib
    from lm_head_projection_amd.build import file_digest, source_digest
    return {"path": os.path.relpath(_lib.LIB_PATH, ROOT), "sha256": file_digest(_lib.LIB_PATH),
            "source_sha256": source_digest()}


def cpu_baseline(wl, target_s: float, forward_only: bool = False):
    """The oracle as it stands, on a bounded sample of supervised rows."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    import oracle as O
    H = wl.H.double().numpy()
    W = wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    y = wl.labels.numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    _, idx, C = O.supervised_rows(y, mask, wl.ignore_index)

    def run(rows):
        sel = idx[:rows]
        t0 = time.perf_counter()
        if forward_only:
            O.dense_forward(H[sel], W, b, y[sel], None, wl.ignore_index)
        else:
            O.dense_forward_backward(H[sel], W, b, y[sel], None, 1.0, wl.ignore_index)
        return time.perf_counter() - t0

    n = 16
    t = run(n)
    while t < 1.0 and n < C:
        n = min(C, n * 4)
        t = run(n)
    n2 = int(min(C, max(n, n * target_s / max(t, 1e-6))))
    if n2 > n:
        n, t = n2, run(n2)
    return {"value": n / t, "unit": "supervised tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "blas": blas_vendor(), "numpy": np.__version__,
            "sample": f"{n} of {C} supervised rows of the {wl.name} workload (full D={wl.D}, V={wl.V}); "
                      f"float64 NumPy dense {'forward' if forward_only else 'forward+backward'}, {t:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path; how it would shard is described in the design notes.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    from lm_head_projection_amd import _lib
    from lm_head_projection_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load()
    dev = "cuda:0"
    t0 = time.time()
    wl = WL.make_workload(args.workload)
    log(f"[bench] workload {args.workload}: N={wl.N} D={wl.D} V={wl.V} {wl.dtype} ({time.time() - t0:.1f}s)")
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    dH = torch.empty_like(H)
    dW = torch.empty_like(W)
    db = None if b is None else torch.empty_like(b)
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    # The backward's arrays take the supervised rows only: size the one
    # workspace that every call of the step shares for this workload's count.
    sup = wl.labels != wl.ignore_index
    if wl.mask is not None:
        sup &= wl.mask.bool()
    ws = torch.empty(_lib.lce_backward_workspace_size(N, int(sup.sum()), D, V, H.dtype), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    m = torch.empty(N, dtype=torch.float32, device=dev)
    logs = torch.empty(N, dtype=torch.float32, device=dev)
    grad = torch.ones(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    red = _lib.REDUCTIONS[args.reduction]
    weights, num = None, 0.0
    if args.reduction == "sum":
        gen = torch.Generator().manual_seed(77)
        weights = torch.rand(N, generator=gen).to(dev)
        num = float(N)
    if args.reduction == "none":
        loss = torch.empty(N, dtype=torch.float32, device=dev)
        gen = torch.Generator().manual_seed(78)
        grad = torch.randn(N, generator=gen).to(dev)
    plain = args.reduction == "mean"
    train = args.mode in ("train", "shard")
    if args.mode == "shard":
        P = args.shards
        bounds = [V * p // P for p in range(P + 1)]
        parts = torch.empty(P * 3 * N, dtype=torch.float32, device=dev)  # [P][3*C] for C <= N
        dH_parts = [torch.empty_like(H) for _ in range(P)]
        g1 = grad if args.reduction == "none" else grad.reshape(1)

        def step(mark=None):
            st, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws, stream)
            assert st == _lib.LCE_OK, _lib.status_string(st)
            for p in range(P):
                v0, v1 = bounds[p], bounds[p + 1]
                st = _lib.lce_forward_shard(H, W[v0:v1], None if b is None else b[v0:v1], labels, idx, C, v0,
                                            parts[p * 3 * C:(p + 1) * 3 * C], ws, stream)
                assert st == _lib.LCE_OK, _lib.status_string(st)
            pc = parts[: P * 3 * C].view(P, 3 * C)
            st = _lib.lce_merge_shards(pc, bounds, labels, idx, C, red, weights, num, loss, m, logs, ws, stream)
            assert st == _lib.LCE_OK, _lib.status_string(st)
            if mark is not None:
                mark()
            for p in range(P):
                v0, v1 = bounds[p], bounds[p + 1]
                st = _lib.lce_backward_shard(H, W[v0:v1], None if b is None else b[v0:v1], labels, idx, C, v0, red,
                                             weights, num, m, logs, g1, dH_parts[p], dW[v0:v1],
                                             None if db is None else db[v0:v1], ws, stream)
                assert st == _lib.LCE_OK, _lib.status_string(st)
            return C

    def step_single(mark=None):
        st, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws, stream)
        assert st == _lib.LCE_OK, _lib.status_string(st)
        if plain and train:
            st = _lib.lce_forward(H, W, b, labels, idx, C, loss, m, logs, None, ws, stream)
        else:  # the _ex entry; forward-only runs without saved statistics
            st = _lib.lce_forward_ex(H, W, b, labels, idx, C, red, weights, num, loss,
                                     m if train else None, logs if train else None, ws, stream)
        assert st == _lib.LCE_OK, _lib.status_string(st)
        if not train:
            return C
        if mark is not None:
            mark()
        if args.filter_eps is not None:
            st = _lib.lce_backward_filtered(H, W, b, labels, idx, C, red, weights, num, m, logs, grad,
                                            args.filter_eps, dH, dW, db, ws, stream,
                                            which={"dh": 1, "both": 3}[args.filter_grads])
        elif plain:
            st = _lib.lce_backward(H, W, b, labels, idx, C, m, logs, grad, dH, dW, db, ws, stream)
        else:
            st = _lib.lce_backward_ex(H, W, b, labels, idx, C, red, weights, num, m, logs, grad, dH, dW, db,
                                      ws, stream)
        assert st == _lib.LCE_OK, _lib.status_string(st)
        return C

    if args.mode != "shard":
        step = step_single

    # HIP events on the stream, one between every two timed steps (per-step
    # times for the median).  They are made before the warm-up, and the
    # output check waits until after the timed region: host work between the
    # warm-up and the timed steps leaves the GPU idle, and after an idle gap
    # its clock needs one packed step (several short ones) to recover.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.warmup):
        C = step()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    if not train:
        log("[bench] forward-only: compaction + forward, no saved statistics")

    # Timed region: K steps bracketed by synchronisation.
    torch.cuda.synchronize()
    evs[0].record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        C = step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = evs[0].elapsed_time(evs[-1])
    ms = total_ms / args.steps
    in_order = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    per_step = sorted(in_order)
    step_ms = {"mean": ms, "median": statistics.median(per_step), "min": per_step[0], "max": per_step[-1],
               "in_order": [round(t, 4) for t in in_order]}
    assert torch.isfinite(loss).all()
    peak_extra = torch.cuda.max_memory_allocated() - base_alloc
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step (median {step_ms['median']:.3f}, min {step_ms['min']:.3f}, "
        f"max {step_ms['max']:.3f}; wall {wall * 1e3 / args.steps:.3f} ms/step), C={C}")

    # Per-kernel durations: the same K steps again, with the library recording
    # a HIP event pair around each of its launches on the launch stream.
    _lib.profile_start(65536)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = _lib.profile_stop()
    log(f"[bench] per-kernel pass done ({sum(v[0] for v in kern.values()) / args.steps:.3f} ms/step in kernels)")

    # Forward (compaction included) and backward apart: the same K steps once
    # more, with one more event between the two on the stream.
    phases = None
    if train:
        marks = []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            step(mark=lambda e=e: e[1].record(stream))
            e[2].record(stream)
            marks.append(e)
        torch.cuda.synchronize()
        fwd = sum(e[0].elapsed_time(e[1]) for e in marks) / args.steps
        bwd = sum(e[1].elapsed_time(e[2]) for e in marks) / args.steps
        phases = {"forward_ms": fwd, "backward_ms": bwd}
        log(f"[bench] phases: forward {fwd:.3f} ms, backward {bwd:.3f} ms per step")

    flops_step = (8.0 if train else 2.0) * C * D * V
    tflops = flops_step / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    lib_flops = sum(v[2] for v in kern.values()) / args.steps
    if abs(lib_flops - step_flops(C, D, V, args.mode)) > 1e-6 * step_flops(C, D, V, args.mode):
        log(f"[bench] warning: the library's per-launch flops sum to {lib_flops:.6g} per step, "
            f"not {step_flops(C, D, V, args.mode):.6g}")
    kb = kernel_bytes(C, N, D, V, 2 if wl.dtype == torch.bfloat16 else 4, mask is not None, b is not None)
    kernels = {}
    for name, (tot, n, fl) in sorted(kern.items(), key=lambda kv: -kv[1][0]):
        e = {"total_ms_per_step": tot / args.steps, "launches_per_step": n / args.steps,
             "avg_ms": tot / max(n, 1)}
        # The filter skips a data-dependent part of the gradient products: no rate for those launches.
        if fl > 0 and not (args.filter_eps is not None and name.startswith("k_grad")):
            e["flops_per_step"] = fl / args.steps
            e["tflops"] = fl / (tot * 1e-3) / 1e12
        if name in kb:
            e["hbm_gbps"] = kb[name] / (e["avg_ms"] * 1e-3) / 1e9
            if name == "k_dh_finalize":
                e["hbm_gbps_lower_bound"] = True
        kernels[name] = e
    dom = max((k for k in kernels if "tflops" in kernels[k]), key=lambda k: kernels[k]["total_ms_per_step"])
    tr = stored_traffic(dom, args.workload)
    rf = {"bound": "mfma", "achieved": kernels[dom]["tflops"], "peak": peak, "unit": "TFLOP/s",
          "frac": kernels[dom]["tflops"] / peak,
          "traffic": None if tr is None else tr["fetch_bytes_per_launch"] + tr["write_bytes_per_launch"],
          "kernel": dom,
          "flops_per_launch": kernels[dom]["flops_per_step"] / kernels[dom]["launches_per_step"],
          "avg_launch_ms": kernels[dom]["avg_ms"],
          "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
          "traffic_source": None if tr is None else tr["path"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample (host cores)")
        cpu = cpu_baseline(wl, args.cpu_seconds, forward_only=not train)
        log(f"[bench] oracle: {cpu['value']:.1f} tok/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC if train else METRIC_FWD,
        "note": (f"{args.shards} vocabulary shards run one after another; the dH sum over shards (an "
                 "all-reduce across devices) is not part of the step") if args.mode == "shard" else
                ("gradient filter on: tflops counts the dense 8*C*D*V (a dense-equivalent rate); k_grad skips "
                 "the products of dropped blocks") if args.filter_eps is not None else None,
        "value": C * args.steps / (total_ms * 1e-3),
        "unit": "supervised tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_ms": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "N": N, "D": D, "V": V, "C": C,
                   "bias": b is not None, "mask": mask is not None, "mode": args.mode,
                   "reduction": args.reduction, "shards": args.shards if args.mode == "shard" else 1,
                   "filter_eps": args.filter_eps,
                   "filter_grads": args.filter_grads if args.filter_eps is not None else None},
        "tflops": tflops,
        "pct_peak": 100.0 * tflops / peak,
        "positions_per_s": N * args.steps / (total_ms * 1e-3),
        "flops_per_step": flops_step,
        "phases": phases,
        "peak_extra_mem_bytes": int(peak_extra),
        "workspace_bytes": int(ws.numel()),
        "dense_logits_bytes_avoided": int(N) * int(V) * (2 if wl.dtype == torch.bfloat16 else 4),
        "roofline": rf,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "library": library_record(),
        "inputs_sha256": wl.sha256(),
        "git": git_rev(),
        "device": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
