"""Benchmark of the batched Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline|c1|c2|c3|c4]
                    [--no-cpu-baseline] [--copy-calibration]

A step is one muon_step_batched call over the whole workload (plus
adamw_step when the workload has AdamW tensors) on inputs already resident in
HBM.  The default workload is 8 independent 4096 x 4096 fp32 weights with
fp32 gradients and momentum, bf16 Newton-Schulz (5 iterations), Moonlight
multiplier.  Prints one JSON line.

Throughput is algorithmic Newton-Schulz TFLOP/s: 5 (3 m'^2 n' + m'^3) flops
per matrix (the Gram and polynomial products are symmetric, so only one
triangle is needed); the dense count 5 (4 m'^2 n' + 2 m'^3) is reported
alongside.  The timed steps run with one event between steps and nothing
else; per-kernel durations come from a second pass of the same number of
steps, with HIP events the library records around each of its launches on
the stream it launches on (those events add their own time to every
launch, so that pass's step time is reported apart, as profiled_ms_per_step).
"""

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (a known-size kernel for counter scaling)")
    return ap.parse_args()


def hbm_roofline(flops, nbytes, avg_ms, peak_tflops, peak_gbs=PEAK_HBM_GBS):
    """The HBM roofline of a launch doing `flops` on `nbytes` of algorithmic
    traffic in avg_ms, if its arithmetic intensity lies below the ridge point
    (peak flop / peak bandwidth); None when the matrix cores bound it."""
    ridge = peak_tflops * 1e12 / (peak_gbs * 1e9)
    if nbytes <= 0 or avg_ms <= 0 or flops / nbytes >= ridge:
        return None
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": peak_gbs, "unit": "GB/s",
            "frac": round(gbs / peak_gbs, 4), "per_launch_bytes": nbytes,
            "arithmetic_intensity": round(flops / nbytes, 1), "ridge": round(ridge, 1)}


def _traffic_record(kernel, root=None):
    """HBM traffic per launch measured with rocprofv3 counters, if the record
    in profiles/ was taken on the current source of the kernel."""
    import hashlib
    root = root or ROOT
    path = os.path.join(root, "profiles", "traffic_%s.md" % kernel)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"^source_sha256:\s*(\w+)", txt, flags=re.M)
    b = re.search(r"^bytes_per_launch:\s*([0-9.eE+]+)", txt, flags=re.M)
    if not m or not b:
        return None
    src = os.path.join(root, "muon_step_02_amd", "csrc", "gemm_bf16.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if h != m.group(1):
        return None
    return float(b.group(1))


def cpu_baseline(wl, budget_s=20.0):
    """The fp64 oracle on the host cores, on a bounded sample of the workload:
    whole matrices of the first step, as many as fit in about budget_s."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    hp = dict(wl.muon_hp)
    kw = dict(lr=hp["lr"], mu=hp["mu"], weight_decay=hp["weight_decay"], nesterov=hp["nesterov"],
              eps=hp["eps"], steps=hp["steps"], scale_mode=hp["scale_mode"])
    done, flops, t_used = 0, 0.0, 0.0
    shapes = wl.muon_shapes()
    for k, v in enumerate(wl.muon):
        W = wl.make_weight(v.tensor, "cpu")[v.row0:v.row0 + v.rows].double().numpy()
        G = wl.make_grad(v.tensor, 1, "cpu")[v.row0:v.row0 + v.rows].double().numpy()
        M = np.zeros_like(W)
        t0 = time.perf_counter()
        oracle.muon_matrix_step(W, G, M, **kw)
        dt = time.perf_counter() - t0
        r, c = shapes[k]
        m, n = min(r, c), max(r, c)
        flops += hp["steps"] * (3 * m * m * n + m ** 3)
        t_used += dt
        done += 1
        if t_used + dt > budget_s:
            break
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d of %d matrices of step 1 (fp64 numpy oracle, %.1f s; BLAS threads %d, "
                      "os.cpu_count() %d)" % (done, len(wl.muon), t_used, threads, os.cpu_count())}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only; --gpus %d is not supported (across GPUs the "
              "Muon step shards by whole matrices, each GPU running the library on its share)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import muon_step_02_amd as mu

    torch.cuda.set_device(0)
    dev = "cuda:0"
    wl = synth.WORKLOADS[args.workload]()
    hpd = wl.muon_hp
    h = mu.muon_init(0)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # inputs resident in HBM
    W = [wl.make_weight(i, dev) for i in range(len(wl.tensors))]
    G = [wl.make_grad(i, 1, dev) for i in range(len(wl.tensors))]
    M = {}
    for v in wl.muon:
        M.setdefault(v.tensor, torch.zeros(wl.tensors[v.tensor].shape, device=dev))
    am = {i: torch.zeros(wl.tensors[i].shape, device=dev) for i in wl.adamw}
    av = {i: torch.zeros(wl.tensors[i].shape, device=dev) for i in wl.adamw}
    mats = []
    for v in wl.muon:
        sl = slice(v.row0, v.row0 + v.rows)
        mats.append(mu.muon_matrix(W[v.tensor][sl], G[v.tensor][sl], M[v.tensor][sl]))
    hp = mu.muon_hparams(lr=hpd["lr"], momentum=hpd["mu"], weight_decay=hpd["weight_decay"],
                         eps=hpd["eps"], nesterov=hpd["nesterov"], ns_steps=hpd["steps"],
                         ns_dtype=hpd["ns_dtype"], scale_mode=hpd["scale_mode"])
    ws = torch.empty(mu.muon_workspace_size(h, mats, hp), dtype=torch.uint8, device=dev)
    ats = [mu.adamw_tensor(W[i], G[i], am[i], av[i]) for i in wl.adamw]
    stream = torch.cuda.current_stream()
    t_counter = [0]

    def step():
        mu.muon_step_batched(h, mats, hp, ws, stream)
        if ats:
            t_counter[0] += 1
            mu.adamw_step(h, ats, mu.adamw_hparams(step=t_counter[0], **wl.adamw_hp), stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: the steps alone, with one event between steps (on the
    # stream the steps run on) for the median; no per-launch events, which
    # would add their own time to every launch.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for k in range(args.steps):
        step()
        marks[k + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)]
    ms_per_step = elapsed * 1e3 / args.steps
    # Profiled region: the same number of steps again with the library's
    # per-launch HIP events (on the same stream), for the per-phase launch
    # times, the roofline and the memory-bound kernels' rates.
    mu.muon_profile_enable(h, True)
    mu.muon_profile_collect(h)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    profiled_ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
    phases = mu.muon_profile_collect(h)
    mu.muon_profile_enable(h, False)

    alg, dense = wl.ns_flops(hpd["steps"])
    value = alg / (ms_per_step * 1e-3) / 1e12
    n_mats = len(wl.muon)

    # per-phase algorithmic work per launch
    per_launch_flops = {"gram": 0.0, "poly": 0.0, "update": 0.0}
    # algorithmic bytes of one update launch: X read and the next X written
    # (m x n each) and B read (m x m), in the iteration's element size
    ns_elem = 4 if hpd["ns_dtype"] == "fp32" else 2
    update_bytes = 0.0
    el = 0
    for r, c in wl.muon_shapes():
        m, n = min(r, c), max(r, c)
        per_launch_flops["gram"] += m * m * n
        per_launch_flops["poly"] += m ** 3
        per_launch_flops["update"] += 2 * m * m * n
        update_bytes += (2 * m * n + m * m) * ns_elem
        el += r * c
    peak_mm = PEAK_F32_TFLOPS if hpd["ns_dtype"] == "fp32" else PEAK_BF16_TFLOPS
    # Per phase and Newton-Schulz iteration: every launch of the phase (one
    # per size class in use, plus the reduce launch of a K-split Gram).
    iters = args.steps * hpd["steps"]
    gemm = {}
    for ph in ("gram", "poly", "update"):
        ms, cnt = phases[ph]
        per_iter = ms / max(iters, 1)
        tf = per_launch_flops[ph] / (per_iter * 1e-3) / 1e12 if per_iter > 0 else 0.0
        gemm[ph] = {"avg_ms": round(per_iter, 4), "launches": cnt,
                    "launches_per_iteration": round(cnt / max(iters, 1), 3),
                    "tflops": round(tf, 1), "frac": round(tf / peak_mm, 4)}
    dom = max(("gram", "poly", "update"), key=lambda p: phases[p][0])
    # memory-bound kernels.  Algorithmic bytes per element: momentum reads G
    # and M, writes M and the Newton-Schulz input (G 4|2 + 4 + 4 + 2|4);
    # apply reads W and O and writes W (4 + 2|4 + 4).  The fp32 iteration
    # also keeps the transposed copy of the input (+4 B), counted in "actual".
    g_bytes = 2 if wl.tensors[wl.muon[0].tensor].grad_dtype == torch.bfloat16 else 4
    ns_b = 4 if hpd["ns_dtype"] == "fp32" else 2
    ns_copies = 2 if hpd["ns_dtype"] == "fp32" else 1
    ew_bytes = {"momentum": ((g_bytes + 4 + 4 + ns_b) * el, (g_bytes + 4 + 4 + ns_copies * ns_b) * el),
                "apply": ((4 + ns_b + 4) * el, (4 + ns_b + 4) * el)}
    hbm = {}
    # A small class alone whose weights are plain fp32 blocks applies the step
    # inside its last update (no apply launch): that launch reads and writes W
    # (8 B per element) where it would have written X (2 B).
    apply_fused = phases["apply"][1] == 0 and phases["update"][1] > 0
    if apply_fused:
        update_bytes += (8 - ns_b) * el / hpd["steps"]
    for ph, (b, b_act) in ew_bytes.items():
        if ph == "apply" and apply_fused:
            hbm[ph] = {"fused_into": "update", "launches_per_step": 0}
            continue
        # per step: every launch of the phase (one per elementwise tile kind in use)
        ms, cnt = phases[ph]
        avg = ms / max(args.steps, 1)
        gbs = b / (avg * 1e-3) / 1e9 if avg > 0 else 0.0
        gbs_act = b_act / (avg * 1e-3) / 1e9 if avg > 0 else 0.0
        hbm[ph] = {"avg_ms": round(avg, 4), "launches_per_step": round(cnt / max(args.steps, 1), 3),
                   "gb_s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                   "bytes_per_step": b, "actual_gb_s": round(gbs_act, 1),
                   "actual_frac": round(gbs_act / PEAK_HBM_GBS, 4)}
    if ats:
        ad_el = sum(int(np.prod(wl.tensors[i].shape)) for i in wl.adamw)
        ms, cnt = phases["adamw"]
        avg_step = ms / max(args.steps, 1)
        gbs = 28 * ad_el / (avg_step * 1e-3) / 1e9 if avg_step > 0 else 0.0
        hbm["adamw"] = {"ms_per_step": round(avg_step, 4), "gb_s": round(gbs, 1),
                        "frac": round(gbs / PEAK_HBM_GBS, 4)}

    dom_avg_ms = gemm[dom]["avg_ms"]
    # HBM bytes per update launch from rocprofv3 counters, where a record for
    # this workload and the current kernel source is committed
    records = {"headline": "update_bf16_headline", "perhead": "update_strip_perhead"}
    traffic = _traffic_record(records[args.workload]) if (dom == "update" and args.workload in records) else None
    upd_name = ("ns_update (X <- B X, B = aI + bA + cAA)" if hpd["ns_dtype"] == "bf16"
                else "fp32 update (X <- aX + BX, B = bA + cAA)")
    roofline = {"bound": "mfma", "kernel": upd_name if dom == "update" else dom,
                "achieved": gemm[dom]["tflops"], "peak": peak_mm, "unit": "TFLOP/s",
                "frac": gemm[dom]["frac"], "traffic": traffic,
                "per_launch_flops": per_launch_flops[dom], "avg_launch_ms": dom_avg_ms,
                "launches_per_iteration": gemm[dom]["launches_per_iteration"],
                "timing": "HIP events around every launch, in a second pass of the same steps "
                          "after the timed region"}
    # An update whose arithmetic intensity lies below the ridge point (short
    # side m: about m/2 flop per byte in bf16) is bound by HBM, not by the
    # matrix cores: per-head blocks (m = 128) are.  Report that roofline then.
    hbm_rf = hbm_roofline(per_launch_flops["update"], update_bytes, dom_avg_ms, peak_mm) if dom == "update" else None
    if hbm_rf:
        roofline.update(hbm_rf)

    out = {
        "metric": "Muon step TFLOP/s (algorithmic, bf16 Newton-Schulz) and matrices/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "profiled_ms_per_step": round(profiled_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if hpd["ns_dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": n_mats,
                   "shapes": sorted(set(map(tuple, wl.muon_shapes()))),
                   "ns_steps": hpd["steps"], "param_dtype": "f32", "momentum_dtype": "f32"},
        "matrices_per_s": round(n_mats / (ms_per_step * 1e-3), 2),
        "dense_equiv_tflops": round(dense / (ms_per_step * 1e-3) / 1e12, 2),
        "algorithmic_tflop_per_step": alg / 1e12,
        "roofline": roofline,
        "gemm_phases": gemm,
        "hbm_kernels": hbm,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))
    mu.muon_destroy(h)


if __name__ == "__main__":
    main()
