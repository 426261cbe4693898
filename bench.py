#!/usr/bin/env python3
"""Throughput of the Shampoo optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]

One step is the whole hot path over one batch of synthetic gradients already
resident in HBM: statistics of every block, the inverse roots when
step % cadence == 0, the two-sided preconditioning, grafting, momentum and
the weight update (plus dense/sparse Adagrad where the workload has them).
The timed steps are t = W .. W+K-1, so K/cadence root passes fall inside the
timed region (the one at t = 0 is warm-up).

Prints one JSON line: steps/s per 100M parameters (the headline), the
inverse-root blocks/s and %MFMA of each MFMA stage, a per-kernel breakdown
from HIP events recorded around the launches inside the timed region, the
roofline of the dominant kernel, and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host.

Inside the timed region the per-launch events are recorded in the steps that
recompute roots and in the step after each (events around every launch of
every step cost about 0.025 ms per step on Transformer-base, 2 %); every
root-pass launch is timed, and each family's launches per step, counted on
the warm-up steps, scale its sampled average to the whole region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

from second_order_optimizer_amd import synth  # noqa: E402

METRIC = "Shampoo optimizer steps/sec per 100M params; inv-root blocks/sec; %MFMA peak"
UNIT = "optimizer steps/s x (params / 1e8)"

# MI355X published peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6}

KERNEL_SOURCES = [os.path.join(HERE, "second_order_optimizer_amd", "csrc", f)
                  for f in ("kernels.hip", "api.cpp", "common.hpp", "kernels.hpp")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ work model
def factor_dims(opt, root_p):
    """(dimension, root exponent) of every factor, in factor order: L and R
    of each Lemma-2 block, then the one factor of each one-sided block
    (exponent root_p / 2)."""
    blocks = [opt.block(i) for i in range(opt.n_blocks)]
    out = []
    for b in blocks:
        if not b.one_sided:
            out += [(b.rows, root_p), (b.cols, root_p)]
    for b in blocks:
        if b.one_sided:
            out.append((b.cols if b.factor_r >= 0 else b.rows, root_p // 2))
    return out


def newton_flops(n, p, iters):
    """Coupled-Newton GEMM flops of one n x n root: X T, then T^p M by
    repeated squaring (log2 p - 1 squarings after T^2) and the M update, per
    iteration; X_0 is diagonal, so the first X T is a row scaling and not a
    product (every root path forms it that way)."""
    gemms = 2 + int(round(math.log2(p))) if p > 1 else 2
    return gemms * 2.0 * n ** 3 * iters - 2.0 * n ** 3


def work_model(wl, opt, n_fp64_factors_per_pass):
    """Algorithmic flops / bytes per launch of each kernel family.

    Statistics and apply count every product of the formulas as a dense GEMM
    (2 M N K); the root counts 4 n^3 GEMMs x 2 flops x iterations per factor,
    less the first X T (a row scaling)
    (p = 4: X T, T^2, T^4, T^4 M).  Elementwise kernels count the bytes the
    formulas must move once (fp32)."""
    nb = opt.n_blocks
    blocks = [opt.block(i) for i in range(nb)]
    onesided = [b for b in blocks if b.one_sided]
    blocks = [b for b in blocks if not b.one_sided]
    gram = sum(2.0 * (b.rows ** 2 * b.cols + b.cols ** 2 * b.rows) for b in blocks)
    apply_t = sum(2.0 * b.rows * b.cols ** 2 for b in blocks)
    apply_d = sum(2.0 * b.rows ** 2 * b.cols for b in blocks)
    # one-sided blocks (Lemma 1): S = G^T G or G G^T and D = G P or P G are
    # each 2 dim numel flops
    def listed_rows(b):   # a sparse table's statistics and apply see the listed rows only
        t = wl.tensors[b.tensor]
        return round(wl.sparse_frac * t.rows) if t.kind == "sparse" else b.rows
    def os_flops(bs):
        return sum(2.0 * (b.cols if b.factor_r >= 0 else b.rows) * listed_rows(b) * b.cols
                   for b in bs)
    sparse_os = [b for b in onesided if wl.tensors[b.tensor].kind == "sparse"]
    dense_os = [b for b in onesided if wl.tensors[b.tensor].kind == "dense"]
    dims = [(dim, p) for dim, p in factor_dims(opt, wl.root_p)]
    root_flops_all = sum(newton_flops(n, p, wl.newton_iters) for n, p in dims)   # full count
    shampoo_params = sum(b.rows * b.cols for b in blocks) + sum(b.rows * b.cols for b in dense_os)
    small = [b for b in blocks if b.rows <= 128 and b.cols <= 128]
    big = [b for b in blocks if not (b.rows <= 128 and b.cols <= 128)] + dense_os
    dense_fallback = sum(t.numel for t in wl.tensors if t.kind == "dense") - shampoo_params
    # tensors whose blocks are all <= 128 get their momentum and weight update
    # inside the fused apply kernel
    has_big = {b.tensor for b in big}
    fused = [b for b in small if b.tensor not in has_big]
    unfused_params = shampoo_params - sum(b.rows * b.cols for b in fused)
    # fused apply bytes: G, a (read+write), the two fp32 roots, and either
    # D (write) or momentum and weight (read+write each)
    apply_small_bytes = sum((28.0 if b.tensor not in has_big else 16.0) * b.rows * b.cols +
                            4.0 * (b.ld_l ** 2 + b.ld_r ** 2) for b in small)
    # fused step kernel (steps without roots, blocks <= 128): statistics
    # (fp64 MFMA, upper triangles read and written in fp64) plus the apply
    step_small_bytes = apply_small_bytes + sum(
        8.0 * (b.rows * (b.rows + 1) + b.cols * (b.cols + 1)) for b in small)
    return {
        "gram": gram, "apply_t": apply_t, "apply_d": apply_d,
        "gram_small": sum(2.0 * (b.rows ** 2 * b.cols + b.cols ** 2 * b.rows) for b in small),
        "step_small_bytes": step_small_bytes,
        "apply_small_bytes": apply_small_bytes, "unfused_params": unfused_params,
        "apply_small": sum(2.0 * (b.rows * b.cols ** 2 + b.rows ** 2 * b.cols) for b in small),
        "apply_t_big": sum(2.0 * b.rows * b.cols ** 2 for b in big if not b.one_sided),
        "apply_d_big": sum(2.0 * b.rows ** 2 * b.cols for b in big if not b.one_sided) +
        os_flops(dense_os),
        "stats_onesided": os_flops(dense_os),
        "stats_onesided_rows": os_flops(sparse_os), "apply_onesided_rows": os_flops(sparse_os),
        "onesided_rows_elems": sum(listed_rows(b) * b.cols for b in sparse_os),
        "shampoo_params_big": sum(b.rows * b.cols for b in big),
        "root_flops_all": root_flops_all,
        "root_flops_per_factor_mean": root_flops_all / max(len(dims), 1),
        "shampoo_params": shampoo_params, "dense_fallback": dense_fallback,
    }


# -------------------------------------------------------------------- CPU leg
def cpu_baseline(wl, sample_ids, steps_plain=3):
    """The fp64 oracle, as it stands, on a bounded sample of the workload."""
    from oracle import shampoo_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cfg = O.OracleConfig(block_size=wl.block_size, max_precond_dim=wl.max_precond_dim,
                         root_p=wl.root_p, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr,
                         eps_rel=wl.eps_rel, graft_eps=wl.graft_eps, cadence=wl.cadence)
    specs = [wl.tensors[i] for i in sample_ids]
    orc = O.ShampooOracle(cfg, [(s.rows, s.cols, s.kind) for s in specs],
                          [synth.initial_weight(wl, i) for i in sample_ids])
    gs = synth.GradientStream(wl, sample_ids)
    times = []
    for t in range(1 + steps_plain):
        g = gs.step(t)
        grads = [g[i] if specs[k].kind == "dense" else g[i] for k, i in enumerate(sample_ids)]
        t0 = time.perf_counter()
        orc.step(grads, t)          # t = 0 recomputes every root
        times.append(time.perf_counter() - t0)
    t_plain = float(np.median(times[1:]))
    t_root = max(times[0] - t_plain, 0.0)
    t_amort = t_plain + t_root / wl.cadence
    params = sum(s.numel for s in specs)
    return {
        "value": (1.0 / t_amort) * params / 1e8,
        "unit": UNIT,
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(sample_ids)} of {len(wl.tensors)} tensors "
                   f"({params / 1e6:.2f}M of {wl.n_params / 1e6:.2f}M params: "
                   f"{', '.join(s.name for s in specs[:6])}{'...' if len(specs) > 6 else ''}); "
                   f"1 step with every root recomputed ({times[0]:.2f} s) + {steps_plain} plain "
                   f"steps (median {t_plain:.2f} s); amortised over cadence {wl.cadence}; "
                   f"scaled by parameter count"),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def default_cpu_sample(wl):
    if wl.wid == 1:   # one encoder and one decoder layer of the Transformer
        return [i for i, t in enumerate(wl.tensors) if t.name.startswith(("enc0.", "dec0."))]
    if wl.wid == 2:
        return [i for i, t in enumerate(wl.tensors) if t.name.startswith("layer0.")][:2]
    if wl.wid == 3:
        return list(range(0, 14))
    if wl.wid == 4:
        return [0, 1, 2, 3]
    return list(range(len(wl.tensors)))


# ------------------------------------------------------------------- GPU leg
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1,
                    help="0: 256x512 b128, 1: Transformer-base b128 (default), 2: BERT-large "
                         "b512, 3: ResNet-50 b256, 4: CTR MLP b1024 + sparse tables")
    ap.add_argument("--root-mode", default=None, choices=["f32", "f64", "auto"])
    ap.add_argument("--newton-tol", type=float, default=None,
                    help="fused-root convergence tolerance (0: the full iteration count)")
    ap.add_argument("--pool", type=int, default=4, help="distinct gradient sets kept in HBM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--root-parts", type=int, default=0,
                    help="staggered root pass: recompute 1/P of the roots every cadence/P "
                         "steps (P must divide the cadence); 0 = one pass every cadence steps")
    ap.add_argument("--async-roots", action="store_true",
                    help="with --root-parts: each part computed in the background on a stream "
                         "of the library's own and swapped in when the next part starts")
    ap.add_argument("--large-layer", action="store_true",
                    help="one-sided preconditioning (Lemma 1) of dense tensors with one "
                         "dimension above max_precond_dim (the embedding of the Transformer "
                         "workload) instead of diagonal Adagrad")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without the per-launch events (no per-kernel breakdown)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(sharding the blocks over GPUs is designed, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from second_order_optimizer_amd import shampoo as S

    wl = synth.workload(args.workload)
    if args.newton_tol is not None:
        wl.newton_tol = args.newton_tol
    if args.root_mode:
        wl.root_mode = args.root_mode
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = S.make_config(wl.block_size, max_precond_dim=wl.max_precond_dim, root_p=wl.root_p,
                        newton_iters=wl.newton_iters, root_mode=wl.root_mode, beta1=wl.beta1,
                        beta2=wl.beta2, lr=wl.lr, eps_rel=wl.eps_rel, graft_eps=wl.graft_eps,
                        fp64_cond_threshold=wl.fp64_cond_threshold, root_parts=args.root_parts,
                        newton_tol=wl.newton_tol,
                        large_layer=1 if args.large_layer else 0)
    shapes = [(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in wl.tensors]
    t0 = time.time()
    opt = S.Shampoo(shapes, cfg, device=dev, async_roots=args.async_roots)
    params = [torch.from_numpy(synth.initial_weight(wl, i)).to(dev) for i in range(len(shapes))]
    gs = synth.GradientStream(wl)
    pool = []
    for k in range(args.pool):
        g = gs.step(k)
        dense, sparse = [], {}
        for i, spec in enumerate(wl.tensors):
            if spec.kind == "dense":
                dense.append(torch.from_numpy(g[i]).to(dev))
            else:
                rows, rg = g[i]
                dense.append(None)
                sparse[i] = (torch.from_numpy(rows).to(dev), torch.from_numpy(rg).to(dev))
        pool.append((dense, sparse))
    torch.cuda.synchronize()
    print(f"# setup {time.time() - t0:.1f} s: {wl.name}, {wl.n_params / 1e6:.2f}M params, "
          f"{opt.n_blocks} blocks, state {opt.state_bytes / 2**30:.2f} GiB", file=sys.stderr,
          flush=True)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step(t):
        dense, sparse = pool[t % len(pool)]
        opt.step(params, dense, t, wl.cadence, sparse if sparse else None)

    def kind(t):   # which roots a step recomputes (S.ROOTS_NONE: none)
        return S.root_selector(t, wl.cadence, cfg.root_parts)

    def sampled(t):   # timed steps that carry per-launch events
        return kind(t) != S.ROOTS_NONE or (t > 0 and kind(t - 1) != S.ROOTS_NONE)

    # warm-up; each family's launches per step, by the roots the step recomputes
    per_kind = {}
    for t in range(args.warmup):
        if not args.no_profile:
            opt.profile(True)
        step(t)
        if not args.no_profile:
            per_kind[kind(t)] = {k: v[0] for k, v in opt.profile_read().items() if v[0] > 0}
            opt.profile(False)
    torch.cuda.synchronize()
    print(f"# warm-up {args.warmup} steps done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_profile:
        opt.profile_read()        # reset
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    marks = []                  # one event after every step: per-step GPU time
    for t in range(args.warmup, args.warmup + args.steps):
        if not args.no_profile:
            opt.profile(sampled(t))
        step(t)
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        marks.append(e)
    if args.async_roots:
        opt.roots_async_end()   # the part still in flight belongs to the timed work
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = ev0.elapsed_time(ev1)
    per_step = [ev0.elapsed_time(marks[0])] + [a.elapsed_time(b) for a, b in zip(marks, marks[1:])]
    per_step.sort()
    step_ms = {"p50": per_step[len(per_step) // 2],
               "p99": per_step[min(len(per_step) - 1, int(0.99 * len(per_step)))],
               "max": per_step[-1]}
    prof = opt.profile_read() if not args.no_profile else {}
    opt.profile(False)
    ms_step = ms_total / args.steps
    # root passes in the timed steps (a staggered pass counts 1/P per part)
    n_root_passes = sum(1 for t in range(args.warmup, args.warmup + args.steps)
                        if t % wl.cadence == 0)
    diag = opt.diagnostics()
    n64 = sum(1 for d in diag if d.status & S.FACTOR_FP64)
    wm = work_model(wl, opt, n64)

    steps_per_s = 1000.0 / ms_step
    value = steps_per_s * wl.n_params / 1e8

    # per-kernel breakdown
    def fam(name):
        return prof.get(name, (0, 0.0))

    stages = {}
    fp64_share = n64 / max(len(diag), 1)
    fdims = factor_dims(opt, wl.root_p)
    # the steps each root ran in the last pass (a fused root with a tolerance
    # stops at convergence; the batched paths run the full count)
    fl = [newton_flops(n, p, d.iters) if d.iters > 0 else 0.0 for (n, p), d in zip(fdims, diag)]
    iters_run = [d.iters for (n, _), d in zip(fdims, diag) if n <= 128 and d.iters > 0]
    f32 = wl.root_mode != "f64"
    flops_fused_root = sum(x for x, (n, _) in zip(fl, fdims) if f32 and n <= 128)
    flops_f32_root = sum(x for x, (n, _) in zip(fl, fdims) if f32 and n > 128)
    flops_f64_root = sum(x for x, d in zip(fl, diag) if d.status & S.FACTOR_FP64)
    alg = {
        # name: (work per launch, unit, bound, peak)
        "stats_gram_f64": (wm["gram"], "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]),
        "stats_onesided": (wm["stats_onesided"], "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]),
        "stats_onesided_rows": (wm["stats_onesided_rows"], "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]),
        "apply_onesided_rows": (wm["apply_onesided_rows"], "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]),
        # g read, a read and written (row ids aside); D read, W read and written
        "onesided_rows_norm": (wm["onesided_rows_elems"] * 12.0, "GB/s", "hbm", PEAK_HBM_GBS),
        "onesided_rows_update": (wm["onesided_rows_elems"] * 12.0, "GB/s", "hbm", PEAK_HBM_GBS),
        "apply_gemm_t": (wm["apply_t_big"], "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]),
        "apply_gemm_d": (wm["apply_d_big"], "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]),
        "adagrad_norm": (wm["shampoo_params_big"] * 12.0, "GB/s", "hbm", PEAK_HBM_GBS),
        "update": (wm["unfused_params"] * 20.0 + wm["dense_fallback"] * 28.0, "GB/s", "hbm",
                   PEAK_HBM_GBS),
    }
    # the fused apply is bounded by whichever of its MFMA and HBM floors is higher
    if wm["apply_small"] / (PEAK_TFLOPS["f32"] * 1e12) >= wm["apply_small_bytes"] / (PEAK_HBM_GBS * 1e9):
        alg["apply_fused"] = (wm["apply_small"], "TFLOP/s", "mfma", PEAK_TFLOPS["f32"])
    else:
        alg["apply_fused"] = (wm["apply_small_bytes"], "GB/s", "hbm", PEAK_HBM_GBS)
    # the fused step kernel: fp64 statistics and fp32 apply share the matrix
    # pipe, so its MFMA floor is the sum of both times at their peaks; its
    # roofline is the higher of that floor and the HBM floor
    t_mfma_step = (wm["gram_small"] / (PEAK_TFLOPS["f64"] * 1e12) +
                   wm["apply_small"] / (PEAK_TFLOPS["f32"] * 1e12))
    t_hbm_step = wm["step_small_bytes"] / (PEAK_HBM_GBS * 1e9)
    timed = range(args.warmup, args.warmup + args.steps)
    for name, (launches, tot) in prof.items():
        if launches == 0:
            continue
        # launches of the family over the whole timed region (from the warm-up
        # counts per step kind); the sampled launches give its average
        total = sum(per_kind.get(kind(t), {}).get(name, 0) for t in timed)
        total = max(total, int(launches))
        rec = {"launches": int(total), "launches_timed": int(launches), "avg_ms": tot / launches,
               "ms_per_step": tot / launches * total / args.steps}
        if name == "step_fused":
            sec = rec["avg_ms"] / 1e3
            rec.update({"mfma_floor_frac": t_mfma_step / sec, "hbm_floor_frac": t_hbm_step / sec,
                        "hbm_achieved_gbs": wm["step_small_bytes"] / sec / 1e9})
            if t_mfma_step >= t_hbm_step:
                # an fp64 flop counts as two fp32 flops (the fp64 peak is half)
                eq = (2.0 * wm["gram_small"] + wm["apply_small"]) / sec / 1e12
                rec.update({"bound": "mfma", "achieved": eq, "peak": PEAK_TFLOPS["f32"],
                            "unit": "TFLOP/s (fp32-equivalent)", "frac": t_mfma_step / sec})
            else:
                rec.update({"bound": "hbm", "achieved": wm["step_small_bytes"] / sec / 1e9,
                            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": t_hbm_step / sec})
            stages[name] = rec
            continue
        work = None
        if name in alg:
            work, unit, bound, peak = alg[name]
        elif name == "newton_fused_f32" and flops_fused_root > 0:
            work = flops_fused_root * n_root_passes / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]
        elif name == "newton_gemm_f32" and flops_f32_root > 0:
            work = flops_f32_root * n_root_passes / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]
        elif name == "newton_gemm_f64" and flops_f64_root > 0:
            work = flops_f64_root * n_root_passes / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]
        if work is not None:
            sec = rec["avg_ms"] / 1e3
            ach = work / sec / (1e12 if unit == "TFLOP/s" else 1e9)
            rec.update({"bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                        "frac": ach / peak})
        stages[name] = rec

    # the dominant kernel family by time in the timed region
    roofline = None
    dom = max(stages.items(), key=lambda kv: kv[1]["ms_per_step"]) if stages else None
    if dom and "achieved" in dom[1]:
        traffic = None
        tf = os.path.join(HERE, "profiles", "traffic.json")
        if os.path.exists(tf):
            with open(tf) as f:
                tj = json.load(f)
            ent = tj.get(dom[0])
            if ent and ent.get("kernel_hash") == kernel_hash() and \
                    ent.get("workload") == wl.name:
                traffic = ent.get("bytes_per_launch")
        roofline = {"kernel": dom[0], "bound": dom[1]["bound"], "achieved": dom[1]["achieved"],
                    "peak": dom[1]["peak"], "unit": dom[1]["unit"], "frac": dom[1]["frac"],
                    "traffic": traffic}

    root_ms = sum(stages[n]["ms_per_step"] * args.steps for n in
                  ("lanczos_stats", "lanczos_roots", "newton_init", "newton_gemm_f32",
                   "newton_gemm_f64", "newton_commit", "newton_fused_f32", "route_compact")
                  if n in stages)
    inv_root_blocks_per_s = (opt.n_blocks * n_root_passes / (root_ms / 1e3)) if root_ms > 0 else None
    mfma_pct = {k: round(100 * v["frac"], 2) for k, v in stages.items() if v.get("bound") == "mfma"}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 gradients/weights; f64 statistics; f32+f64 (routed) roots",
        "data": "synthetic",
        "config": {"workload": wl.name, "params": wl.n_params, "blocks": opt.n_blocks,
                   "block_size": wl.block_size, "root_cadence": wl.cadence,
                   "newton_iters": wl.newton_iters, "newton_tol": wl.newton_tol,
                   "root_mode": wl.root_mode,
                   "root_parts": args.root_parts, "async_roots": bool(args.async_roots),
                   "large_layer": bool(args.large_layer),
                   "max_precond_dim": wl.max_precond_dim, "parallelism": "single-gpu"},
        "steps_per_s": steps_per_s,
        "inv_root_blocks_per_s": inv_root_blocks_per_s,
        "root_passes_timed": n_root_passes,
        "fp64_factor_share_last_pass": fp64_share,
        "fused_root_iters_last_pass": ({"mean": sum(iters_run) / len(iters_run),
                                        "min": min(iters_run), "max": max(iters_run)}
                                       if iters_run else None),
        "mfma_pct": mfma_pct,
        "stages": stages,
        "roofline": roofline,
        "wall_s_timed": wall,
        "step_ms": step_ms,
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, default_cpu_sample(wl))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
