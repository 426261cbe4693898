#!/usr/bin/env python3
"""Throughput of the Shampoo optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step is the whole hot path over one batch of synthetic gradients already
resident in HBM: statistics of every block, the inverse roots when
step % cadence == 0, the two-sided preconditioning, grafting, momentum and
the weight update (plus dense/sparse Adagrad where the workload has them).
The timed steps are t = W .. W+K-1, so the root passes at multiples of the
cadence inside that range are timed (the one at t = 0 is warm-up).

The default workload is BERT-large (302M parameters, 1152 blocks of 512,
fp64 roots for ill-conditioned factors), the largest of the five.  The
headline `value` is taken with the workload's convergence tolerance of the
fp32 roots; the same line also reports a second timed pass with the full
iteration count (newton_tol 0).

Prints one JSON line: steps/s per 100M parameters (the headline), the
inverse-root blocks/s and %MFMA of each MFMA stage, a per-kernel breakdown
from HIP events recorded around the launches inside the timed region, the
roofline of the dominant kernel, the machine peaks measured on the device,
and the fp64 CPU oracle timed per stage on a bounded sample of the same
workload on this host, with all threads and with one.

Work is counted as the method needs it: a product whose result is symmetric
(the statistics G G^T and G^T G, every product of the coupled Newton
iteration, whose iterates are all polynomials in one matrix) counts the
multiply-adds of its upper triangle, n (n + 1) k flops for an n x n result
over k; other products count 2 m n k.

The timed steps carry no per-launch events (one event after each step).  The
per-kernel breakdown comes from as many steps again, run right after them:
there the per-launch events are recorded in the steps that recompute roots
and in the step after each; every root-pass launch is timed, and each
family's launches per step, counted on the warm-up steps, scale its sampled
average to the whole region.

Two offline modes turn rocprofv3 output into the summaries under profiles/:
    python bench.py --trace-summary DIR --title T --command C > profiles/X.md
    python bench.py --counters-summary DIR --workload N [--kernel-trace DIR2]
The second reads the FETCH_SIZE, WRITE_SIZE and SQ counter runs (one
rocprofv3 --pmc run each, under DIR/pmc_fetch, DIR/pmc_write, DIR/pmc_sq),
scales FETCH_SIZE and WRITE_SIZE by what they read for the peak probe's
plain copy (k_peak_copy, of known size), and writes profiles/traffic.json
entries for the workload and a counters table to stdout.
"""
from __future__ import annotations

import argparse
import csv
import glob
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
PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6, "bf16": 2500.0}

KERNEL_SOURCES = [os.path.join(HERE, "second_order_optimizer_amd", "csrc", f)
                  for f in ("kernels.hip", "api.cpp", "common.hpp", "kernels.hpp")]
TRAFFIC_JSON = os.path.join(HERE, "profiles", "traffic.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ work model
def sym(n, k):
    """Flops of a product with a symmetric n x n result over k: the upper
    triangle's n (n + 1) / 2 entries, 2 k flops each."""
    return float(n) * (n + 1) * k


def newton_products(p):
    """Products per coupled-Newton step: X T, then T^p by repeated squaring
    (log2 p squarings), then T^p M; p = 1: X T and T M."""
    return 2 if p == 1 else 2 + int(round(math.log2(p)))


def newton_flops(n, p, iters, batched):
    """One n x n root of `iters` steps.  X, M and T are polynomials in the
    same matrix, so every product is symmetric (counted on its triangle);
    X_0 is diagonal, so the first X T is a row scaling and not a product.  The
    batched chains form only X in their last step (that step's M is never
    read)."""
    if batched:
        return newton_products(p) * sym(n, n) * max(iters - 1, 0)
    return newton_products(p) * sym(n, n) * iters - sym(n, n)


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


def work_model(wl, opt):
    """Algorithmic flops / bytes per launch of each kernel family: the
    statistics are symmetric products (their triangle's flops), the apply two
    general products (2 m n k each), elementwise kernels the bytes the
    formulas must move once (fp32)."""
    nb = opt.n_blocks
    blocks = [opt.block(i) for i in range(nb)]
    onesided = [b for b in blocks if b.one_sided]
    blocks = [b for b in blocks if not b.one_sided]

    def gram(bs):
        return sum(sym(b.rows, b.cols) + sym(b.cols, b.rows) for b in bs)

    def apply(bs):
        return sum(2.0 * (b.rows * b.cols ** 2 + b.rows ** 2 * b.cols) for b in bs)

    def listed_rows(b):   # a sparse table's statistics and apply see the listed rows only
        t = wl.tensors[b.tensor]
        return round(wl.sparse_frac * t.rows) if t.kind == "sparse" else b.rows

    def os_dim(b):
        return b.cols if b.factor_r >= 0 else b.rows

    def os_stats(bs):      # S = G^T G (or G G^T): symmetric, over the long dimension
        return sum(sym(os_dim(b), listed_rows(b) if b.factor_r >= 0 else b.cols) for b in bs)

    def os_apply(bs):      # D = G P or P G
        return sum(2.0 * os_dim(b) * listed_rows(b) * b.cols for b in bs)

    sparse_os = [b for b in onesided if wl.tensors[b.tensor].kind == "sparse"]
    dense_os = [b for b in onesided if wl.tensors[b.tensor].kind == "dense"]
    shampoo_params = sum(b.rows * b.cols for b in blocks) + sum(b.rows * b.cols for b in dense_os)
    small = [b for b in blocks if b.rows <= 128 and b.cols <= 128]
    big = [b for b in blocks if not (b.rows <= 128 and b.cols <= 128)]
    dense_fallback = sum(t.numel for t in wl.tensors if t.kind == "dense") - shampoo_params
    # tensors whose blocks are all <= 128 get their momentum and weight update
    # inside the fused apply kernel
    has_big = {b.tensor for b in big + dense_os}
    fused = [b for b in small if b.tensor not in has_big]
    unfused_params = shampoo_params - sum(b.rows * b.cols for b in fused)
    # fused apply bytes: G, a (read+write), the two fp32 roots, and either
    # D (write) or momentum and weight (read+write each)
    apply_small_bytes = sum((28.0 if b.tensor not in has_big else 16.0) * b.rows * b.cols +
                            4.0 * (b.ld_l ** 2 + b.ld_r ** 2) for b in small)
    # fused step kernel (steps without roots, blocks <= 128): statistics
    # (upper triangles read and written in fp64) plus the apply, and the
    # dense-Adagrad rows its launch also runs (g, a, momentum, weight: 28 B)
    fold = dense_fallback * 28.0 if small else 0.0
    step_small_bytes = apply_small_bytes + fold + sum(
        8.0 * (b.rows * (b.rows + 1) + b.cols * (b.cols + 1)) for b in small)
    return {
        "gram": gram(blocks), "gram_small": gram(small), "gram_big": gram(big),
        "apply_small": apply(small), "step_small_bytes": step_small_bytes,
        "apply_small_bytes": apply_small_bytes, "unfused_params": unfused_params,
        "apply_t_big": sum(2.0 * b.rows * b.cols ** 2 for b in big),
        "apply_d_big": sum(2.0 * b.rows ** 2 * b.cols for b in big) + os_apply(dense_os),
        # split-precision apply: the first product reads P_R and G and takes
        # G through the Adagrad accumulator (a read and written) and writes
        # T^T; the second reads P_L and T^T and writes D
        "apply_t_bytes": sum(16.0 * b.rows * b.cols + 4.0 * b.ld_r ** 2 for b in big),
        "apply_d_bytes": sum(8.0 * b.rows * b.cols + 4.0 * b.ld_l ** 2 for b in big) +
        sum(8.0 * b.rows * b.cols + 4.0 * (b.ld_r if b.factor_r >= 0 else b.ld_l) ** 2
            for b in dense_os),
        "stats_onesided": os_stats(dense_os),
        "stats_onesided_rows": os_stats(sparse_os), "apply_onesided_rows": os_apply(sparse_os),
        "onesided_rows_elems": sum(listed_rows(b) * b.cols for b in sparse_os),
        "shampoo_params_big": sum(b.rows * b.cols for b in big + dense_os),
        "shampoo_params": shampoo_params, "dense_fallback": dense_fallback,
        "fold_bytes": fold,
        "sparse_elems": sum(round(wl.sparse_frac * t.rows) * t.cols
                            for i, t in enumerate(wl.tensors)
                            if t.kind == "sparse" and i not in {b.tensor for b in sparse_os}),
    }


# -------------------------------------------------------------------- CPU leg
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return 1


def _oracle_stage_times(wl, sample_ids, steps):
    """Per-stage seconds of the fp64 oracle's own functions on the sample's
    Lemma-2 blocks, one step with every root recomputed (t = 0) and then
    plain steps, in the order the oracle's step runs them: statistics, roots,
    precondition, then the elementwise graft, momentum and update."""
    from oracle import shampoo_oracle as O
    cfg = O.OracleConfig(block_size=wl.block_size, max_precond_dim=wl.max_precond_dim,
                         root_p=wl.root_p, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr,
                         eps_rel=wl.eps_rel, graft_eps=wl.graft_eps, cadence=wl.cadence)
    gs = synth.GradientStream(wl, sample_ids)
    grads = [gs.step(t) for t in range(steps)]       # drawn before any timing
    specs = {i: wl.tensors[i] for i in sample_ids}
    st = {}
    for i in sample_ids:
        s = specs[i]
        st[i] = dict(blocks=[(bk, np.zeros((bk[1], bk[1])), np.zeros((bk[3], bk[3])),
                              np.eye(bk[1]), np.eye(bk[3]))
                             for bk in O.blocks(s.rows, s.cols, cfg.block_size)],
                     a=np.zeros((s.rows, s.cols)), mom=np.zeros((s.rows, s.cols)),
                     W=synth.initial_weight(wl, i).astype(np.float64))
    per = {"stats": [], "roots": [], "precondition": [], "elementwise": []}
    for t in range(steps):
        g = grads[t]
        t0 = time.perf_counter()
        for i in sample_ids:
            bl = st[i]["blocks"]
            for k, (bk, L, R, PL, PR) in enumerate(bl):
                r0, mb, c0, nb = bk
                L, R = O.update_statistics(L, R, g[i][r0:r0 + mb, c0:c0 + nb], cfg.beta2)
                bl[k] = (bk, L, R, PL, PR)
        t1 = time.perf_counter()
        if t == 0:
            for i in sample_ids:
                bl = st[i]["blocks"]
                for k, (bk, L, R, PL, PR) in enumerate(bl):
                    rl = O.inverse_root(L, cfg.eps_rel, cfg.root_p)
                    rr = O.inverse_root(R, cfg.eps_rel, cfg.root_p)
                    bl[k] = (bk, L, R, rl.P if rl.ok else PL, rr.P if rr.ok else PR)
        t2 = time.perf_counter()
        Ds = {}
        for i in sample_ids:
            Ds[i] = [O.precondition(PL, g[i][bk[0]:bk[0] + bk[1], bk[2]:bk[2] + bk[3]], PR)
                     for bk, L, R, PL, PR in st[i]["blocks"]]
        t3 = time.perf_counter()
        for i in sample_ids:
            s = st[i]
            s["a"] = O.adagrad_accumulate(s["a"], g[i])
            A = O.adagrad_direction(s["a"], g[i], cfg.graft_eps)
            U = np.empty_like(A)
            for (bk, *_), D in zip(s["blocks"], Ds[i]):
                r0, mb, c0, nb = bk
                U[r0:r0 + mb, c0:c0 + nb] = O.graft(A[r0:r0 + mb, c0:c0 + nb], D)
            s["mom"], s["W"] = O.momentum_update(s["mom"], s["W"], U, cfg.beta1, cfg.lr)
        t4 = time.perf_counter()
        per["stats"].append(t1 - t0)
        if t == 0:
            per["roots"].append(t2 - t1)
        per["precondition"].append(t3 - t2)
        per["elementwise"].append(t4 - t3)
    return {k: float(np.median(v)) for k, v in per.items()}


def cpu_baseline(wl, sample_ids, steps=3):
    """The fp64 oracle, as it stands, per stage on a bounded sample of the
    workload, with all of the host's BLAS threads and with one.  The sample
    is whole Lemma-2 tensors of the workload; its per-stage times are scaled
    to the workload by parameter count.  The amortised step is
    stats + precondition + elementwise + roots / cadence."""
    params = sum(wl.tensors[i].numel for i in sample_ids)
    scale = wl.n_params / params
    out = {"unit": UNIT, "kind": "oracle"}
    runs = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    for label in ("all", "one"):
        if label == "one" and threadpool_limits is None:
            continue
        if label == "one":
            with threadpool_limits(limits=1):
                times = _oracle_stage_times(wl, sample_ids, steps)
            threads = 1
        else:
            times = _oracle_stage_times(wl, sample_ids, steps)
            threads = _blas_threads()
        amort = (times["stats"] + times["precondition"] + times["elementwise"] +
                 times["roots"] / wl.cadence)
        runs[label] = {
            "threads": int(threads),
            "value": (1.0 / (amort * scale)) * wl.n_params / 1e8,
            "ms_per_step_workload": 1e3 * amort * scale,
            "stage_ms_workload": {k: 1e3 * v * scale for k, v in times.items()},
        }
    out["value"] = runs["all"]["value"]
    out["cores"] = runs["all"]["threads"]
    out["host_cpus"] = len(os.sched_getaffinity(0))
    out["per_thread_count"] = runs
    names = [wl.tensors[i].name for i in sample_ids]
    out["sample"] = (f"{len(sample_ids)} of {len(wl.tensors)} tensors ({params / 1e6:.2f}M of "
                     f"{wl.n_params / 1e6:.2f}M params: {', '.join(names[:6])}"
                     f"{'...' if len(names) > 6 else ''}); {steps} steps, roots at the first; "
                     f"oracle stage functions timed per stage (median over the steps), scaled "
                     f"to the workload by parameter count; roots amortised over cadence "
                     f"{wl.cadence}")
    return out


def default_cpu_sample(wl):
    if wl.wid == 1:   # one encoder layer of the Transformer
        return [i for i, t in enumerate(wl.tensors) if t.name.startswith("enc0.")]
    if wl.wid == 2:   # a 1024 x 1024 projection and a 1024 x 4096 FFN matrix
        return [i for i, t in enumerate(wl.tensors)
                if t.name in ("layer0.attn.q", "layer0.ffn1")]
    if wl.wid == 3:
        return list(range(0, 14))
    if wl.wid == 4:
        return [0, 1, 2]
    return list(range(len(wl.tensors)))


# ------------------------------------------------------------------- GPU leg
def run_pass(wl, args, tol, pool, dev, peaks):
    """Warm-up and timed steps of one optimizer at fp32 root tolerance tol."""
    import torch
    from second_order_optimizer_amd import shampoo as S
    cfg = S.make_config(wl.block_size, max_precond_dim=wl.max_precond_dim, root_p=wl.root_p,
                        newton_iters=wl.newton_iters, root_mode=wl.root_mode, beta1=wl.beta1,
                        beta2=wl.beta2, lr=wl.lr, eps_rel=wl.eps_rel, graft_eps=wl.graft_eps,
                        fp64_cond_threshold=wl.fp64_cond_threshold, root_parts=args.root_parts,
                        newton_tol=tol, large_layer=1 if args.large_layer else 0,
                        apply_precision=wl.apply_precision)
    shapes = [(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in wl.tensors]
    opt = S.Shampoo(shapes, cfg, device=dev, async_roots=args.async_roots)
    params = [torch.from_numpy(synth.initial_weight(wl, i)).to(dev) for i in range(len(shapes))]
    torch.cuda.synchronize()
    print(f"# pass newton_tol={tol}: {wl.name}, {opt.n_blocks} blocks, state "
          f"{opt.state_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)

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
    # the timed steps: no per-launch events (only one event after each step)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    marks = []                  # one event after every step: per-step GPU time
    for t in range(args.warmup, args.warmup + args.steps):
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
    print(f"# timed {args.steps} steps: {ms_total / args.steps:.3f} ms per step", file=sys.stderr,
          flush=True)
    per_step = [ev0.elapsed_time(marks[0])] + [a.elapsed_time(b) for a, b in zip(marks, marks[1:])]
    per_step.sort()
    step_ms = {"p50": per_step[len(per_step) // 2],
               "p99": per_step[min(len(per_step) - 1, int(0.99 * len(per_step)))],
               "max": per_step[-1]}
    ms_step = ms_total / args.steps
    # the per-kernel breakdown: as many steps again, right after, with events
    # around the launches of the steps that recompute roots and the step
    # after each (kept out of the timed steps: events around many short
    # launches would slow them)
    prof = {}
    timed = range(args.warmup + args.steps, args.warmup + 2 * args.steps)
    if not args.no_profile:
        opt.profile_read()        # reset
        for t in timed:
            opt.profile(sampled(t))
            step(t)
        if args.async_roots:
            opt.roots_async_end()
        torch.cuda.synchronize()
        prof = opt.profile_read()
        opt.profile(False)
    n_root_passes = sum(1 for t in range(args.warmup, args.warmup + args.steps)
                        if t % wl.cadence == 0)
    n_root_passes_prof = sum(1 for t in timed if t % wl.cadence == 0)
    diag = opt.diagnostics()
    n64 = sum(1 for d in diag if d.status & S.FACTOR_FP64)
    wm = work_model(wl, opt)
    steps_per_s = 1000.0 / ms_step
    value = steps_per_s * wl.n_params / 1e8

    stages = {}
    fdims = factor_dims(opt, wl.root_p)
    # the steps each root ran in the last pass (with a tolerance the fused
    # fp32 roots stop at convergence and the batched chains run the count of
    # their scaled steps' bound)
    fl = [newton_flops(n, p, d.iters, n > 128 or bool(d.status & S.FACTOR_FP64)) if d.iters > 0
          else 0.0 for (n, p), d in zip(fdims, diag)]
    iters32 = {"fused": [d.iters for (n, _), d in zip(fdims, diag)
                         if n <= 128 and d.iters > 0 and not d.status & S.FACTOR_FP64],
               "chain": [d.iters for (n, _), d in zip(fdims, diag)
                         if n > 128 and d.iters > 0 and not d.status & S.FACTOR_FP64],
               "fp64": [d.iters for d in diag if d.iters > 0 and d.status & S.FACTOR_FP64]}
    f32 = wl.root_mode != "f64"
    # in AUTO mode the fp32 iteration runs on every factor first and the
    # routed ones are redone in fp64; a routed factor's fp32 steps are not
    # recorded, so it counts at the steps of its fp64 root
    flops_fused_root = sum(x for x, (n, _) in zip(fl, fdims) if f32 and n <= 128)
    flops_f32_root = sum(x for x, (n, _) in zip(fl, fdims) if f32 and n > 128)
    flops_f64_root = sum(x for x, d in zip(fl, diag) if d.status & S.FACTOR_FP64)
    alg = {
        # name: (work per launch, unit, bound, peak)
        "stats_gram_f64": (wm["gram_big"], "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]),
        "stats_gram128": (wm["gram_small"], "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]),
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
        # g read, a and W read and written, row ids
        "sparse_rows": (wm["sparse_elems"] * 20.0, "GB/s", "hbm", PEAK_HBM_GBS),
    }
    if wl.apply_precision == "bf16x3":
        # three bf16 products per fp32 product on the bf16 matrix cores; each
        # launch is bounded by whichever of that floor and its HBM floor
        # (bytes above) is higher
        for name, fk, bk in (("apply_gemm_t", "apply_t_big", "apply_t_bytes"),
                             ("apply_gemm_d", "apply_d_big", "apply_d_bytes")):
            t_m = 3.0 * wm[fk] / (PEAK_TFLOPS["bf16"] * 1e12)
            t_h = wm[bk] / (PEAK_HBM_GBS * 1e9)
            alg[name] = ((3.0 * wm[fk], "TFLOP/s", "mfma", PEAK_TFLOPS["bf16"]) if t_m >= t_h
                         else (wm[bk], "GB/s", "hbm", PEAK_HBM_GBS))
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
    for name, (launches, tot) in prof.items():
        if launches == 0:
            continue
        # launches of the family over the whole timed region (from the warm-up
        # counts per step kind); the sampled launches give its average
        total = sum(per_kind.get(kind(t), {}).get(name, 0) for t in timed)
        total = max(total, int(launches))
        rec = {"launches": int(total), "launches_timed": int(launches), "avg_ms": tot / launches,
               "ms_per_step": tot / launches * total / args.steps}
        if name == "update" and wm["fold_bytes"] > 0:
            # the update of a step through the fused step kernel leaves the
            # dense-Adagrad rows to that kernel: bytes per launch by the kind
            # of step each sampled launch came from
            nr = nf = 0
            for t in timed:
                if sampled(t):
                    n = per_kind.get(kind(t), {}).get(name, 0)
                    if kind(t) == S.ROOTS_NONE:
                        nf += n
                    else:
                        nr += n
            wr = wm["unfused_params"] * 20.0 + wm["dense_fallback"] * 28.0
            wf = wm["unfused_params"] * 20.0
            alg[name] = ((nr * wr + nf * wf) / max(nr + nf, 1), "GB/s", "hbm", PEAK_HBM_GBS)
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
            work = flops_fused_root * n_root_passes_prof / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]
        elif name == "newton_gemm_f32" and flops_f32_root > 0:
            work = flops_f32_root * n_root_passes_prof / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f32"]
        elif name == "newton_gemm_f64" and flops_f64_root > 0:
            work = flops_f64_root * n_root_passes_prof / total
            unit, bound, peak = "TFLOP/s", "mfma", PEAK_TFLOPS["f64"]
        if work is not None and work > 0:
            sec = rec["avg_ms"] / 1e3
            ach = work / sec / (1e12 if unit == "TFLOP/s" else 1e9)
            rec.update({"bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                        "frac": ach / peak})
            if peaks:
                mp = (peaks["copy_gbs"] if unit == "GB/s" else
                      peaks["mfma_f64_tflops"] if peak == PEAK_TFLOPS["f64"] else
                      peaks["mfma_bf16_tflops"] if peak == PEAK_TFLOPS["bf16"] else
                      peaks["mfma_f32_tflops"])
                rec["frac_of_measured_peak"] = ach / mp
        stages[name] = rec

    # counters of this workload's kernels (profiles/traffic.json), valid while
    # the kernel sources are unchanged
    counters = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            tj = json.load(f)
        kh = kernel_hash()
        for fam, ent in tj.get(wl.name, {}).items():
            if isinstance(ent, dict) and ent.get("kernel_hash") == kh:
                counters[fam] = ent
    # MFMA busy as the counter run measured it (SQ_VALU_MFMA_BUSY_CYCLES over
    # the family's own dispatches; that run's launch mix includes the t = 0
    # root pass, so it is not divided by this run's launch times)
    for name, rec in stages.items():
        ent = counters.get(name)
        if ent and ent.get("mfma_busy") is not None and rec.get("bound") == "mfma":
            rec["mfma_busy_counters"] = ent["mfma_busy"]

    # the dominant kernel family by time in the timed region
    roofline = None
    dom = max(stages.items(), key=lambda kv: kv[1]["ms_per_step"]) if stages else None
    if dom and "achieved" in dom[1]:
        ent = counters.get(dom[0])
        roofline = {"kernel": dom[0], "bound": dom[1]["bound"], "achieved": dom[1]["achieved"],
                    "peak": dom[1]["peak"], "unit": dom[1]["unit"], "frac": dom[1]["frac"],
                    "traffic": ent.get("bytes_per_launch") if ent else None,
                    "count": "symmetric results at their upper triangle's flops"}
        for k in ("frac_of_measured_peak", "mfma_busy_counters"):
            if k in dom[1]:
                roofline[k] = dom[1][k]

    root_ms = sum(stages[n]["ms_per_step"] * args.steps for n in
                  ("lanczos_stats", "lanczos_roots", "newton_init", "newton_gemm_f32",
                   "newton_gemm_f64", "newton_commit", "newton_fused_f32", "route_compact",
                   "newton_split_sum")
                  if n in stages)
    inv_root_blocks_per_s = (opt.n_blocks * n_root_passes_prof / (root_ms / 1e3)) if root_ms > 0 else None
    mfma_pct = {k: round(100 * v["frac"], 2) for k, v in stages.items() if v.get("bound") == "mfma"}
    res = {
        "value": value, "ms_per_step": ms_step, "steps_per_s": steps_per_s,
        "newton_tol": tol, "inv_root_blocks_per_s": inv_root_blocks_per_s,
        "root_passes_timed": n_root_passes, "fp64_factor_share_last_pass": n64 / max(len(diag), 1),
        "root_steps_last_pass": {k: ({"mean": sum(v) / len(v), "min": min(v), "max": max(v),
                                           "factors": len(v)} if v else None)
                                      for k, v in iters32.items()},
        "mfma_pct": mfma_pct, "stages": stages, "roofline": roofline, "wall_s_timed": wall,
        "step_ms": step_ms, "n_blocks": opt.n_blocks,
    }
    del opt, params
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2,
                    help="0: 256x512 b128, 1: Transformer-base b128, 2: BERT-large b512 "
                         "(default), 3: ResNet-50 b256, 4: CTR MLP b1024 + sparse tables")
    ap.add_argument("--root-mode", default=None, choices=["f32", "f64", "auto"])
    ap.add_argument("--apply-precision", default=None, choices=["fp32", "bf16x3"],
                    help="products of the apply for blocks above 128 (default: the workload's)")
    ap.add_argument("--newton-tol", type=float, default=None,
                    help="fp32-root convergence tolerance (0: the full iteration count)")
    ap.add_argument("--no-full-count", action="store_true",
                    help="skip the second timed pass at newton_tol 0")
    ap.add_argument("--pool", type=int, default=4, help="distinct gradient sets kept in HBM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the machine-peak probes")
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
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="offline: kernel table of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--counters-summary", default=None, metavar="DIR",
                    help="offline: traffic.json entries and a counters table from the "
                         "rocprofv3 --pmc runs under DIR/pmc_fetch, DIR/pmc_write, DIR/pmc_sq")
    ap.add_argument("--kernel-trace", default=None, metavar="DIR",
                    help="with --counters-summary: kernel-trace run for the durations")
    ap.add_argument("--title", default="", help="with --trace-summary / --counters-summary")
    ap.add_argument("--command", default="", help="with --trace-summary / --counters-summary")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.title, args.command))
        return
    if args.counters_summary:
        print(counters_summary(args.counters_summary, synth.workload(args.workload),
                               args.kernel_trace, args.title, args.command))
        return

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
    if args.apply_precision:
        wl.apply_precision = args.apply_precision
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.time()
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
        del g
    torch.cuda.synchronize()
    print(f"# setup {time.time() - t0:.1f} s: {wl.name}, {wl.n_params / 1e6:.2f}M params, "
          f"{args.pool} gradient sets", file=sys.stderr, flush=True)
    peaks = None
    if not args.no_peaks:
        peaks = S.measure_peaks(dev)
        print(f"# measured peaks: {peaks}", file=sys.stderr, flush=True)

    main_pass = run_pass(wl, args, wl.newton_tol, pool, dev, peaks)
    full = None
    if wl.newton_tol > 0.0 and not args.no_full_count:
        full = run_pass(wl, args, 0.0, pool, dev, peaks)

    out = {
        "metric": METRIC,
        "value": main_pass["value"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_pass["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 gradients/weights; f64 statistics; f32+f64 (routed) roots",
        "data": "synthetic",
        "config": {"workload": wl.name, "params": wl.n_params, "blocks": main_pass["n_blocks"],
                   "block_size": wl.block_size, "root_cadence": wl.cadence,
                   "newton_iters": wl.newton_iters, "newton_tol": wl.newton_tol,
                   "root_mode": wl.root_mode, "apply_precision": wl.apply_precision,
                   "root_parts": args.root_parts, "async_roots": bool(args.async_roots),
                   "large_layer": bool(args.large_layer),
                   "max_precond_dim": wl.max_precond_dim, "parallelism": "single-gpu"},
        "steps_per_s": main_pass["steps_per_s"],
        "inv_root_blocks_per_s": main_pass["inv_root_blocks_per_s"],
        "root_passes_timed": main_pass["root_passes_timed"],
        "fp64_factor_share_last_pass": main_pass["fp64_factor_share_last_pass"],
        "root_steps_last_pass": main_pass["root_steps_last_pass"],
        "mfma_pct": main_pass["mfma_pct"],
        "stages": main_pass["stages"],
        "roofline": main_pass["roofline"],
        "wall_s_timed": main_pass["wall_s_timed"],
        "step_ms": main_pass["step_ms"],
        "peaks_measured": peaks,
        "peaks_published": {"mfma_f32_tflops": PEAK_TFLOPS["f32"],
                            "mfma_f64_tflops": PEAK_TFLOPS["f64"],
                            "mfma_bf16_tflops": PEAK_TFLOPS["bf16"], "hbm_gbs": PEAK_HBM_GBS},
    }
    if full is not None:
        out["full_iteration_count"] = {
            k: full[k] for k in ("value", "ms_per_step", "steps_per_s", "newton_tol",
                                 "inv_root_blocks_per_s", "fp64_factor_share_last_pass",
                                 "root_steps_last_pass", "roofline", "mfma_pct")}
        out["full_iteration_count"]["stages_ms_per_step"] = {
            k: v["ms_per_step"] for k, v in full["stages"].items()}
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle) ...", file=sys.stderr, flush=True)
        cb = cpu_baseline(wl, default_cpu_sample(wl))
        cb["gpu_over_cpu"] = main_pass["value"] / cb["value"]
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------ offline summaries
def _csv_rows(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name):
    """Kernel name without its argument list and return type."""
    name = name.replace("(anonymous namespace)::", "").replace("shampoo::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i].strip()
    return name.strip()


def trace_summary(d, title, command):
    rows = _csv_rows(os.path.join(d, "**", "*kernel_stats.csv"))
    if not rows:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    lines = [f"# rocprofv3 kernel statistics: {title}", "",
             "Command (run from /tmp; R = repository root, OUT = an output directory):", "",
             "```", command, "```", "",
             "| kernel | calls | total ms | average us | % |", "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    return "\n".join(lines)


# kernel -> bench family (one kernel per family here: its per-dispatch
# average is the family's per-launch figure); precision of its MFMA work
FAMILY_OF = [
    ("k_step128", "step_fused", "f64"),
    ("k_gram128", "stats_gram128", "f64"),
    ("k_apply128", "apply_fused", "f32"),
    ("k_newton128", "newton_fused_f32", "f32"),
    ("k_gemm<double, float, float, 2, true, false", "stats_gram_f64", "f64"),
    ("k_gemm<float, float, float, 1, false, false, 1>", "apply_gemm_t", "f32"),
    ("k_gemm<float, float, float, 1, false, false, 2>", "apply_gemm_d", "f32"),
    ("k_gemm_nt3<true", "apply_gemm_t", "bf16"),
    ("k_gemm_nt3<false", "apply_gemm_d", "bf16"),
    ("k_gemm<float, float, float, 3, false, false", "newton_gemm_f32", "f32"),
    ("k_gemm<double, double, double, 2", "newton_gemm_f64", "f64"),
    ("k_adagrad_norm", "adagrad_norm", None),
    ("k_update", "update", None),
    ("k_sparse_rows", "sparse_rows", None),
    ("k_lanczos_big<double", "lanczos_stats", None),
    ("k_lanczos_big<float", "lanczos_roots", None),
]


def _family(kname):
    for prefix, fam, prec in FAMILY_OF:
        if kname.startswith(prefix):
            return fam, prec
    return None, None


def _per_kernel_counters(d):
    """{kernel: {counter: mean per dispatch}, ...}, dispatches per kernel."""
    rows = _csv_rows(os.path.join(d, "**", "*counter_collection.csv"))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    acc = {}
    for r in rows:
        k = _short(r["Kernel_Name"])
        disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})
        cell = acc[k][r["Counter_Name"]]
        cell[disp] = cell.get(disp, 0.0) + float(r["Counter_Value"])
    out, ndisp = {}, {}
    for k, cs in acc.items():
        out[k] = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        ndisp[k] = max(len(v) for v in cs.values())
    return out, ndisp


def counters_summary(d, wl, trace_dir, title, command):
    fetch, nf = _per_kernel_counters(os.path.join(d, "pmc_fetch"))
    write, _ = _per_kernel_counters(os.path.join(d, "pmc_write"))
    sq = {}
    if os.path.isdir(os.path.join(d, "pmc_sq")):
        sq, _ = _per_kernel_counters(os.path.join(d, "pmc_sq"))
    copy = [k for k in fetch if k.startswith("k_peak_copy")]
    if not copy:
        raise SystemExit("no k_peak_copy dispatch to scale FETCH_SIZE / WRITE_SIZE by")
    # the probe's copy reads and writes half of its 2 GiB scratch
    copy_bytes = float(1 << 30)
    fs = copy_bytes / (fetch[copy[0]]["FETCH_SIZE"] * 1024.0)
    ws = copy_bytes / (write[copy[0]]["WRITE_SIZE"] * 1024.0)
    dur = {}
    if trace_dir:
        for r in _csv_rows(os.path.join(trace_dir, "**", "*kernel_stats.csv")):
            dur[_short(r["Name"])] = float(r["AverageNs"]) / 1e9
    kh = kernel_hash()
    tj = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            tj = json.load(f)
    ent_wl = {}
    lines = [f"# rocprofv3 counters: {title}", "",
             "Counter runs, each its own process (from /tmp; R = repository root, OUT = an "
             "output directory):", "", "```", command, "```", "",
             f"Values are per dispatch, summed over the counter's instances, averaged over the "
             f"dispatches. The peak probe's copy kernel (k_peak_copy) reads and writes "
             f"{copy_bytes / 2**30:.0f} GiB: FETCH_SIZE reads {fetch[copy[0]]['FETCH_SIZE']:.0f} "
             f"KiB and WRITE_SIZE {write[copy[0]]['WRITE_SIZE']:.0f} KiB for it, so HBM bytes = "
             f"{fs:.3f} x FETCH_SIZE + {ws:.3f} x WRITE_SIZE (KiB x 1024). Executed flops = "
             f"SQ_INSTS_VALU_MFMA_MOPS_* x 512. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             f"(1024 SIMDs x GRBM_GUI_ACTIVE / 8).", "",
             "| kernel | family | dispatches | HBM MB | executed GFLOP | MFMA busy | "
             "avg us (trace) | HBM GB/s | executed TFLOP/s |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for k in sorted(fetch, key=lambda k: -fetch[k].get("FETCH_SIZE", 0)):
        fam, prec = _family(k)
        if fam is None and not k.startswith("k_peak"):
            continue
        fb = fetch[k].get("FETCH_SIZE", 0.0) * 1024.0 * fs
        wb = write.get(k, {}).get("WRITE_SIZE", 0.0) * 1024.0 * ws
        c = sq.get(k, {})
        mops = (c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F64", 0.0) +
                c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
        exe = mops * 512.0
        busy = None
        if c.get("GRBM_GUI_ACTIVE"):
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024.0 * c["GRBM_GUI_ACTIVE"] / 8.0)
        t = dur.get(k)
        lines.append(f"| {k} | {fam or 'probe'} | {nf[k]} | {(fb + wb) / 1e6:.1f} | {exe / 1e9:.2f} | "
                     f"{'' if busy is None else f'{100 * busy:.1f}%'} | "
                     f"{'' if t is None else f'{t * 1e6:.1f}'} | "
                     f"{'' if t is None else f'{(fb + wb) / t / 1e9:.0f}'} | "
                     f"{'' if t is None or not exe else f'{exe / t / 1e12:.1f}'} |")
        if fam is None or fam in ent_wl:
            continue
        ent_wl[fam] = {"kernel": k, "kernel_hash": kh, "dispatches": nf[k],
                       "fetch_kib_per_dispatch": fetch[k].get("FETCH_SIZE", 0.0),
                       "write_kib_per_dispatch": write.get(k, {}).get("WRITE_SIZE", 0.0),
                       "fetch_scale": fs, "write_scale": ws, "bytes_per_launch": fb + wb,
                       "precision": prec, "executed_flops_per_launch": exe or None,
                       "mfma_busy": busy}
    tj[wl.name] = ent_wl
    tj["_note"] = ("per workload and kernel family: HBM bytes per launch from rocprofv3 --pmc "
                   "FETCH_SIZE and WRITE_SIZE (separate runs) scaled by what they read for a "
                   "plain copy of known size, executed MFMA flops from SQ_INSTS_VALU_MFMA_MOPS; "
                   "valid while kernel_hash matches the kernel sources")
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(tj, f, indent=1, sort_keys=True)
    return "\n".join(lines)


if __name__ == "__main__":
    main()
