"""Host tests (no GPU) of the measurement bookkeeping in bench.py.

Every roofline fraction the bench line reports divides an algorithmic work
count by a measured time, so the counts are checked here against what they
claim to count:
- a product with a symmetric result counted on its upper triangle, against a
  brute-force tally;
- the flops of one inverse root, against an explicit coupled-Newton run in
  NumPy that counts the products it forms (and checks that each is symmetric,
  which is what licenses the triangle count, and that the run reaches
  A^(-1/p));
- the per-launch work of the statistics and the apply, against the block
  shapes of the oracle's own partition of every workload;
- the HBM bytes a counter summary writes, against FETCH_SIZE / WRITE_SIZE
  scaled by the copy kernel of known size (synthetic counter files).
"""
import csv
import json
import math
import os

import numpy as np
import pytest

import bench
from oracle import shampoo_oracle as O
from second_order_optimizer_amd import shampoo as S
from second_order_optimizer_amd import synth


@pytest.mark.parametrize("n,k", [(1, 1), (3, 5), (16, 7), (130, 64)])
def test_symmetric_product_counts_its_upper_triangle(n, k):
    # 2 k flops (k multiply-adds) for every entry (i, j) with i <= j
    tally = 0
    for i in range(n):
        for _ in range(i, n):
            tally += 2 * k
    assert bench.sym(n, k) == tally


def counted_coupled_newton(A, p, iters, batched):
    """The coupled iteration X <- X T, M <- T^p M with T = ((p+1) I - M) / p,
    started from X_0 = z^(1/p) I, M_0 = z A.  Returns (X, flops) where every
    matrix product the kernels form is counted at its upper triangle and the
    forms the kernels skip are done without a product: X_0 T is a row
    scaling (X_0 is diagonal), and a batched chain's last step forms X only."""
    n = A.shape[0]
    lam = np.linalg.eigvalsh(A)[-1]
    z = (p + 1) / (2.0 * lam)
    X = z ** (1.0 / p) * np.eye(n)
    M = z * A
    flops = 0.0

    def product(P, Q):
        nonlocal flops
        R = P @ Q
        # every product here is a polynomial in A: symmetric
        assert np.allclose(R, R.T, rtol=1e-10, atol=1e-12 * np.abs(R).max())
        flops += n * (n + 1) * n
        return R

    for it in range(iters):
        T = ((p + 1) * np.eye(n) - M) / p
        X = np.diag(X)[:, None] * T if it == 0 else product(X, T)
        if batched and it == iters - 1:
            break
        Tp = T
        for _ in range(int(round(math.log2(p)))):
            Tp = product(Tp, Tp)
        M = product(Tp, M)
    return X, flops


@pytest.mark.parametrize("p", [1, 2, 4, 8])
@pytest.mark.parametrize("iters", [1, 2, 7, 20])
@pytest.mark.parametrize("batched", [False, True])
def test_newton_flops_match_a_counted_run(p, iters, batched):
    rng = np.random.default_rng(p * 100 + iters)
    n = 12
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    A = (Q * np.geomspace(1.0, 1e-2, n)) @ Q.T
    A = 0.5 * (A + A.T)
    _, flops = counted_coupled_newton(A, p, iters, batched)
    assert bench.newton_flops(n, p, iters, batched) == flops


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_counted_run_is_the_inverse_root(p):
    rng = np.random.default_rng(7 + p)
    n = 10
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = np.geomspace(1.0, 1e-2, n)
    A = (Q * lam) @ Q.T
    A = 0.5 * (A + A.T)
    X, _ = counted_coupled_newton(A, p, 40, batched=False)
    want = (Q * lam ** (-1.0 / p)) @ Q.T
    assert np.linalg.norm(X - want) / np.linalg.norm(want) < 1e-10


@pytest.mark.parametrize("wid", range(5))
def test_work_model_matches_the_oracle_partition(wid):
    wl = synth.workload(wid)
    cfg = S.make_config(wl.block_size, max_precond_dim=wl.max_precond_dim, root_mode=wl.root_mode)
    plan = S.Plan([(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in wl.tensors], cfg)
    wm = bench.work_model(wl, plan)
    ocfg = O.OracleConfig(block_size=wl.block_size, max_precond_dim=wl.max_precond_dim)
    gram = apply = 0.0
    shampoo_params = fallback = 0
    for t in wl.tensors:
        if t.kind != "dense":
            continue
        if not O.uses_shampoo(t.rows, t.cols, ocfg):
            fallback += t.rows * t.cols
            continue
        for _, m, _, n in O.blocks(t.rows, t.cols, wl.block_size):
            gram += bench.sym(m, n) + bench.sym(n, m)        # G G^T and G^T G
            apply += 2.0 * (m * n * n + m * m * n)            # (G P_R), then P_L (G P_R)
            shampoo_params += m * n
    plan.close()
    assert wm["gram"] == gram
    assert wm["apply_small"] + wm["apply_t_big"] + wm["apply_d_big"] == apply
    assert wm["shampoo_params"] == shampoo_params
    assert wm["dense_fallback"] == fallback


def _write_counters(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(traffic))
    d = tmp_path / "run"
    copy, upd = "void shampoo::k_peak_copy<4, false>(float4 const*, float4*, long)", \
        "shampoo::k_update(shampoo::RowChunk const*, unsigned long const*, int, float*, float const*)"
    # the copy reads and writes 1 GiB: here FETCH_SIZE reads half of that
    # (two sectors per 64 B line) and WRITE_SIZE all of it, in KiB, summed
    # over two counter instances; k_update has two dispatches
    fetch = [{"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
             for v in (131072, 131072)]
    fetch += [{"Dispatch_Id": i, "Kernel_Name": upd, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
              for i, v in ((2, 1000), (2, 1000), (3, 3000), (3, 3000))]
    write = [{"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": v}
             for v in (524288, 524288)]
    write += [{"Dispatch_Id": i, "Kernel_Name": upd, "Counter_Name": "WRITE_SIZE", "Counter_Value": v}
              for i, v in ((2, 500), (2, 500), (3, 500), (3, 500))]
    _write_counters(str(d / "pmc_fetch" / "x" / "run_counter_collection.csv"), fetch)
    _write_counters(str(d / "pmc_write" / "x" / "run_counter_collection.csv"), write)
    text = bench.counters_summary(str(d), synth.workload(1), None, "synthetic", "(none)")
    ent = json.loads(traffic.read_text())[synth.workload(1).name]["update"]
    fs = (1 << 30) / (262144 * 1024.0)      # bytes per FETCH_SIZE byte: 4
    ws = (1 << 30) / (1048576 * 1024.0)     # bytes per WRITE_SIZE byte: 1
    assert ent["fetch_scale"] == fs and ent["write_scale"] == ws
    assert ent["dispatches"] == 2
    # per dispatch: fetch (2000 + 6000) / 2 KiB, write (1000 + 1000) / 2 KiB
    assert ent["bytes_per_launch"] == 4000 * 1024.0 * fs + 1000 * 1024.0 * ws
    assert ent["kernel_hash"] == bench.kernel_hash()
    assert "k_update" in text
