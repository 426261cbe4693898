"""Host-side tests (no GPU): the C-ABI library loads and exports every symbol
include/shampoo.h declares, the struct layouts agree, and the planner's block
partition and state layout are right for every workload."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import shampoo_oracle as O
from second_order_optimizer_amd import shampoo as S
from second_order_optimizer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shampoo.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(shampoo_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = S.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(S.SIGNATURES), set(names) ^ set(S.SIGNATURES)


def test_struct_sizes_match_header():
    # sizes the C compiler gives (natural alignment, x86-64 / amdgcn agree)
    assert ctypes.sizeof(S.TensorDesc) == 24
    assert ctypes.sizeof(S.Config) == 96
    assert ctypes.sizeof(S.SparseRows) == 24
    assert ctypes.sizeof(S.FactorDiag) == 56
    assert ctypes.sizeof(S.BlockLayout) == 88
    assert ctypes.sizeof(S.KernelTime) == 48
    assert ctypes.sizeof(S.Peaks) == 40


def test_strerror_and_argument_errors():
    L = S.lib()
    assert L.shampoo_strerror(0) == b"ok"
    assert L.shampoo_strerror(-1) == b"invalid argument"
    cfg = S.make_config(128)
    h = S._P()
    descs = (S.TensorDesc * 1)(S.TensorDesc(4, 4, 0, 0))
    assert L.shampoo_create(None, 1, descs, ctypes.byref(h)) == -1
    assert L.shampoo_create(ctypes.byref(cfg), 0, descs, ctypes.byref(h)) == -1
    bad = (S.TensorDesc * 1)(S.TensorDesc(0, 4, 0, 0))
    assert L.shampoo_create(ctypes.byref(cfg), 1, bad, ctypes.byref(h)) == -1
    badk = (S.TensorDesc * 1)(S.TensorDesc(4, 4, 7, 0))
    assert L.shampoo_create(ctypes.byref(cfg), 1, badk, ctypes.byref(h)) == -1
    c = S.make_config(128, root_p=2, apply_precision="bf16x3")
    assert L.shampoo_create(ctypes.byref(c), 1, descs, ctypes.byref(h)) == -5
    for field, val, rc in (("root_p", 3, -5), ("root_p", 16, -5), ("beta2", 0.0, -1),
                           ("beta2", 1.5, -1), ("block_size", 0, -1), ("newton_iters", 0, -1),
                           ("root_mode", 5, -1), ("eps_rel", -1.0, -1), ("newton_tol", -1e-3, -1),
                           ("apply_precision", 2, -1), ("apply_precision", -1, -1),
                           ("reserved", 1, -1),
                           ("newton_tol", 1.0, -1), ("newton_tol", float("nan"), -1)):
        c = S.make_config(128)
        setattr(c, field, val)
        assert L.shampoo_create(ctypes.byref(c), 1, descs, ctypes.byref(h)) == rc, field
    # a dimension above the supported factor size is rejected up front
    big = (S.TensorDesc * 1)(S.TensorDesc(2048, 64, 0, 0))
    assert L.shampoo_create(ctypes.byref(S.make_config(2048)), 1, big, ctypes.byref(h)) == -5
    # calls on an unbound handle
    p = S.Plan([(8, 8, 0)], cfg)
    arr = (S._P * 1)()
    assert L.shampoo_update_stats(p.h, arr, None, None) == -2
    assert L.shampoo_compute_inverse_roots(p.h, None) == -2
    assert L.shampoo_compute_inverse_roots_noalloc(p.h, None) == -2
    assert L.shampoo_compute_inverse_roots_noalloc(None, None) == -1
    assert L.shampoo_step(p.h, arr, arr, None, S.ROOTS_NONE, None) == -2
    assert L.shampoo_step(p.h, None, arr, None, S.ROOTS_ALL, None) == -1
    # a part index needs a plan with root_parts >= 2
    assert L.shampoo_step(p.h, arr, arr, None, 0, None) == -1
    assert L.shampoo_compute_inverse_roots_part(p.h, 0, None) == -1
    p.close()
    p = S.Plan([(8, 8, 0), (8, 8, 0), (8, 8, 0)], S.make_config(4, root_parts=3))
    assert L.shampoo_compute_inverse_roots_part(p.h, 3, None) == -1
    assert L.shampoo_compute_inverse_roots_part(p.h, -1, None) == -1
    assert L.shampoo_compute_inverse_roots_part(p.h, 2, None) == -2      # unbound
    assert L.shampoo_step(p.h, arr, arr, None, 3, None) == -1
    c = S.make_config(4)
    c.root_parts = -1
    assert L.shampoo_create(ctypes.byref(c), 1, descs, ctypes.byref(h)) == -1
    assert L.shampoo_update_stats(p.h, None, None, None) == -1
    p.close()
    # the peak probe checks its scratch before touching the device
    pk = S.Peaks()
    assert L.shampoo_measure_peaks(None, S._P(256), 1 << 22, None) == -1
    assert L.shampoo_measure_peaks(ctypes.byref(pk), None, 1 << 22, None) == -1
    assert L.shampoo_measure_peaks(ctypes.byref(pk), S._P(257), 1 << 22, None) == -1
    assert L.shampoo_measure_peaks(ctypes.byref(pk), S._P(256), 1 << 20, None) == -1


EXPECTED_BLOCKS = {0: 8, 1: 2688, 2: 1152, 3: 422, 4: 3}


@pytest.mark.parametrize("wid", range(5))
def test_planner_matches_oracle_partition(wid):
    wl = synth.workload(wid)
    cfg = S.make_config(wl.block_size, max_precond_dim=wl.max_precond_dim, root_mode=wl.root_mode)
    p = S.Plan([(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in wl.tensors], cfg)
    assert p.n_blocks == EXPECTED_BLOCKS[wid]
    assert p.n_factors == 2 * p.n_blocks
    ocfg = O.OracleConfig(block_size=wl.block_size, max_precond_dim=wl.max_precond_dim)
    b = 0
    for ti, t in enumerate(wl.tensors):
        a_off, m_off, fb, nb = p.tensor(ti)
        assert a_off >= 0 and a_off % 256 == 0
        if t.kind == "sparse":
            assert m_off == -1 and nb == 0
            continue
        assert m_off % 256 == 0
        if not O.uses_shampoo(t.rows, t.cols, ocfg):
            assert nb == 0
            continue
        assert fb == b
        ob = O.blocks(t.rows, t.cols, wl.block_size)
        assert nb == len(ob)
        for (r0, mb, c0, ncol) in ob:
            bl = p.block(b)
            assert (bl.tensor, bl.row0, bl.rows, bl.col0, bl.cols) == (ti, r0, mb, c0, ncol)
            assert bl.ld_l >= mb and bl.ld_r >= ncol and bl.ld_l % 32 == 0
            assert (bl.factor_l, bl.factor_r) == (2 * b, 2 * b + 1)
            b += 1
    assert b == p.n_blocks
    p.close()


@pytest.mark.parametrize("large_layer", [0, 1])
def test_state_regions_do_not_overlap(large_layer):
    """Every byte range the layout hands out is disjoint and inside the state
    (with large_layer, the 5000 x 64 tensor and the sparse table are
    one-sided blocks)."""
    T = synth.TensorSpec
    wl = synth.Workload(90, "mix", [T("a", 300, 200), T("b", 64, 147), T("e", 5000, 64),
                                   T("s", 1000, 32, kind="sparse")], 128, max_precond_dim=4096)
    cfg = S.make_config(128, root_mode="auto", max_precond_dim=4096, large_layer=large_layer)
    p = S.Plan([(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in wl.tensors], cfg)
    spans = []
    for i in range(p.n_blocks):
        bl = p.block(i)
        spans += [(bl.off_l, bl.ld_l ** 2 * 8), (bl.off_r, bl.ld_r ** 2 * 8),
                  (bl.off_pl, bl.ld_l ** 2 * 4), (bl.off_pr, bl.ld_r ** 2 * 4),
                  (bl.off_pl64, bl.ld_l ** 2 * 8), (bl.off_pr64, bl.ld_r ** 2 * 8)]
    # large_layer: the 5000 x 64 tensor and the sparse table
    assert sum(p.block(i).one_sided for i in range(p.n_blocks)) == 2 * large_layer
    spans = [(o, n) for o, n in spans if o >= 0]
    for ti, t in enumerate(wl.tensors):
        a_off, m_off, _, _ = p.tensor(ti)
        spans.append((a_off, t.numel * 4))
        if m_off >= 0:
            spans.append((m_off, t.numel * 4))
    spans.sort()
    for (o1, n1), (o2, _) in zip(spans, spans[1:]):
        assert o1 + n1 <= o2
    assert spans[-1][0] + spans[-1][1] <= p.state_bytes
    p.close()


def test_one_sided_plan_numbering_and_layout():
    """large_layer = 1 (Lemma 1): a dense tensor with one dimension above
    max_precond_dim gets one block with one factor for the side that fits,
    numbered after every Lemma-2 block, as the oracle numbers it for the root
    schedule; a tensor with both dimensions too large stays diagonal Adagrad."""
    T = synth.TensorSpec
    tensors = [T("tall", 3000, 96), T("a", 250, 200), T("wide", 100, 5000), T("huge", 900, 900),
               T("s", 1000, 32, kind="sparse"), T("b", 64, 147)]
    shapes = [(t.rows, t.cols, 0 if t.kind == "dense" else 1) for t in tensors]
    cfg = S.make_config(128, max_precond_dim=256, root_mode="auto", large_layer=1)
    ocfg = O.OracleConfig(block_size=128, max_precond_dim=256, large_layer=1)
    orc = O.ShampooOracle(ocfg, [(t.rows, t.cols, t.kind) for t in tensors],
                          [np.zeros((t.rows, t.cols), np.float32) for t in tensors])
    p = S.Plan(shapes, cfg)
    n_reg = sum(len(v) for v in orc.blocks.values())
    assert n_reg == 2 * 2 + 1 * 2   # a: 2x2 blocks, b: 1x2
    assert p.n_blocks == n_reg + 3
    assert p.n_factors == 2 * n_reg + 3
    expect = {0: "R", 2: "L", 4: "R"}   # 4: the sparse table
    for ti, side in expect.items():
        idx, st = orc.one_sided[ti]
        assert st.side == side
        _, _, fb, nb = p.tensor(ti)
        assert (fb, nb) == (idx, 1)
        bl = p.block(fb)
        t = tensors[ti]
        assert bl.one_sided == 1
        assert (bl.tensor, bl.row0, bl.col0, bl.rows, bl.cols) == (ti, 0, 0, t.rows, t.cols)
        if side == "R":
            assert bl.factor_l == -1 and bl.off_l == -1 and bl.off_pl == -1 and bl.ld_l == 0
            assert bl.factor_r == 2 * n_reg + (idx - n_reg)
            assert bl.ld_r == (96 if ti == 0 else 32)
        else:
            assert bl.factor_r == -1 and bl.off_r == -1 and bl.off_pr == -1 and bl.ld_r == 0
            assert bl.factor_l == 2 * n_reg + (idx - n_reg) and bl.ld_l == 128
    assert p.tensor(3)[3] == 0 and 3 not in orc.one_sided   # both sides too large
    # regular blocks keep their numbering and factor ids
    for b in range(n_reg):
        bl = p.block(b)
        assert bl.one_sided == 0 and (bl.factor_l, bl.factor_r) == (2 * b, 2 * b + 1)
    p.close()
    # large_layer off: the same tensors plan no one-sided block
    p = S.Plan(shapes, S.make_config(128, max_precond_dim=256))
    assert p.n_blocks == n_reg and p.tensor(0)[3] == 0
    p.close()


def test_one_sided_config_errors():
    L = S.lib()
    h = S._P()
    descs = (S.TensorDesc * 1)(S.TensorDesc(3000, 64, 0, 0))
    c = S.make_config(64, max_precond_dim=128, large_layer=2)
    assert L.shampoo_create(ctypes.byref(c), 1, descs, ctypes.byref(h)) == -1
    # the one factor takes the exponent -2/root_p: root_p must be even
    c = S.make_config(64, max_precond_dim=128, large_layer=1, root_p=1)
    assert L.shampoo_create(ctypes.byref(c), 1, descs, ctypes.byref(h)) == -5
    # a one-sided factor above the supported dimension
    big = (S.TensorDesc * 1)(S.TensorDesc(5000, 2048, 0, 0))
    c = S.make_config(64, max_precond_dim=4096, large_layer=1)
    assert L.shampoo_create(ctypes.byref(c), 1, big, ctypes.byref(h)) == -5


def _newton_split_bytes(nf, ld, esz):
    """Partial-product scratch of the split-K stages of a Newton chunk of nf
    factors: a stage of fewer than 256 upper 128-tiles is split over k into
    the largest power of two (up to 8) of parts that keeps its tiles within
    1024 and each part a multiple of 32 and at least 64 deep; stage 0 has two
    products per factor, the others one."""
    t1 = -(-ld // 128)
    ut = t1 * (t1 + 1) // 2
    best = 0
    for tasks in (2 * nf, nf):
        tiles, s = tasks * ut, 1
        if tiles < 256:
            while s < 8 and tiles * s * 2 <= 1024 and ld % (64 * s) == 0 and ld // (2 * s) >= 64:
                s *= 2
        if s > 1:
            best = max(best, tasks * s * ld * ld * esz)
    return best


def test_newton_scratch_budget_from_environment(monkeypatch):
    """The batched Newton scratch (six ld x ld matrices per factor of a chunk)
    follows SHAMPOO_NEWTON_SCRATCH_BYTES, read at create: 8 factors of 256 in
    AUTO mode take 8 slots per precision by default, and with a budget of
    3 MiB two fp32 slots and one fp64 slot (more chunks, more launch tables);
    the partial products of split-K stages shrink with the chunks."""
    shapes = [(512, 512, 0)]
    cfg = S.make_config(256, root_mode="auto")
    p = S.Plan(shapes, cfg)
    full = p.state_bytes
    p.close()
    monkeypatch.setenv("SHAMPOO_NEWTON_SCRATCH_BYTES", str(3 << 20))
    p = S.Plan(shapes, cfg)
    small = p.state_bytes
    p.close()
    per32, per64 = 6 * 256 * 256 * 4, 6 * 256 * 256 * 8
    saved = (8 - 2) * per32 + (8 - 1) * per64
    saved += _newton_split_bytes(8, 256, 4) - _newton_split_bytes(2, 256, 4)
    saved += _newton_split_bytes(8, 256, 8) - _newton_split_bytes(1, 256, 8)
    # the launch tables of the extra chunks (tens of KB) take some of it back
    assert 0 <= saved - (full - small) < 256 << 10


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_newton_step_count_model(p):
    """The step-count model the GPU test holds the fused root's convergence
    exit to: a dense fp64 coupled Newton iteration (Guo & Higham: X_0 =
    z^(1/p) I, M_0 = z A, T = ((p+1) I - M) / p, X <- X T, M <- T^p M) on an
    SPD matrix with a log-spaced spectrum has, step by step, the Frobenius
    norm ||M_k - I||_F the scalar eigenvalue map gives (the norm is unitarily
    invariant), so it stops at the model's step; the root it leaves is
    within the bound the exit rule implies."""
    from harness import newton_steps
    rng = np.random.default_rng(7)
    for kappa in (10.0, 1e3, 1e5):
        n = 24
        lam = np.logspace(-np.log10(kappa), 0.0, n)
        q, _ = np.linalg.qr(rng.standard_normal((n, n)))
        A = (q * lam) @ q.T
        z = (p + 1) / 2.0
        X, M = z ** (1.0 / p) * np.eye(n), z * A
        m = z * lam
        stop, dense_steps = False, None
        for k in range(1, 41):
            T = ((p + 1) * np.eye(n) - M) / p
            X = X @ T
            M = np.linalg.matrix_power(T, p) @ M
            m = m * ((p + 1 - m) / p) ** p
            d_dense = np.linalg.norm(M - np.eye(n))
            d_map = np.sqrt(np.sum((m - 1.0) ** 2))
            assert abs(d_dense - d_map) <= 1e-9 * max(1.0, d_map), (p, kappa, k, d_dense, d_map)
            if stop:
                dense_steps = k
                break
            stop = d_dense < 1e-3
        assert dense_steps == newton_steps(lam, 1.0, 0.0, p, 1e-3, 40), (p, kappa)
        # one step after ||M - I||_F < 1e-3 the spectral error is at most about
        # (p+1)/(2p) 1e-6, and the root's relative error about that over p
        # the stopped iterate is the root to about the map's last residual
        ref = (q * lam ** (-1.0 / p)) @ q.T
        assert np.linalg.norm(X - ref) / np.linalg.norm(ref) < 2e-6, (p, kappa)
    if p == 4:
        assert [newton_steps(np.logspace(-e, 0, 50), 1.0, 0.0, 4, 1e-3, 40)
                for e in (1, 3, 5)] == [6, 11, 16]


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_scaled_newton_model(p):
    """The scaled steps the batched chains take with a convergence exit: a
    dense fp64 coupled Newton iteration that scales M by mu_k and X by
    mu_k^(1/p) before each step keeps M_k = X_k^p A, its ||M_k - I||_F follows
    the scalar map with the same scalings step by step, and after the
    schedule's count (its interval bound within 1e-3 of 1, plus two steps) the
    root is exact to rounding, also at the worst conditioning the eps floor
    allows (an eigenvalue of S at 0: kappa = 1 + 1/eps_rel).  The count is
    well below the unscaled iteration's, and the bound holds: every scaled
    eigenvalue stays inside the interval."""
    from harness import newton_scaling
    eps_rel = 1e-6
    n_full = {1: 26, 2: 23, 4: 20, 8: 20}[p]
    mus, conv = newton_scaling(p, eps_rel, n_full)
    assert conv < n_full and all(m >= 1.0 for m in mus)
    assert conv == {1: 19, 2: 14, 4: 11, 8: 10}[p], conv
    rng = np.random.default_rng(11)
    n = 32
    for spec in ("floor", "log3", "flat"):
        if spec == "floor":
            lam_s = np.concatenate([[0.0], np.logspace(-6, 0, n - 1)])
        elif spec == "log3":
            lam_s = np.logspace(-3, 0, n)
        else:
            lam_s = np.full(n, 0.5)
        q, _ = np.linalg.qr(rng.standard_normal((n, n)))
        lmax = lam_s.max()
        eps = eps_rel * lmax
        lam = lam_s + eps
        A = (q * lam) @ q.T
        z = (p + 1) / (2.0 * lmax * (1 + eps_rel))
        X, M = z ** (1.0 / p) * np.eye(n), z * A
        m = z * lam
        for k in range(conv):
            mu = mus[k]
            T = ((p + 1) * np.eye(n) - mu * M) / p
            X = mu ** (1.0 / p) * X @ T
            M = np.linalg.matrix_power(T, p) @ (mu * M)
            m = mu * m * ((p + 1 - mu * m) / p) ** p
            assert abs(np.linalg.norm(M - np.eye(n)) - np.sqrt(np.sum((m - 1) ** 2))) <= \
                1e-9 * max(1.0, np.sqrt(np.sum((m - 1) ** 2))), (p, spec, k)
            assert np.all(m > 0) and np.all(m < p + 1), (p, spec, k)
        ref = (q * lam ** (-1.0 / p)) @ q.T
        err = np.linalg.norm(X - ref) / np.linalg.norm(ref)
        assert err < 1e-9, (p, spec, err)   # fp64 rounding: up to about kappa^(1/p) u
