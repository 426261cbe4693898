"""Seeded synthetic workloads for the Shampoo optimizer step.

This module only draws inputs: parameter shapes, initial weights and per-step
gradients (dense matrices and sparse embedding rows).  It holds none of the
optimizer's arithmetic, so the fp64 oracle and the GPU library can both be fed
from it without sharing any part of the method.

Shapes stand in for the workloads named in "Scalable Second Order Optimization
for Deep Learning" (abstract page; Shampoo-at-scale podcast transcript, cue 18):
a Transformer for WMT'14 en->fr, BERT-Large, ResNet-50 on ImageNet and a
click-through-rate model on Criteo.  None of those datasets is used: gradients
are synthetic with the value distributions described per workload below.

Every random draw comes from ``numpy.random.SeedSequence`` entropy tuples
(root seed, workload id, tensor index[, step]), so any tensor of any step can
be regenerated on its own, in any order.  Gradients are drawn in fp64 and
rounded to fp32 once.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

ROOT_SEED = 20260101


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    kind: str = "dense"          # "dense" or "sparse" (row-sparse embedding table)
    grad: str = "lowrank"        # "lowrank", "student_t", "sparse_rows"
    rank: int = 0                # low-rank part's rank (0: min(rows, cols))
    noise: float = 0.01          # noise std (lowrank); <0: per-matrix 10^U(-4,-1)

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass
class Workload:
    wid: int
    name: str
    tensors: List[TensorSpec]
    block_size: int
    max_precond_dim: int = 0        # 0: no limit; larger dims use diagonal Adagrad
    root_mode: str = "auto"         # "f32", "f64" or "auto" (fp64 when kappa > threshold)
    fp64_cond_threshold: float = 1e5
    cadence: int = 1                # inverse roots recomputed when step % cadence == 0
    newton_iters: int = 20
    newton_tol: float = 1e-3        # fused roots stop one step after ||M - I||_F < this
    apply_precision: str = "bf16x3" # products of the apply above 128: "fp32" or "bf16x3"
    root_p: int = 4
    beta1: float = 0.9
    beta2: float = 0.999
    lr: float = 1e-3
    eps_rel: float = 1e-6
    graft_eps: float = 1e-10
    steps: int = 10
    sparse_frac: float = 0.05
    zipf_s: float = 1.1
    notes: str = ""

    @property
    def n_params(self) -> int:
        return sum(t.numel for t in self.tensors)

    def dense_tensors(self) -> List[TensorSpec]:
        return [t for t in self.tensors if t.kind == "dense"]


def _transformer_base() -> List[TensorSpec]:
    d, f = 512, 2048
    ts: List[TensorSpec] = []
    for i in range(6):
        for p in "qkvo":
            ts.append(TensorSpec(f"enc{i}.attn.{p}", d, d))
        ts.append(TensorSpec(f"enc{i}.ffn1", d, f))
        ts.append(TensorSpec(f"enc{i}.ffn2", f, d))
    for i in range(6):
        for a in ("self", "cross"):
            for p in "qkvo":
                ts.append(TensorSpec(f"dec{i}.{a}.{p}", d, d))
        ts.append(TensorSpec(f"dec{i}.ffn1", d, f))
        ts.append(TensorSpec(f"dec{i}.ffn2", f, d))
    ts.append(TensorSpec("embedding", 32000, d))
    return ts


def _bert_large() -> List[TensorSpec]:
    h, f = 1024, 4096
    ts: List[TensorSpec] = []
    for i in range(24):
        for p in "qkvo":
            ts.append(TensorSpec(f"layer{i}.attn.{p}", h, h, rank=64, noise=-1.0))
        ts.append(TensorSpec(f"layer{i}.ffn1", h, f, rank=64, noise=-1.0))
        ts.append(TensorSpec(f"layer{i}.ffn2", f, h, rank=64, noise=-1.0))
    return ts


def _resnet50() -> List[TensorSpec]:
    # conv weights as (out_channels) x (in_channels * k * k), plus the FC layer
    shapes: List[Tuple[str, int, int]] = [("conv1", 64, 147)]
    stages = [  # (name, width, out, first-block in, blocks)
        ("layer1", 64, 256, 64, 3),
        ("layer2", 128, 512, 256, 4),
        ("layer3", 256, 1024, 512, 6),
        ("layer4", 512, 2048, 1024, 3),
    ]
    for name, w, out, first_in, nblk in stages:
        for b in range(nblk):
            cin = first_in if b == 0 else out
            shapes.append((f"{name}.{b}.conv1", w, cin))
            shapes.append((f"{name}.{b}.conv2", w, w * 9))
            shapes.append((f"{name}.{b}.conv3", out, w))
            if b == 0:
                shapes.append((f"{name}.{b}.downsample", out, cin))
    shapes.append(("fc", 2048, 1000))
    return [TensorSpec(n, r, c, grad="student_t") for n, r, c in shapes]


def _ctr() -> List[TensorSpec]:
    ts = [TensorSpec("mlp0", 1024, 1024), TensorSpec("mlp1", 1024, 512),
          TensorSpec("mlp2", 512, 256)]
    for i in range(26):
        rows = int(round(10 ** (5 + i / 25)))
        ts.append(TensorSpec(f"table{i}", rows, 128, kind="sparse", grad="sparse_rows"))
    return ts


def workload(wid: int) -> Workload:
    """The five synthetic workloads, by id 0..4."""
    if wid == 0:
        return Workload(0, "single-256x512-b128", [TensorSpec("w", 256, 512)], 128,
                        cadence=1, steps=10, newton_tol=0.0,
                        notes="one fp32 weight, 8 blocks of 128x128, roots every step "
                              "with the full 20 coupled-Newton iterations")
    if wid == 1:
        return Workload(1, "transformer-base-b128", _transformer_base(), 128,
                        max_precond_dim=4096, cadence=20, steps=80,
                        notes="6+6 layers, d_model 512, ffn 2048, 32000x512 embedding "
                              "on diagonal Adagrad")
    if wid == 2:
        return Workload(2, "bert-large-b512", _bert_large(), 512, cadence=20, steps=80,
                        notes="24 layers, hidden 1024, ffn 4096; fp64 roots for "
                              "condition number > 1e5")
    if wid == 3:
        return Workload(3, "resnet50-b256", _resnet50(), 256, cadence=20, steps=80,
                        notes="conv weights reshaped to out x in*k*k plus FC 2048x1000")
    if wid == 4:
        return Workload(4, "ctr-mlp-b1024-sparse-tables", _ctr(), 1024, cadence=20,
                        steps=80,
                        notes="MLP tower on Shampoo, 26 embedding tables (1e5..1e6 rows "
                              "x 128) on sparse-row Adagrad")
    raise ValueError(f"unknown workload {wid}")


# ---------------------------------------------------------------- random draws
def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *entropy])))


def _orthonormal(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    """n x r matrix with orthonormal columns: QR of a Gaussian, signs fixed."""
    q, rr = np.linalg.qr(rng.standard_normal((n, r)))
    return q * np.where(np.diag(rr) < 0, -1.0, 1.0)


@dataclass
class _Fixed:
    u: Optional[np.ndarray] = None
    s: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    noise: float = 0.0
    row_scale: Optional[np.ndarray] = None
    perm: Optional[np.ndarray] = None
    logw: Optional[np.ndarray] = None


class GradientStream:
    """Per-step gradients for one workload.

    Dense low-rank:  G = U diag(s) V^T + noise * N(0,1); U, V have orthonormal
                     columns, s_i = 10^U(-3,0); U, s, V fixed per matrix, the
                     noise fresh each step.  noise < 0 in the spec draws a fixed
                     per-matrix std 10^U(-4,-1).
    Student-t:       G_ij = c_i * t_ij, t ~ Student-t(3) fresh each step,
                     c_i = 10^U(-4,0) fixed per row.
    Sparse rows:     each step round(frac * rows) distinct rows, drawn without
                     replacement with weight rank^-zipf_s over a fixed random
                     rank -> row permutation; row gradients N(0,1); indices
                     int32, sorted.
    """

    def __init__(self, wl: Workload, tensor_ids: Optional[List[int]] = None):
        self.wl = wl
        self.ids = list(range(len(wl.tensors))) if tensor_ids is None else list(tensor_ids)
        self._fixed: dict = {}

    def _fixed_for(self, i: int) -> _Fixed:
        if i in self._fixed:
            return self._fixed[i]
        spec = self.wl.tensors[i]
        rng = _rng(self.wl.wid, i, 0)
        fx = _Fixed()
        if spec.grad == "lowrank":
            r = spec.rank or min(spec.rows, spec.cols)
            fx.u = _orthonormal(rng, spec.rows, r)
            fx.v = _orthonormal(rng, spec.cols, r)
            fx.s = 10.0 ** rng.uniform(-3.0, 0.0, size=r)
            fx.noise = spec.noise if spec.noise >= 0 else 10.0 ** rng.uniform(-4.0, -1.0)
        elif spec.grad == "student_t":
            fx.row_scale = 10.0 ** rng.uniform(-4.0, 0.0, size=spec.rows)
        elif spec.grad == "sparse_rows":
            fx.perm = rng.permutation(spec.rows)
            ranks = np.arange(1, spec.rows + 1, dtype=np.float64)
            fx.logw = -self.wl.zipf_s * np.log(ranks)
        self._fixed[i] = fx
        return fx

    def dense(self, i: int, step: int) -> np.ndarray:
        """fp32 gradient of dense tensor i at this step (row-major)."""
        spec = self.wl.tensors[i]
        fx = self._fixed_for(i)
        rng = _rng(self.wl.wid, i, 1 + step)
        if spec.grad == "lowrank":
            g = (fx.u * fx.s) @ fx.v.T
            g += fx.noise * rng.standard_normal((spec.rows, spec.cols))
        elif spec.grad == "student_t":
            g = fx.row_scale[:, None] * rng.standard_t(3.0, size=(spec.rows, spec.cols))
        else:
            raise ValueError(f"{spec.name} is not dense")
        return np.ascontiguousarray(g, dtype=np.float32)

    def sparse(self, i: int, step: int) -> Tuple[np.ndarray, np.ndarray]:
        """(sorted distinct int32 row ids, fp32 row gradients) of table i."""
        spec = self.wl.tensors[i]
        fx = self._fixed_for(i)
        rng = _rng(self.wl.wid, i, 1 + step)
        k = int(round(self.wl.sparse_frac * spec.rows))
        # weighted sampling without replacement (Efraimidis-Spirakis keys)
        keys = np.log(rng.random(spec.rows)) / np.exp(fx.logw)
        top = np.argpartition(keys, spec.rows - k)[spec.rows - k:]
        rows = np.sort(fx.perm[top]).astype(np.int32)
        grads = rng.standard_normal((k, spec.cols)).astype(np.float32)
        return rows, grads

    def step(self, step: int):
        """Dict tensor index -> dense fp32 array, or (rows, row_grads) for sparse."""
        out = {}
        for i in self.ids:
            if self.wl.tensors[i].kind == "dense":
                out[i] = self.dense(i, step)
            else:
                out[i] = self.sparse(i, step)
        return out


def initial_weight(wl: Workload, i: int) -> np.ndarray:
    """W0 = 0.02 * N(0,1), fp32."""
    spec = wl.tensors[i]
    rng = _rng(wl.wid, i, 1_000_000)
    return (0.02 * rng.standard_normal((spec.rows, spec.cols))).astype(np.float32)


def spd_with_spectrum(n: int, eigvals: np.ndarray, seed: int) -> np.ndarray:
    """Symmetric matrix Q diag(eigvals) Q^T with a seeded random orthogonal Q
    (fp64).  Used for inverse-root test inputs with a known spectrum."""
    q = _orthonormal(_rng(9, seed, n), n, n)
    return (q * eigvals) @ q.T


def log_spectrum(n: int, kappa: float) -> np.ndarray:
    """n eigenvalues log-uniform in [1/kappa, 1], both ends included."""
    return np.logspace(-np.log10(kappa), 0.0, n)
