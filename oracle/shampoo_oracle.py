"""fp64 CPU oracle for the Shampoo optimizer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it, and the
two share no code: this file restates the method from the pages with NumPy in
fp64, block by block, with no blocking, fusion or reordering beyond what the
definition states.

Sources.  The method is described in "Scalable Second Order Optimization for
Deep Learning" (Anil, Gupta, Koren, Regan, Singer); the only technical account
on the pages is the Shampoo-at-scale podcast transcript:
  * cue 6-8   -- one small statistics matrix per dimension of a 2-D weight,
                 "L" for rows and "R" for columns, standing in for full-matrix
                 Adagrad through a Kronecker product;
  * cue 10    -- three extra pieces of work per step: accumulate gradient outer
                 products into L and R; the inverse fourth roots of L and R;
                 the preconditioned gradient multiply;
  * cue 12    -- the root is the expensive step, done by coupled Newton or an
                 SVD, in double precision because L and R are ill-conditioned;
  * cue 14-16 -- roots recomputed only every so often and the last ones reused
                 meanwhile; over-large layers split into blocks that are each
                 preconditioned on their own (Lemma 2).
Everything else (EMA weighting of the statistics, the damping rule
eps = eps_rel * lambda_max, grafting to diagonal Adagrad, heavy-ball momentum,
the Adagrad fallback for very large dimensions and for sparse embedding rows)
is not on the pages; it is this library's stated configuration and every such
choice is named where it is used.

Root.  For a symmetric PSD factor the inverse p-th root is unique (the principal
SPD root); the oracle obtains it from the symmetric eigendecomposition
(numpy.linalg.eigh, LAPACK), which for SPD matrices is the SVD the transcript
names in cue 12.  The GPU reaches the same matrix by coupled Newton iteration.

Pins.  tests/test_oracle_pins.py checks every function here against exact
rational brute force, 50-digit mpmath eigenvalues, SciPy's Schur-Pade
fractional power, closed forms for diagonal and rank-1 gradients, and
invariants.  The constants beta1, graft_eps and the cadence of the larger
workloads are configuration, not outputs; no page fixes their values (their
parity is unpinned, though both sides read them from one config).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------- config
@dataclass
class OracleConfig:
    block_size: int
    max_precond_dim: int = 0      # 0: no limit
    root_p: int = 4
    beta1: float = 0.9
    beta2: float = 0.999
    lr: float = 1e-3
    eps_rel: float = 1e-6
    graft_eps: float = 1e-10
    cadence: int = 1
    root_parts: int = 1           # > 1: staggered root recompute (see root_due)
    root_delay: int = 0           # steps between computing roots and using them
    large_layer: int = 0          # 1: one-sided preconditioning (see one_sided_side)


# ------------------------------------------------------- blocking (Lemma 2)
def split_dim(d: int, b: int) -> List[Tuple[int, int]]:
    """Chunks (start, length) of one dimension: full chunks of b from the top
    or left, the last one ragged.  Lemma 2 (podcast cue 16) blocks a layer and
    preconditions each block separately; the pages give no partition rule, so
    the plainest one is used: top-left aligned b x b tiles."""
    if d <= 0:
        return []
    return [(s, min(b, d - s)) for s in range(0, d, b)]


def blocks(m: int, n: int, b: int) -> List[Tuple[int, int, int, int]]:
    """(r0, mb, c0, nb) for every block of an m x n tensor, row-major order."""
    return [(r0, mb, c0, nb) for r0, mb in split_dim(m, b) for c0, nb in split_dim(n, b)]


def uses_shampoo(m: int, n: int, cfg: OracleConfig) -> bool:
    """Tensors with a dimension above max_precond_dim take diagonal Adagrad
    instead (a configuration of this library, not of the pages)."""
    return cfg.max_precond_dim <= 0 or max(m, n) <= cfg.max_precond_dim


# -------------------------------------------------------------- statistics
def one_sided_side(m: int, n: int, cfg: "OracleConfig", kind: str = "dense") -> Optional[str]:
    """Lemma 1 (podcast cue 16): for a layer too large to precondition on both
    sides (a giant embedding or softmax), only one of L or R is used.  A
    dense tensor that does not use Shampoo blocks gets one-sided
    preconditioning when large_layer is set and one dimension fits under
    max_precond_dim: "R" (statistics G^T G, D = G P) when the columns fit,
    else "L" (G G^T, D = P G).  A sparse-row table (an embedding) gets "R"
    when large_layer is set and its columns fit (any, when max_precond_dim
    is 0).  None: diagonal (or sparse-row) Adagrad."""
    if not cfg.large_layer:
        return None
    if kind == "sparse":
        return "R" if cfg.max_precond_dim <= 0 or n <= cfg.max_precond_dim else None
    if cfg.max_precond_dim <= 0 or uses_shampoo(m, n, cfg):
        return None
    if n <= cfg.max_precond_dim:
        return "R"
    if m <= cfg.max_precond_dim:
        return "L"
    return None


def ema_weights(beta2: float) -> Tuple[float, float]:
    """(decay, weight of the new outer product).  The transcript says the
    statistics accumulate outer products (cue 10); this library keeps an
    exponential moving average with decay beta2, weighting the new term by
    1 - beta2, and a plain sum when beta2 == 1."""
    return beta2, (1.0 - beta2) if beta2 < 1.0 else 1.0


def update_statistics(L: np.ndarray, R: np.ndarray, G: np.ndarray, beta2: float):
    """L <- beta2 L + w G G^T,  R <- beta2 R + w G^T G  (cue 10), in fp64."""
    d, w = ema_weights(beta2)
    g = np.asarray(G, dtype=np.float64)
    return d * L + w * (g @ g.T), d * R + w * (g.T @ g)


# ------------------------------------------------------------ inverse root
@dataclass
class RootResult:
    P: Optional[np.ndarray]     # None when the input is not finite
    lam_max: float
    lam_min: float
    eps: float
    kappa: float                # (lam_max + eps) / (lam_min + eps), eigenvalues clamped at 0
    ok: bool


def inverse_root(S: np.ndarray, eps_rel: float, p: int, eps: Optional[float] = None,
                 clamp: bool = True) -> RootResult:
    """(S + eps I)^(-1/p) by symmetric eigendecomposition (cue 10: inverse
    fourth root; cue 12: SVD route, double precision).

    eps = eps_rel * lambda_max(S) unless an explicit eps is given (the GPU's own
    eps, for stage-isolated comparison).  With clamp=True (the optimizer's own
    statistics), eigenvalues below zero -- rounding of a PSD matrix -- are
    clamped to zero before eps is added.  With clamp=False the result is the
    exact principal root of the damped matrix as given (used to check a GPU
    root against the very matrix the GPU received); it requires
    S + eps I to be positive definite, else ok=False.  A factor whose largest
    eigenvalue is not positive (no statistics yet) gets P = I.  A non-finite
    factor returns ok=False and no P, so the caller keeps the previous root
    (cue 14-16: training carries on with the last preconditioner).  The input
    is symmetrised as (S + S^T)/2 first."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    if not np.all(np.isfinite(S)):
        return RootResult(None, np.nan, np.nan, np.nan, np.nan, False)
    S = 0.5 * (S + S.T)
    lam, V = np.linalg.eigh(S)
    lmax = float(lam[-1]) if n else 0.0
    if n == 0 or lmax <= 0.0:
        return RootResult(np.eye(n), lmax, lmax, 0.0, 1.0, True)
    e = eps_rel * lmax if eps is None else float(eps)
    if clamp:
        lam = np.maximum(lam, 0.0)
    elif lam[0] + e <= 0.0:
        return RootResult(None, lmax, float(lam[0]), e, np.inf, False)
    P = (V * (lam + e) ** (-1.0 / p)) @ V.T
    return RootResult(P, lmax, float(lam[0]), e, (lmax + e) / (lam[0] + e), True)


# --------------------------------------------------------- precondition
def precondition(PL: np.ndarray, G: np.ndarray, PR: np.ndarray) -> np.ndarray:
    """D = L^(-1/4) G R^(-1/4): the preconditioned gradient multiply (cue 10,
    cue 14)."""
    return PL @ np.asarray(G, dtype=np.float64) @ PR


# ---------------------------------------------------------------- graft
def adagrad_accumulate(a: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Diagonal Adagrad accumulator a <- a + G*G (a plain running sum)."""
    g = np.asarray(G, dtype=np.float64)
    return a + g * g


def adagrad_direction(a: np.ndarray, G: np.ndarray, delta: float) -> np.ndarray:
    """A = G / (sqrt(a) + delta), with a already including this step."""
    return np.asarray(G, dtype=np.float64) / (np.sqrt(a) + delta)


def graft(A_b: np.ndarray, D_b: np.ndarray) -> np.ndarray:
    """Per-block grafting: keep D's direction, take Adagrad's magnitude,
    U = D * ||A||_F / ||D||_F; U = 0 when ||D||_F = 0.  Not on the pages; a
    configuration of this library (magnitude from diagonal Adagrad, direction
    from Shampoo, per Lemma-2 block)."""
    nd = float(np.sqrt(np.sum(D_b * D_b)))
    if nd == 0.0:
        return np.zeros_like(D_b)
    return D_b * (float(np.sqrt(np.sum(A_b * A_b))) / nd)


def momentum_update(mom: np.ndarray, W: np.ndarray, U: np.ndarray, beta1: float, lr: float):
    """Heavy-ball momentum and the weight update: mom <- beta1 mom + U,
    W <- W - lr mom.  Returns (mom, W)."""
    mom = beta1 * mom + U
    return mom, W - lr * mom


def sparse_rows_update(a: np.ndarray, W: np.ndarray, rows: np.ndarray, g: np.ndarray,
                       lr: float, delta: float):
    """Sparse-row Adagrad for embedding tables: for each touched row r,
    a_r += g_r^2 and W_r -= lr g_r / (sqrt(a_r) + delta); untouched rows and
    momentum are left alone.  Rows must be distinct.  Returns (a, W)."""
    a = a.copy()
    W = W.copy()
    gr = np.asarray(g, dtype=np.float64)
    for k, r in enumerate(np.asarray(rows)):
        a[r] = a[r] + gr[k] * gr[k]
        W[r] = W[r] - lr * gr[k] / (np.sqrt(a[r]) + delta)
    return a, W


# ----------------------------------------------------------- whole step
class _BlockState:
    def __init__(self, mb: int, nb: int):
        self.L = np.zeros((mb, mb))
        self.R = np.zeros((nb, nb))
        self.PL = np.eye(mb)
        self.PR = np.eye(nb)
        self.root_L: Optional[RootResult] = None
        self.root_R: Optional[RootResult] = None
        # roots computed but not yet in effect: (step they take effect, L, R)
        self.pending = None


class _OneSidedState:
    """Statistics and root of a one-sided (Lemma 1) tensor."""

    def __init__(self, side: str, dim: int):
        self.side = side
        self.S = np.zeros((dim, dim))
        self.P = np.eye(dim)
        self.root: Optional[RootResult] = None
        self.pending = None


def root_due(block_index: int, t: int, cadence: int, parts: int) -> bool:
    """Whether the roots of Shampoo block `block_index` (counted over all
    tensors, in order) are recomputed at step t, after that step's statistics.

    The roots are recomputed only every so often and the accelerator keeps
    using the last ones in between (podcast cue 14); the pages move that work
    off the critical path by computing it in the background (cues 14-16).
    With parts == 1 every root is recomputed at t = 0, k, 2k, ... (k the
    cadence).  With parts = P > 1 (P dividing k) the blocks are split by
    index modulo P and one part is recomputed every k/P steps, part
    (t / (k/P)) mod P: each root is still refreshed once every k steps, and
    the cost of a root pass is spread evenly over the steps."""
    if parts <= 1:
        return t % cadence == 0
    if cadence % parts != 0:
        raise ValueError("root_parts must divide the cadence")
    window = cadence // parts
    return t % window == 0 and (t // window) % parts == block_index % parts


class ShampooOracle:
    """The whole optimizer step over a list of tensors, fp64.

    shapes: list of (rows, cols, kind) with kind "dense" or "sparse".
    weights: initial fp32 weights (converted to fp64).

    step(grads, t) with grads[i] an (m, n) array for dense tensors or a
    (rows, row_grads) pair for sparse tensors, t counted from 0:
      1. statistics of every Shampoo block (cue 10);
      2. inverse p-th roots of the factors of every block that root_due
         selects (all of them at t % cadence == 0 by default; cue 10, 12,
         14), keeping the previous root for a non-finite factor.  With
         root_delay = d > 0 the roots computed at step t (from the statistics
         after step t) take effect at step t + d, before that step's apply:
         the roots are produced in the background while the accelerator keeps
         using the last ones (cues 14-16);
      3. D = PL G PR per block (cue 10);
      4. a += G*G per tensor, A = G/(sqrt(a)+delta), per-block graft U;
         tensors over max_precond_dim use U = A, or with large_layer the
         one-sided preconditioner (Lemma 1) of the side that fits, grafted
         over the whole tensor;
      5. heavy-ball momentum and weight update;
      6. sparse tables: sparse-row Adagrad.
    """

    def __init__(self, cfg: OracleConfig, shapes: Sequence[Tuple[int, int, str]],
                 weights: Sequence[np.ndarray]):
        self.cfg = cfg
        self.shapes = [(int(m), int(n), k) for m, n, k in shapes]
        self.W = [np.asarray(w, dtype=np.float64).copy() for w in weights]
        self.a = [np.zeros((m, n)) for m, n, _ in self.shapes]
        self.mom = [np.zeros((m, n)) for m, n, _ in self.shapes]
        self.blocks: Dict[int, List[Tuple[Tuple[int, int, int, int], _BlockState]]] = {}
        for i, (m, n, kind) in enumerate(self.shapes):
            if kind == "dense" and uses_shampoo(m, n, cfg):
                self.blocks[i] = [(bk, _BlockState(bk[1], bk[3]))
                                  for bk in blocks(m, n, cfg.block_size)]
        # one-sided tensors, numbered for the root schedule after every block
        n_blocks = sum(len(v) for v in self.blocks.values())
        self.one_sided: Dict[int, Tuple[int, _OneSidedState]] = {}
        for i, (m, n, kind) in enumerate(self.shapes):
            side = one_sided_side(m, n, cfg, kind)
            if side is not None:
                if cfg.root_p % 2:
                    raise ValueError("one-sided preconditioning needs an even root_p")
                self.one_sided[i] = (n_blocks + len(self.one_sided),
                                     _OneSidedState(side, n if side == "R" else m))
        self.last_D: Dict[int, np.ndarray] = {}

    def step(self, grads, t: int) -> List[np.ndarray]:
        cfg = self.cfg
        deltas = []
        gblock = 0   # global block index over the tensors, in order
        # roots computed root_delay steps ago take effect now
        for blist in self.blocks.values():
            for _, st in blist:
                if st.pending is not None and st.pending[0] <= t:
                    _, rl, rr = st.pending
                    st.pending = None
                    if rl.ok:
                        st.PL = rl.P
                    if rr.ok:
                        st.PR = rr.P
        for _, os_st in self.one_sided.values():
            if os_st.pending is not None and os_st.pending[0] <= t:
                _, rr = os_st.pending
                os_st.pending = None
                if rr.ok:
                    os_st.P = rr.P
        for i, (m, n, kind) in enumerate(self.shapes):
            W_old = self.W[i]
            if kind == "sparse":
                rows, g = grads[i]
                if i in self.one_sided:
                    self._sparse_one_sided(i, np.asarray(rows), np.asarray(g, dtype=np.float64), t)
                else:
                    self.a[i], self.W[i] = sparse_rows_update(self.a[i], self.W[i], rows, g,
                                                              cfg.lr, cfg.graft_eps)
                deltas.append(self.W[i] - W_old)
                continue
            G = np.asarray(grads[i], dtype=np.float64)
            self.a[i] = adagrad_accumulate(self.a[i], G)
            A = adagrad_direction(self.a[i], G, cfg.graft_eps)
            if i in self.blocks:
                U = np.zeros((m, n))
                D_full = np.zeros((m, n))
                for (r0, mb, c0, nb), st in self.blocks[i]:
                    Gb = G[r0:r0 + mb, c0:c0 + nb]
                    st.L, st.R = update_statistics(st.L, st.R, Gb, cfg.beta2)
                    recompute = root_due(gblock, t, cfg.cadence, cfg.root_parts)
                    gblock += 1
                    if recompute:
                        st.root_L = inverse_root(st.L, cfg.eps_rel, cfg.root_p)
                        st.root_R = inverse_root(st.R, cfg.eps_rel, cfg.root_p)
                        if cfg.root_delay > 0:
                            st.pending = (t + cfg.root_delay, st.root_L, st.root_R)
                        else:
                            if st.root_L.ok:
                                st.PL = st.root_L.P
                            if st.root_R.ok:
                                st.PR = st.root_R.P
                    Db = precondition(st.PL, Gb, st.PR)
                    D_full[r0:r0 + mb, c0:c0 + nb] = Db
                    U[r0:r0 + mb, c0:c0 + nb] = graft(A[r0:r0 + mb, c0:c0 + nb], Db)
                self.last_D[i] = D_full
            elif i in self.one_sided:
                # Lemma 1: S <- beta2 S + w G^T G (or G G^T), P = (S + eps I)^(-2/p)
                # (the one factor carries the whole -1/2), D = G P (or P G),
                # grafted over the whole tensor
                _, st = self.one_sided[i]
                self._one_sided_stats_and_root(i, (G.T @ G) if st.side == "R" else (G @ G.T), t)
                D = (G @ st.P) if st.side == "R" else (st.P @ G)
                self.last_D[i] = D
                U = graft(A, D)
            else:
                U = A
            self.mom[i], self.W[i] = momentum_update(self.mom[i], self.W[i], U,
                                                     cfg.beta1, cfg.lr)
            deltas.append(self.W[i] - W_old)
        return deltas

    def _one_sided_stats_and_root(self, i: int, outer: np.ndarray, t: int):
        """S <- beta2 S + w outer; on a root step of this tensor's block,
        P = (S + eps I)^(-2/p): the one factor carries the whole -1/2."""
        cfg = self.cfg
        idx, st = self.one_sided[i]
        d, w = ema_weights(cfg.beta2)
        st.S = d * st.S + w * outer
        if root_due(idx, t, cfg.cadence, cfg.root_parts):
            st.root = inverse_root(st.S, cfg.eps_rel, cfg.root_p // 2)
            if cfg.root_delay > 0:
                st.pending = (t + cfg.root_delay, st.root)
            elif st.root.ok:
                st.P = st.root.P

    def _sparse_one_sided(self, i: int, rows: np.ndarray, g: np.ndarray, t: int):
        """One-sided preconditioning of a sparse-row table: the R side, with
        the row-sparse gradient G (g on the listed rows, 0 elsewhere):
        S <- beta2 S + w G^T G = beta2 S + w g^T g; D = G P (nonzero on the
        listed rows only); a += G*G and A = G / (sqrt(a) + delta) on those
        rows; U = graft(A, D) over the table; W -= lr U.  No momentum, as
        for the sparse-row Adagrad this replaces, so untouched rows keep
        their weights.  Rows must be distinct."""
        cfg = self.cfg
        _, st = self.one_sided[i]
        self._one_sided_stats_and_root(i, g.T @ g, t)
        D = g @ st.P
        a = self.a[i].copy()
        a[rows] = a[rows] + g * g
        A = g / (np.sqrt(a[rows]) + cfg.graft_eps)
        U = graft(A, D)
        W = self.W[i].copy()
        W[rows] = W[rows] - cfg.lr * U
        self.a[i], self.W[i] = a, W
        self.last_D[i] = D

    def block_states(self, i: int):
        return self.blocks.get(i, [])
