"""Thin Python binding of libshampoo_mi355x.so (ctypes; argument marshalling only).

Every step of the optimizer runs in the library's HIP kernels; this module
only checks tensor shapes/dtypes, passes device pointers and the current HIP
stream, and allocates the library's state buffer as a PyTorch uint8 tensor.
It raises if the library has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libshampoo_mi355x.so")

ROOT_MODES = {"f32": 0, "f64": 1, "auto": 2}
APPLY_PRECISIONS = {"fp32": 0, "bf16x3": 1}
DENSE, SPARSE_ROWS = 0, 1

FACTOR_NONFINITE_INPUT = 1
FACTOR_NONFINITE_ROOT = 2
FACTOR_RESIDUAL_HIGH = 4
FACTOR_FP64 = 8
FACTOR_ZERO = 16


class TensorDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("max_precond_dim", ctypes.c_int32),
                ("root_p", ctypes.c_int32), ("newton_iters", ctypes.c_int32),
                ("root_mode", ctypes.c_int32), ("lanczos_steps", ctypes.c_int32),
                ("root_parts", ctypes.c_int32), ("large_layer", ctypes.c_int32),
                ("apply_precision", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("lr", ctypes.c_double),
                ("eps_rel", ctypes.c_double), ("graft_eps", ctypes.c_double),
                ("fp64_cond_threshold", ctypes.c_double), ("newton_tol", ctypes.c_double)]


class SparseRows(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("row_grads", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64)]


class FactorDiag(ctypes.Structure):
    _fields_ = [("lambda_max", ctypes.c_double), ("eps", ctypes.c_double),
                ("kappa_est", ctypes.c_double), ("residual", ctypes.c_double),
                ("block", ctypes.c_int32), ("side", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("status", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BlockLayout(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("row0", ctypes.c_int32), ("col0", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("ld_l", ctypes.c_int32),
                ("ld_r", ctypes.c_int32), ("factor_l", ctypes.c_int32),
                ("factor_r", ctypes.c_int32), ("one_sided", ctypes.c_int32),
                ("off_l", ctypes.c_int64),
                ("off_r", ctypes.c_int64), ("off_pl", ctypes.c_int64), ("off_pr", ctypes.c_int64),
                ("off_pl64", ctypes.c_int64), ("off_pr64", ctypes.c_int64)]


class Peaks(ctypes.Structure):
    _fields_ = [("mfma_f32_tflops", ctypes.c_double), ("mfma_f64_tflops", ctypes.c_double),
                ("mfma_bf16_tflops", ctypes.c_double),
                ("copy_gbs", ctypes.c_double), ("copy_bytes", ctypes.c_int64)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


# name -> (restype, argtypes); every symbol declared in include/shampoo.h
_P = ctypes.c_void_p
SIGNATURES = {
    "shampoo_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int32,
                                      ctypes.POINTER(TensorDesc), ctypes.POINTER(_P)]),
    "shampoo_state_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "shampoo_bind_state": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "shampoo_update_stats": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(SparseRows), _P]),
    "shampoo_compute_inverse_roots": (ctypes.c_int, [_P, _P]),
    "shampoo_compute_inverse_roots_part": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "shampoo_compute_inverse_roots_noalloc": (ctypes.c_int, [_P, _P]),
    "shampoo_roots_async_begin": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "shampoo_roots_async_end": (ctypes.c_int, [_P, _P]),
    "shampoo_precondition_and_apply": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                                      ctypes.POINTER(SparseRows), _P]),
    "shampoo_step": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                    ctypes.POINTER(SparseRows), ctypes.c_int32, _P]),
    "shampoo_num_factors": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]),
    "shampoo_get_diagnostics": (ctypes.c_int, [_P, ctypes.POINTER(FactorDiag), ctypes.c_int32, _P]),
    "shampoo_block_info": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(BlockLayout)]),
    "shampoo_tensor_info": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]),
    "shampoo_profile_enable": (ctypes.c_int, [_P, ctypes.c_int32]),
    "shampoo_profile_read": (ctypes.c_int, [_P, ctypes.POINTER(KernelTime), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32)]),
    "shampoo_measure_peaks": (ctypes.c_int, [ctypes.POINTER(Peaks), _P, ctypes.c_size_t, _P]),
    "shampoo_destroy": (None, [_P]),
    "shampoo_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m second_order_optimizer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class ShampooError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise ShampooError(f"{what}: {lib().shampoo_strerror(rc).decode()} ({rc})")


def make_config(block_size: int, *, max_precond_dim: int = 0, root_p: int = 4,
                newton_iters: int = 20, root_mode: str = "f32", lanczos_steps: int = 0,
                beta1: float = 0.9, beta2: float = 0.999, lr: float = 1e-3,
                eps_rel: float = 1e-6, graft_eps: float = 1e-10,
                fp64_cond_threshold: float = 1e5, root_parts: int = 0,
                large_layer: int = 0, newton_tol: float = 1e-3,
                apply_precision: str = "fp32") -> Config:
    return Config(block_size, max_precond_dim, root_p, newton_iters, ROOT_MODES[root_mode],
                  lanczos_steps, root_parts, large_layer, APPLY_PRECISIONS[apply_precision], 0,
                  beta1, beta2, lr, eps_rel, graft_eps, fp64_cond_threshold, newton_tol)


ROOTS_NONE, ROOTS_ALL = -1, -2


def measure_peaks(device="cuda", scratch_mib: int = 2048) -> dict:
    """Matrix-core and copy peaks of the device (shampoo_measure_peaks): fp32
    and fp64 MFMA TFLOP/s with no memory traffic, and the GB/s of a plain
    device copy of scratch_mib / 2 MiB."""
    import torch
    dev = torch.device(device)
    buf = torch.empty(scratch_mib << 20, dtype=torch.uint8, device=dev)
    out = Peaks()
    s = _P(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib().shampoo_measure_peaks(ctypes.byref(out), buf.data_ptr(), buf.numel(), s),
           "shampoo_measure_peaks")
    del buf
    return {"mfma_f32_tflops": out.mfma_f32_tflops, "mfma_f64_tflops": out.mfma_f64_tflops,
            "mfma_bf16_tflops": out.mfma_bf16_tflops, "copy_gbs": out.copy_gbs,
            "copy_bytes": out.copy_bytes}


def root_selector(step: int, cadence: int, parts: int) -> int:
    """Which roots a step recomputes: every root at step % cadence == 0, or,
    with parts = P >= 2 (P dividing the cadence), part (step / (cadence/P)) % P
    whenever step % (cadence/P) == 0."""
    if parts <= 1:
        return ROOTS_ALL if step % cadence == 0 else ROOTS_NONE
    if cadence % parts:
        raise ValueError("root_parts must divide the cadence")
    window = cadence // parts
    return (step // window) % parts if step % window == 0 else ROOTS_NONE


class Plan:
    """A handle without device state: planning and layout queries only."""

    def __init__(self, shapes: Sequence[Tuple[int, int, int]], cfg: Config):
        L = lib()
        self.shapes = [(int(r), int(c), int(k)) for r, c, k in shapes]
        descs = (TensorDesc * len(self.shapes))(*[TensorDesc(r, c, k, 0) for r, c, k in self.shapes])
        h = _P()
        _check(L.shampoo_create(ctypes.byref(cfg), len(self.shapes), descs, ctypes.byref(h)),
               "shampoo_create")
        self.h = h
        self.cfg = cfg
        nf, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(L.shampoo_num_factors(h, ctypes.byref(nf), ctypes.byref(nb)), "shampoo_num_factors")
        self.n_factors, self.n_blocks = nf.value, nb.value
        sb = ctypes.c_size_t()
        _check(L.shampoo_state_bytes(h, ctypes.byref(sb)), "shampoo_state_bytes")
        self.state_bytes = sb.value

    def block(self, i: int) -> BlockLayout:
        out = BlockLayout()
        _check(lib().shampoo_block_info(self.h, i, ctypes.byref(out)), "shampoo_block_info")
        return out

    def tensor(self, t: int):
        a, m = ctypes.c_int64(), ctypes.c_int64()
        fb, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().shampoo_tensor_info(self.h, t, ctypes.byref(a), ctypes.byref(m),
                                         ctypes.byref(fb), ctypes.byref(nb)), "shampoo_tensor_info")
        return a.value, m.value, fb.value, nb.value

    def close(self):
        if getattr(self, "h", None):
            lib().shampoo_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Shampoo(Plan):
    """Device-bound optimizer: the state buffer is a uint8 CUDA tensor."""

    def __init__(self, shapes, cfg: Config, device="cuda", async_roots: bool = False):
        """async_roots (needs cfg.root_parts >= 2): each due part of the root
        pass runs in the background from the statistics of the step that
        starts it, and its roots take effect when the next part starts
        (cadence / root_parts steps later)."""
        import torch
        if async_roots and cfg.root_parts < 2:
            raise ValueError("async_roots needs root_parts >= 2")
        self.async_roots = async_roots
        super().__init__(shapes, cfg)
        self.torch = torch
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.state = torch.empty(self.state_bytes, dtype=torch.uint8, device=self.device)
        _check(lib().shampoo_bind_state(self.h, self.state.data_ptr(), self.state_bytes,
                                        self._stream()), "shampoo_bind_state")

    def _stream(self):
        return _P(self.torch.cuda.current_stream(self.device).cuda_stream)

    def _ptrs(self, ts, need, what):
        arr = (_P * len(self.shapes))()
        for i, ((r, c, k), t) in enumerate(zip(self.shapes, ts)):
            if t is None:
                if need(k):
                    raise ValueError(f"{what}[{i}] is required")
                continue
            if (t.dtype != self.torch.float32 or not t.is_contiguous() or t.device != self.device
                    or tuple(t.shape) != (r, c)):
                raise ValueError(f"{what}[{i}] must be a contiguous fp32 {r}x{c} tensor on "
                                 f"{self.device}")
            arr[i] = t.data_ptr()
        return arr

    def update_stats(self, grads, sparse=None):
        """sparse: as in precondition_and_apply; read for sparse-row tables
        with one-sided preconditioning (large_layer)."""
        arr = self._ptrs(grads, lambda k: False, "grads")
        sp, _keep = self._sparse_args(sparse)
        _check(lib().shampoo_update_stats(self.h, arr, sp, self._stream()), "shampoo_update_stats")

    def compute_inverse_roots(self):
        _check(lib().shampoo_compute_inverse_roots(self.h, self._stream()),
               "shampoo_compute_inverse_roots")

    def compute_inverse_roots_noalloc(self):
        """The same root pass with the Newton iterates in the library's static
        device scratch (shampoo_compute_inverse_roots_noalloc)."""
        _check(lib().shampoo_compute_inverse_roots_noalloc(self.h, self._stream()),
               "shampoo_compute_inverse_roots_noalloc")

    def compute_inverse_roots_part(self, part: int):
        _check(lib().shampoo_compute_inverse_roots_part(self.h, part, self._stream()),
               "shampoo_compute_inverse_roots_part")

    def _apply_args(self, params, grads, sparse):
        pa = self._ptrs(params, lambda k: True, "params")
        ga = self._ptrs(grads, lambda k: k == DENSE, "grads")
        sp, keep = self._sparse_args(sparse)
        return pa, ga, sp, keep

    def _sparse_args(self, sparse):
        sp = None
        keep = []
        if any(k == SPARSE_ROWS for _, _, k in self.shapes):
            sp = (SparseRows * len(self.shapes))()
            for i, (r, c, k) in enumerate(self.shapes):
                if k != SPARSE_ROWS or sparse is None or i not in sparse:
                    continue
                rows, g = sparse[i]
                if (rows.dtype != self.torch.int32 or g.dtype != self.torch.float32
                        or not rows.is_contiguous() or not g.is_contiguous()
                        or g.shape != (rows.numel(), c)):
                    raise ValueError(f"sparse[{i}] must be (int32 rows, fp32 rows x {c})")
                keep.append((rows, g))
                sp[i] = SparseRows(rows.data_ptr(), g.data_ptr(), rows.numel())
        return sp, keep

    def precondition_and_apply(self, params, grads, sparse=None):
        """sparse: dict tensor index -> (int32 rows, fp32 row grads) device tensors."""
        pa, ga, sp, _keep = self._apply_args(params, grads, sparse)
        _check(lib().shampoo_precondition_and_apply(self.h, pa, ga, sp, self._stream()),
               "shampoo_precondition_and_apply")

    def step(self, params, grads, step: int, cadence: int, sparse=None):
        """One optimizer step (shampoo_step): statistics, roots when
        step % cadence == 0, apply."""
        pa, ga, sp, _keep = self._apply_args(params, grads, sparse)
        sel = root_selector(step, cadence, self.cfg.root_parts)
        if self.async_roots:
            if sel >= 0:   # the part started cadence/P steps ago takes effect now
                self.roots_async_end()
            _check(lib().shampoo_step(self.h, pa, ga, sp, ROOTS_NONE, self._stream()),
                   "shampoo_step")
            if sel >= 0:
                self.roots_async_begin(sel)
            return
        _check(lib().shampoo_step(self.h, pa, ga, sp, sel, self._stream()), "shampoo_step")

    def roots_async_begin(self, part: int):
        _check(lib().shampoo_roots_async_begin(self.h, part, self._stream()),
               "shampoo_roots_async_begin")

    def roots_async_end(self):
        _check(lib().shampoo_roots_async_end(self.h, self._stream()), "shampoo_roots_async_end")

    def step_separate(self, params, grads, step: int, cadence: int, sparse=None):
        """The same step as three calls on one stream (no concurrency)."""
        sel = root_selector(step, cadence, self.cfg.root_parts)
        if self.async_roots:
            if sel >= 0:
                self.roots_async_end()
            self.update_stats(grads, sparse)
            self.precondition_and_apply(params, grads, sparse)
            if sel >= 0:
                self.roots_async_begin(sel)
            return
        self.update_stats(grads, sparse)
        if sel == ROOTS_ALL:
            self.compute_inverse_roots()
        elif sel >= 0:
            self.compute_inverse_roots_part(sel)
        self.precondition_and_apply(params, grads, sparse)

    def profile(self, on: bool = True):
        _check(lib().shampoo_profile_enable(self.h, 1 if on else 0), "shampoo_profile_enable")

    def profile_read(self):
        """{kernel family: (launches, total_ms)} since the last read."""
        out = (KernelTime * 64)()
        n = ctypes.c_int32()
        _check(lib().shampoo_profile_read(self.h, out, 64, ctypes.byref(n)), "shampoo_profile_read")
        return {out[i].name.decode(): (out[i].launches, out[i].total_ms) for i in range(n.value)}

    def diagnostics(self) -> List[FactorDiag]:
        out = (FactorDiag * max(self.n_factors, 1))()
        _check(lib().shampoo_get_diagnostics(self.h, out, self.n_factors, self._stream()),
               "shampoo_get_diagnostics")
        return list(out[: self.n_factors])

    # ---- views into the state buffer (for tests and inspection)
    def _view(self, off: int, shape, dtype):
        torch = self.torch
        es = torch.empty((), dtype=dtype).element_size()
        n = 1
        for s in shape:
            n *= s
        return self.state[off: off + n * es].view(dtype).view(*shape)

    def _sq(self, off: int, ld: int, n: int, dtype):
        # the n x n leading part of a padded square matrix, None when absent
        if off < 0:
            return None
        return self._view(off, (ld, ld), dtype)[:n, :n]

    def stats(self, b: int, raw: bool = False):
        """L, R of block b (None for the side a one-sided block does not
        keep).  The library maintains the upper triangle of each symmetric
        factor (a one-sided factor also its lower one); unless raw=True the
        full matrix is rebuilt from the upper triangle (a copy)."""
        bl = self.block(b)
        f64 = self.torch.float64
        L = self._sq(bl.off_l, bl.ld_l, bl.rows, f64)
        R = self._sq(bl.off_r, bl.ld_r, bl.cols, f64)
        if raw:
            return L, R
        sym = lambda x: None if x is None else self.torch.triu(x) + self.torch.triu(x, 1).T
        return sym(L), sym(R)

    def roots(self, b: int, fp64: bool = False):
        bl = self.block(b)
        if fp64:
            if bl.off_pl64 < 0 and bl.off_pr64 < 0:
                return None, None
            dt, ol, orr = self.torch.float64, bl.off_pl64, bl.off_pr64
        else:
            dt, ol, orr = self.torch.float32, bl.off_pl, bl.off_pr
        return self._sq(ol, bl.ld_l, bl.rows, dt), self._sq(orr, bl.ld_r, bl.cols, dt)

    def accumulators(self, t: int):
        a_off, m_off, _, _ = self.tensor(t)
        r, c, _ = self.shapes[t]
        a = self._view(a_off, (r, c), self.torch.float32)
        m = self._view(m_off, (r, c), self.torch.float32) if m_off >= 0 else None
        return a, m
