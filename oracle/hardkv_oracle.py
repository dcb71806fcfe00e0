"""ctypes wrapper of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this module.  It knows nothing of the HIP library: it sizes its own
host buffers from a workload description (any object with the workload
attributes) and calls the plain C definition in ``hardkv_oracle.c``.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_hardkv.so")
BK = 64

_lib = None


class OrcCfg(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("elem_bytes", C.c_int32), ("dense_window", C.c_int32),
        ("pool_blocks", C.c_int32), ("sparse_cap", C.c_int32), ("view_cap", C.c_int32),
        ("condensed_slots", C.c_int32), ("cond_mode", C.c_int32), ("merge_bias", C.c_int32),
        ("top_p", C.c_double), ("tau", C.POINTER(C.c_float)),
        ("regularize", C.c_int32), ("mti_lower", C.c_int32), ("mti_upper", C.c_int32),
        ("view_layout", C.c_int32), ("view_total", C.c_int32),
        ("calibration", C.c_int32), ("tau_unit", C.POINTER(C.c_float)), ("sink", C.c_int32),
        ("mti_horizon", C.c_int32), ("mti_c_view", C.c_uint32), ("mti_c_write", C.c_uint32),
        ("mti_c_scan", C.c_uint32), ("mti_c_hold", C.c_uint32), ("mti_c_score", C.c_uint32),
        ("mti_c_gather", C.c_uint32 * 9), ("mti_fixed", C.c_int64),
        ("selection", C.c_int32),
    ]

# selection modes: a view of the whole pool at every selection, or destructive (a selection
# drops for good the survivors it does not keep)
SEL_VIEW, SEL_DESTRUCTIVE = 0, 1

MTI_FIELDS = ("mti_horizon", "mti_c_view", "mti_c_write", "mti_c_scan", "mti_c_hold", "mti_c_score",
              "mti_c_gather", "mti_fixed")


def set_mti(cfg, mti: Optional[dict]) -> None:
    """Copies the memory-time controller's inputs (a dict with MTI_FIELDS keys, mti_c_gather a
    sequence of 9) into an OrcCfg."""
    if not mti:
        return
    for k, v in mti.items():
        if k == "mti_c_gather":
            arr = (C.c_uint32 * 9)(*[int(x) for x in v])
            setattr(cfg, k, arr)
        else:
            setattr(cfg, k, int(v))


class OrcState(C.Structure):
    _fields_ = [
        ("dense_k", C.c_void_p), ("dense_v", C.c_void_p), ("pool_k", C.c_void_p),
        ("pool_v", C.c_void_p), ("view_k", C.c_void_p), ("view_v", C.c_void_p),
        ("view_pos", C.c_void_p), ("cond_kn", C.c_void_p), ("cond_vn", C.c_void_p),
        ("cond_omega", C.c_void_p), ("cond_n", C.c_void_p), ("cond_cursor", C.c_void_p),
        ("seq_len", C.c_void_p), ("pool_head", C.c_void_p), ("scores", C.c_void_p),
        ("weights", C.c_void_p), ("mask", C.c_void_p), ("budget", C.c_void_p),
        ("n_condense", C.c_void_p), ("w_all", C.c_void_p), ("w_u", C.c_void_p),
        ("thresh", C.c_void_p), ("regularized", C.c_void_p), ("view_off", C.c_void_p),
        ("tau_fit", C.c_void_p), ("error_word", C.c_uint32), ("sink_k", C.c_void_p), ("sink_v", C.c_void_p),
        ("pend_sel", C.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b  # noqa: F401  (relative import when used as package)
        L = C.CDLL(LIB_PATH)
        f, u32, i32, i64, d = C.c_float, C.c_uint32, C.c_int32, C.c_int64, C.c_double
        vp = C.c_void_p
        L.orc_dot_pairwise.restype = f
        L.orc_dot_pairwise.argtypes = [vp, vp, i32]
        L.orc_score_row.restype = f
        L.orc_score_row.argtypes = [vp, i32, vp, i32]
        L.orc_kappa.restype = f
        L.orc_kappa.argtypes = [i32, f]
        L.orc_fit_tau.restype = f
        L.orc_fit_tau.argtypes = [vp, i32, vp, i64, i32, C.POINTER(d)]
        L.orc_calibrated_entropy.restype = d
        L.orc_calibrated_entropy.argtypes = [vp, i64, i32, d]
        L.orc_poly_coeff.restype = f
        L.orc_poly_coeff.argtypes = [i32]
        L.orc_exp2_poly.restype = f
        L.orc_exp2_poly.argtypes = [f]
        L.orc_exp2_poly_batch.restype = None
        L.orc_exp2_poly_batch.argtypes = [vp, vp, i64]
        L.orc_weight.restype = u32
        L.orc_weight.argtypes = [f, f, f]
        L.orc_weight_batch.restype = None
        L.orc_weight_batch.argtypes = [vp, vp, i64]
        L.orc_pq.restype = u32
        L.orc_pq.argtypes = [d]
        L.orc_topp.restype = i32
        L.orc_topp.argtypes = [vp, vp, i32, u32, vp, vp]
        L.orc_prefill.restype = i32
        L.orc_prefill.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcState), vp, vp, vp, i64]
        L.orc_step.restype = i32
        L.orc_step.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcState), vp, vp, vp, vp, i32, i32]
        L.orc_step_reuse.restype = i32
        L.orc_step_reuse.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcState), vp, vp, vp, vp, i32]
        L.orc_mti_rewrite.restype = i32
        L.orc_mti_rewrite.argtypes = [C.POINTER(OrcCfg), i64, i64]
        L.orc_mti_thresholds.restype = None
        L.orc_mti_thresholds.argtypes = [C.POINTER(OrcCfg), i64, C.POINTER(i64), C.POINTER(i64)]
        L.orc_mti_period.restype = i32
        L.orc_mti_period.argtypes = [C.POINTER(OrcCfg), i64, i64, i64, i32]
        L.orc_select_ahead.restype = i32
        L.orc_select_ahead.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcState), vp]
        L.orc_condense_plan.restype = i32
        L.orc_condense_plan.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcState)]
        L.orc_full_attention.restype = None
        L.orc_full_attention.argtypes = [vp, vp, vp, i32, i32, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _store_np(x) -> np.ndarray:
    """A torch tensor or numpy array in storage type -> contiguous numpy (bf16 as uint16)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


# ---- building blocks --------------------------------------------------------------------
def dot_pairwise(a: np.ndarray, b: np.ndarray) -> np.float32:
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return np.float32(lib().orc_dot_pairwise(_p(a), _p(b), a.size))


def score_row(q: np.ndarray, k: np.ndarray) -> np.float32:
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    return np.float32(lib().orc_score_row(_p(q), q.shape[0], _p(k), k.size))


def kappa(D: int, tau: float) -> np.float32:
    return np.float32(lib().orc_kappa(D, tau))


def poly_coeffs() -> np.ndarray:
    return np.array([lib().orc_poly_coeff(i) for i in range(10)], np.float32)


def exp2_poly(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, np.float32)
    y = np.empty_like(f)
    lib().orc_exp2_poly_batch(_p(f), _p(y), f.size)
    return y


def weight(s: float, m: float, kap: float) -> int:
    return int(lib().orc_weight(s, m, kap))


def weight_of_t(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, np.float32)
    w = np.empty(t.shape, np.uint32)
    lib().orc_weight_batch(_p(t), _p(w), t.size)
    return w


def fit_tau(d: np.ndarray, s: np.ndarray, D: int = 128):
    """Entropy-matched temperature: d are the [G, n] raw dot products, s the n max-pooled
    scores; returns (tau, target entropy in nats)."""
    d = np.ascontiguousarray(d, np.float32)
    s = np.ascontiguousarray(s, np.float32)
    h = C.c_double(0.0)
    tau = lib().orc_fit_tau(_p(d), int(d.shape[0]), _p(s), int(s.shape[0]), D, C.byref(h))
    return float(tau), float(h.value)


def calibrated_entropy(s: np.ndarray, tau: float, D: int = 128) -> float:
    s = np.ascontiguousarray(s, np.float32)
    return float(lib().orc_calibrated_entropy(_p(s), int(s.shape[0]), D, float(tau)))


def pq(p: float) -> int:
    return int(lib().orc_pq(p))


def topp(w: np.ndarray, pos: np.ndarray, p: float):
    """Returns (k*, selected flags, T) for survivor weights w at positions pos."""
    w = np.ascontiguousarray(w, np.uint32)
    pos = np.ascontiguousarray(pos, np.int64)
    sel = np.zeros(max(w.size, 1), np.uint8)
    T = np.zeros(1, np.uint64)
    k = lib().orc_topp(_p(w), _p(pos), w.size, lib().orc_pq(p), _p(sel), _p(T))
    return int(k), sel[:w.size].astype(bool), int(T[0])


def _mti_cfg(mti: dict) -> OrcCfg:
    cfg = OrcCfg()
    cfg.regularize = 3
    set_mti(cfg, mti)
    return cfg


def mti_rewrite(mti: dict, kstar: int, n: int) -> bool:
    """The memory-time controller's decision for a head with kstar kept of n survivors."""
    return bool(lib().orc_mti_rewrite(C.byref(_mti_cfg(mti)), int(kstar), int(n)))


def mti_thresholds(mti: dict, n: int):
    """(L_lower, L_upper): the smallest and largest rewritten budgets in [1, n] ((0, -1): none)."""
    lo, hi = C.c_int64(0), C.c_int64(0)
    lib().orc_mti_thresholds(C.byref(_mti_cfg(mti)), int(n), C.byref(lo), C.byref(hi))
    return int(lo.value), int(hi.value)


def mti_period(mti: dict, n_pool: int, n: int, kstar: int, max_period: int) -> int:
    """Steps per selection in [1, max_period] with the least memory time per step."""
    return int(lib().orc_mti_period(C.byref(_mti_cfg(mti)), int(n_pool), int(n), int(kstar), int(max_period)))


def full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    out = np.zeros(q.size, np.float64)
    lib().orc_full_attention(_p(q), _p(k), _p(v), k.shape[0], q.size, _p(out))
    return out


# ---- the step -----------------------------------------------------------------------------
class Oracle:
    """Host state of one layer and the oracle's step on it.

    ``wl`` provides: batch, num_q_heads, num_kv_heads, head_dim, elem_bytes,
    dense_window, P_blk, sparse_cap, V_cap, condensed_slots, cond_mode, top_p.
    """

    def __init__(self, wl, tau: Optional[np.ndarray] = None, merge_bias: bool = True,
                 top_p: Optional[float] = None, regularize: int = 0, mti_lower: int = 0,
                 mti_upper: int = 0, view_layout: int = 0, view_total: int = 0,
                 calibration: int = 0, tau_unit: Optional[np.ndarray] = None,
                 mti: Optional[dict] = None, selection: int = SEL_VIEW):
        self.wl = wl
        B, H, Hq, D = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim
        W, P, V, Cs = wl.dense_window, wl.P_blk, wl.V_cap, wl.condensed_slots
        st = np.uint16 if wl.elem_bytes == 2 else np.float32
        self.tau = np.ascontiguousarray(
            np.full(H, wl.tau, np.float32) if tau is None else np.asarray(tau, np.float32))
        self.cfg = OrcCfg(B, Hq, H, D, wl.elem_bytes, W, P, wl.sparse_cap, V, Cs, wl.cond_mode,
                          1 if merge_bias else 0, float(wl.top_p if top_p is None else top_p),
                          self.tau.ctypes.data_as(C.POINTER(C.c_float)), int(regularize),
                          int(mti_lower), int(mti_upper), int(view_layout), int(view_total),
                          int(calibration), None, int(getattr(wl, "sink", 0)))
        set_mti(self.cfg, mti)
        if selection not in (SEL_VIEW, SEL_DESTRUCTIVE):
            raise ValueError(f"selection mode {selection}")
        if selection == SEL_DESTRUCTIVE and calibration != 0:
            raise ValueError("destructive selection takes a fixed temperature")
        self.cfg.selection = int(selection)
        self.tau_unit = None
        if tau_unit is not None:
            self.tau_unit = np.ascontiguousarray(np.asarray(tau_unit, np.float32).ravel())
            self.cfg.tau_unit = self.tau_unit.ctypes.data_as(C.POINTER(C.c_float))
        S = int(getattr(wl, "sink", 0))
        self.sink_k = np.zeros((B, H, max(S, 1), D), st)
        self.sink_v = np.zeros((B, H, max(S, 1), D), st)
        self.dense_k = np.zeros((B, H, W, D), st)
        self.dense_v = np.zeros((B, H, W, D), st)
        self.pool_k = np.zeros((B, H, P, BK, D), st)
        self.pool_v = np.zeros((B, H, P, BK, D), st)
        if view_layout == 1:  # packed (CSR) views
            Vt = max(1, view_total)
            self.view_k = np.zeros((Vt, D), st)
            self.view_v = np.zeros((Vt, D), st)
            self.view_pos = np.full(Vt, -1, np.int32)
        else:
            self.view_k = np.zeros((B, H, V, D), st)
            self.view_v = np.zeros((B, H, V, D), st)
            self.view_pos = np.full((B, H, V), -1, np.int32)
        self.view_off = np.zeros(B * H + 1, np.int32)
        self.tau_fit = np.zeros((B, H), np.float32)
        self.cond_kn = np.zeros((B, H, Cs, D), np.float64)
        self.cond_vn = np.zeros((B, H, Cs, D), np.float64)
        self.cond_omega = np.zeros((B, H, Cs), np.float64)
        self.cond_n = np.zeros((B, H, Cs), np.int32)
        self.cond_cursor = np.zeros((B, H), np.int32)
        self.seq_len = np.zeros(B, np.int64)
        self.pool_head = np.zeros((B, H), np.int64)
        self.scores = np.zeros((B, H, P * BK), np.float32)
        self.weights = np.zeros((B, H, P * BK), np.uint32)
        self.mask = np.zeros((B, H, P), np.uint64)
        self.budget = np.zeros((B, H), np.int32)
        self.n_condense = np.zeros((B, H), np.int32)
        self.w_all = np.zeros((B, H), np.uint64)
        self.w_u = np.zeros((B, H), np.uint64)
        self.thresh = np.zeros((B, H), np.uint64)
        self.regularized = np.zeros((B, H), np.int32)
        self.pend_sel = np.zeros((B, H), np.int64)
        self.st = OrcState(*[_p(getattr(self, n)) for n in (
            "dense_k", "dense_v", "pool_k", "pool_v", "view_k", "view_v", "view_pos", "cond_kn",
            "cond_vn", "cond_omega", "cond_n", "cond_cursor", "seq_len", "pool_head", "scores",
            "weights", "mask", "budget", "n_condense", "w_all", "w_u", "thresh", "regularized",
            "view_off", "tau_fit")], 0, _p(self.sink_k), _p(self.sink_v), _p(self.pend_sel))

    @property
    def error_word(self) -> int:
        return int(self.st.error_word)

    def prefill(self, k_ctx, v_ctx, ctx_len) -> int:
        k = _store_np(k_ctx)
        v = _store_np(v_ctx)
        L = np.ascontiguousarray(np.asarray(ctx_len.cpu() if hasattr(ctx_len, "cpu") else ctx_len, np.int64))
        return lib().orc_prefill(C.byref(self.cfg), C.byref(self.st), _p(k), _p(v), _p(L), k.shape[2])

    def step(self, q, k_new, v_new, attend: bool = True, nthreads: int = 0) -> np.ndarray:
        qn, kn, vn = _store_np(q), _store_np(k_new), _store_np(v_new)
        out = np.zeros((self.wl.batch, self.wl.num_q_heads, self.wl.head_dim), np.float64)
        rc = lib().orc_step(C.byref(self.cfg), C.byref(self.st), _p(qn), _p(kn), _p(vn), _p(out),
                            1 if attend else 0, nthreads)
        if rc != 0:
            raise RuntimeError(f"orc_step failed: {rc}")
        return out

    def step_reuse(self, q, k_new, v_new, nthreads: int = 0) -> np.ndarray:
        """A step that keeps the last selection: append, then attention over the sinks,
        condensed slots, the last selection's kept rows, the pool positions since it, and
        the dense window."""
        qn, kn, vn = _store_np(q), _store_np(k_new), _store_np(v_new)
        out = np.zeros((self.wl.batch, self.wl.num_q_heads, self.wl.head_dim), np.float64)
        rc = lib().orc_step_reuse(C.byref(self.cfg), C.byref(self.st), _p(qn), _p(kn), _p(vn), _p(out),
                                  nthreads)
        if rc != 0:
            raise RuntimeError(f"orc_step_reuse failed: {rc}")
        return out

    # the asynchronous pipeline -----------------------------------------------------------
    SHARED = ("dense_k", "dense_v", "pool_k", "pool_v", "cond_kn", "cond_vn", "cond_omega", "cond_n",
              "cond_cursor", "pool_head", "sink_k", "sink_v")

    def twin(self) -> "Oracle":
        """A state for a selection made ahead: it shares this one's pool, dense and sink rows,
        condensed tier and pool head, and has its own step counter and selection buffers."""
        o = Oracle.__new__(Oracle)
        o.__dict__.update({k: v for k, v in self.__dict__.items()})
        for n in ("view_k", "view_v", "view_pos", "view_off", "tau_fit", "scores", "weights", "mask", "budget",
                  "n_condense", "w_all", "w_u", "thresh", "regularized", "pend_sel", "seq_len"):
            setattr(o, n, getattr(self, n).copy())
        o.st = OrcState(*[_p(getattr(o, n)) for n in (
            "dense_k", "dense_v", "pool_k", "pool_v", "view_k", "view_v", "view_pos", "cond_kn",
            "cond_vn", "cond_omega", "cond_n", "cond_cursor", "seq_len", "pool_head", "scores",
            "weights", "mask", "budget", "n_condense", "w_all", "w_u", "thresh", "regularized",
            "view_off", "tau_fit")], 0, _p(o.sink_k), _p(o.sink_v), _p(o.pend_sel))
        for n in self.SHARED:
            assert getattr(o, n) is getattr(self, n)
        return o

    def select_ahead(self, q, t_snapshot) -> None:
        """The selection made ahead for the step whose append left seq_len = t_snapshot."""
        self.seq_len[:] = np.asarray(t_snapshot, np.int64)
        rc = lib().orc_select_ahead(C.byref(self.cfg), C.byref(self.st), _p(_store_np(q)))
        if rc != 0:
            raise RuntimeError(f"orc_select_ahead failed: {rc}")

    def condense_plan(self) -> None:
        """The switch: the planned condensation of the selection made ahead."""
        lib().orc_condense_plan(C.byref(self.cfg), C.byref(self.st))

    # logical views used by the tests ----------------------------------------------------
    def pool_row_index(self, p: np.ndarray) -> np.ndarray:
        P = self.wl.P_blk
        return (p // BK) % P * BK + p % BK

    def selected_positions(self, b: int, h: int) -> np.ndarray:
        """The kept positions in ascending order, from the mask words (valid whether or not
        the head was rewritten this step)."""
        P = self.wl.P_blk
        c = int(self.pool_head[b, h]) - BK * int(self.n_condense[b, h])  # pool head before condensing
        t = int(self.seq_len[b])
        pend = max(int(getattr(self.wl, "sink", 0)), t - self.wl.dense_window)
        p = np.arange(c, pend, dtype=np.int64)
        words = self.mask[b, h][(p // BK) % P]
        bits = (words >> (p % BK).astype(np.uint64)) & np.uint64(1)
        return p[bits.astype(bool)]
