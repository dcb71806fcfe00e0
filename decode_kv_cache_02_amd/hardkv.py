"""Python binding of libhardkv.so: argument marshalling only.

Every function here has the name of the C entry point it calls and passes tensor
data pointers and the current HIP stream; all computation runs in the HIP kernels
of the library.  PyTorch only allocates device memory and provides the stream.
If the library is missing, or there is no GPU, calls fail loudly.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhardkv.so")

HARDKV_OK, HARDKV_EINVAL, HARDKV_EUNSUPPORTED, HARDKV_ECAPACITY, HARDKV_EHIP, HARDKV_ESCRATCH = 0, -1, -2, -3, -4, -5
HARDKV_STATIC_SCRATCH_BYTES = 128 << 20
HARDKV_BF16, HARDKV_F32 = 0, 1
HARDKV_COND_OFF, HARDKV_COND_EVICT, HARDKV_COND_MERGE = 0, 1, 2
HARDKV_REG_REWRITE, HARDKV_REG_SPARSE, HARDKV_REG_MTI, HARDKV_REG_MTI_AUTO = 0, 1, 2, 3
# the memory-time controller's default costs (fs per row of K and V; the header's
# HARDKV_MTI_C_* values, measured with this library's kernels on a bf16 layer)
MTI_DEFAULT = dict(mti_horizon=0, mti_c_view=97000, mti_c_write=68000, mti_c_scan=0, mti_c_hold=0,
                   mti_c_score=44000, mti_c_gather=[124000] * 9, mti_fixed=0)
HARDKV_VIEW_MAXLEN, HARDKV_VIEW_SUM = 0, 1
HARDKV_POOL_RING, HARDKV_POOL_SHARED = 0, 1
HARDKV_SEL_VIEW, HARDKV_SEL_DESTRUCTIVE = 0, 1
HARDKV_CAL_FIXED, HARDKV_CAL_ENTROPY = 0, 1
HARDKV_ERR_POOL_OVERFLOW, HARDKV_ERR_VIEW_OVERFLOW, HARDKV_ERR_NONFINITE = 1, 2, 4
BLOCK, HEAD_DIM = 64, 128

EXPORTS = ("hardkv_workspace_size", "hardkv_prefill", "hardkv_append", "hardkv_select",
           "hardkv_regularize", "hardkv_condense", "hardkv_attend", "hardkv_attend_sparse", "hardkv_step",
           "hardkv_step_reuse", "hardkv_step_noalloc", "hardkv_step_stage", "hardkv_step_num_stages", "hardkv_step_stage_name",
           "hardkv_mti_thresholds", "hardkv_mti_period", "hardkv_select_fork", "hardkv_select_ahead",
           "hardkv_shared_pool_blocks",
           "hardkv_strerror")


class HardKVError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


class hardkv_config(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("dtype", C.c_int32), ("dense_window", C.c_int32),
        ("pool_blocks", C.c_int32), ("sparse_cap", C.c_int32), ("view_cap", C.c_int32),
        ("condensed_slots", C.c_int32), ("cond_mode", C.c_int32), ("merge_bias", C.c_int32),
        ("top_p", C.c_double), ("tau", C.POINTER(C.c_float)),
        ("regularize", C.c_int32), ("mti_lower", C.c_int32), ("mti_upper", C.c_int32),
        ("view_layout", C.c_int32), ("view_total", C.c_int32), ("calibration", C.c_int32),
        ("sink", C.c_int32),
        ("mti_horizon", C.c_int32), ("mti_c_view", C.c_uint32), ("mti_c_write", C.c_uint32),
        ("mti_c_scan", C.c_uint32), ("mti_c_hold", C.c_uint32), ("mti_c_score", C.c_uint32),
        ("mti_c_gather", C.c_uint32 * 9), ("mti_fixed", C.c_int64),
        ("pool_layout", C.c_int32), ("pool_total_blocks", C.c_int32), ("selection", C.c_int32),
    ]


_STATE_FIELDS = ("dense_k", "dense_v", "pool_k", "pool_v", "view_k", "view_v", "view_pos",
                 "cond_kn", "cond_vn", "cond_omega", "cond_n", "cond_cursor", "seq_len",
                 "pool_head", "scores", "weights", "mask", "budget", "n_condense", "w_all",
                 "w_u", "thresh", "regularized", "view_off", "tau_fit", "sink_k", "sink_v", "error_word",
                 "workspace")


# the shared block pool's table and free list (after workspace_bytes in the struct)
_STATE_POOL_FIELDS = ("block_table", "free_list", "free_top")
_STATE_PTRS = _STATE_FIELDS + _STATE_POOL_FIELDS


class hardkv_state(C.Structure):
    _fields_ = ([(n, C.c_void_p) for n in _STATE_FIELDS] + [("workspace_bytes", C.c_size_t)] +
                [(n, C.c_void_p) for n in _STATE_POOL_FIELDS])


_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -m decode_kv_cache_02_amd.build`")
        L = C.CDLL(LIB_PATH)
        cp, sp, vp, i32, i64 = C.POINTER(hardkv_config), C.POINTER(hardkv_state), C.c_void_p, C.c_int32, C.c_int64
        L.hardkv_workspace_size.argtypes = [cp, C.POINTER(C.c_size_t)]
        L.hardkv_prefill.argtypes = [cp, sp, vp, vp, vp, i64, vp]
        L.hardkv_append.argtypes = [cp, sp, vp, vp, vp]
        L.hardkv_select.argtypes = [cp, sp, vp, vp]
        L.hardkv_regularize.argtypes = [cp, sp, vp]
        L.hardkv_condense.argtypes = [cp, sp, vp]
        L.hardkv_attend.argtypes = [cp, sp, vp, vp, vp]
        L.hardkv_attend_sparse.argtypes = [cp, sp, vp, vp, vp]
        L.hardkv_step.argtypes = [cp, sp, vp, vp, vp, vp, vp]
        L.hardkv_step_reuse.argtypes = [cp, sp, vp, vp, vp, vp, vp]
        L.hardkv_step_noalloc.argtypes = [cp, sp, vp, vp, vp, vp, vp]
        L.hardkv_step_stage.argtypes = [cp, sp, vp, vp, vp, vp, i32, vp]
        L.hardkv_step_num_stages.argtypes = []
        L.hardkv_mti_thresholds.argtypes = [cp, i64, C.POINTER(i32), C.POINTER(i32)]
        L.hardkv_select_fork.argtypes = [cp, sp, sp, vp]
        L.hardkv_select_ahead.argtypes = [cp, sp, vp, i32, i32, vp]
        L.hardkv_mti_period.argtypes = [cp, i64, i64, i64, i32, C.POINTER(i32)]
        L.hardkv_shared_pool_blocks.argtypes = [cp, C.POINTER(i64), i64, C.POINTER(i64)]
        L.hardkv_step_stage_name.argtypes = [i32]
        L.hardkv_step_stage_name.restype = C.c_char_p
        L.hardkv_strerror.argtypes = [i32]
        L.hardkv_strerror.restype = C.c_char_p
        for n in EXPORTS:
            if n not in ("hardkv_step_stage_name", "hardkv_strerror"):
                getattr(L, n).restype = i32
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().hardkv_strerror(code).decode()


def _check(fn: str, rc: int) -> None:
    if rc != HARDKV_OK:
        raise HardKVError(fn, rc)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhardkv must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---- configuration and state ----------------------------------------------------------------
class Config:
    """hardkv_config plus the host array of per-head temperatures it points to."""

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, dtype: str,
                 dense_window: int, pool_blocks: int, sparse_cap: int, view_cap: int,
                 condensed_slots: int, cond_mode: int, top_p: float,
                 tau: Sequence[float], head_dim: int = HEAD_DIM, merge_bias: bool = True,
                 regularize: int = HARDKV_REG_REWRITE, mti_lower: int = 0, mti_upper: int = 0,
                 view_layout: int = HARDKV_VIEW_MAXLEN, view_total: int = 0,
                 calibration: int = HARDKV_CAL_FIXED, sink: int = 0, mti: Optional[dict] = None,
                 pool_layout: int = HARDKV_POOL_RING, pool_total_blocks: int = 0,
                 selection: int = HARDKV_SEL_VIEW):
        self.tau_arr = (C.c_float * max(1, len(tau)))(*[float(x) for x in tau])
        self.c = hardkv_config(batch, num_q_heads, num_kv_heads, head_dim,
                               HARDKV_BF16 if dtype == "bf16" else HARDKV_F32, dense_window,
                               pool_blocks, sparse_cap, view_cap, condensed_slots, cond_mode,
                               1 if merge_bias else 0, float(top_p),
                               C.cast(self.tau_arr, C.POINTER(C.c_float)),
                               int(regularize), int(mti_lower), int(mti_upper),
                               int(view_layout), int(view_total), int(calibration), int(sink))
        m = dict(MTI_DEFAULT)
        m.update(mti or {})
        for k, v in m.items():
            setattr(self.c, k, (C.c_uint32 * 9)(*[int(x) for x in v]) if k == "mti_c_gather" else int(v))
        self.c.pool_layout = int(pool_layout)
        self.c.pool_total_blocks = int(pool_total_blocks)
        self.c.selection = int(selection)
        self.dtype = dtype

    @classmethod
    def from_workload(cls, wl, top_p: Optional[float] = None, tau=None, cond_mode=None,
                      merge_bias: bool = True, regularize: int = HARDKV_REG_REWRITE,
                      mti_lower: int = 0, mti_upper: int = 0, view_layout: int = HARDKV_VIEW_MAXLEN,
                      view_total: int = 0, calibration: int = HARDKV_CAL_FIXED,
                      sink: Optional[int] = None, mti: Optional[dict] = None,
                      pool_layout: int = HARDKV_POOL_RING, pool_total_blocks: int = 0,
                      selection: int = HARDKV_SEL_VIEW) -> "Config":
        return cls(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.dtype, wl.dense_window, wl.P_blk,
                   wl.sparse_cap, wl.V_cap, wl.condensed_slots,
                   wl.cond_mode if cond_mode is None else cond_mode,
                   wl.top_p if top_p is None else top_p,
                   [wl.tau] * wl.num_kv_heads if tau is None else list(tau),
                   head_dim=wl.head_dim, merge_bias=merge_bias, regularize=regularize,
                   mti_lower=mti_lower, mti_upper=mti_upper, view_layout=view_layout,
                   view_total=view_total, calibration=calibration,
                   sink=int(getattr(wl, "sink", 0)) if sink is None else int(sink), mti=mti,
                   pool_layout=pool_layout, pool_total_blocks=pool_total_blocks, selection=selection)

    def __getattr__(self, name):
        return getattr(self.__dict__["c"], name)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.c.dtype == HARDKV_BF16 else torch.float32


def hardkv_workspace_size(cfg: Config) -> int:
    n = C.c_size_t(0)
    _check("hardkv_workspace_size", lib().hardkv_workspace_size(C.byref(cfg.c), C.byref(n)))
    return int(n.value)


class State:
    """Device buffers of one layer, allocated as tensors, and the hardkv_state pointing at them."""

    def __init__(self, cfg: Config, device="cuda"):
        c = cfg.c
        B, H, W, P, V, Cs, D = (c.batch, c.num_kv_heads, c.dense_window, c.pool_blocks, c.view_cap,
                                c.condensed_slots, c.head_dim)
        dt = cfg.torch_dtype
        kw = dict(device=device)
        self.cfg = cfg
        self.dense_k = torch.zeros((B, H, W, D), dtype=dt, **kw)
        self.dense_v = torch.zeros((B, H, W, D), dtype=dt, **kw)
        if c.pool_layout == HARDKV_POOL_SHARED:  # physical blocks, a table per unit, a free list
            NB = c.pool_total_blocks
            self.pool_k = torch.zeros((NB, BLOCK, D), dtype=dt, **kw)
            self.pool_v = torch.zeros((NB, BLOCK, D), dtype=dt, **kw)
            self.block_table = torch.full((B, H, P), -1, dtype=torch.int32, **kw)
            self.free_list = torch.zeros((NB,), dtype=torch.int32, **kw)
            self.free_top = torch.zeros((4,), dtype=torch.int32, **kw)
        else:
            self.pool_k = torch.zeros((B, H, P, BLOCK, D), dtype=dt, **kw)
            self.pool_v = torch.zeros((B, H, P, BLOCK, D), dtype=dt, **kw)
            self.block_table = self.free_list = self.free_top = None
        if c.view_layout == HARDKV_VIEW_SUM:   # packed (CSR) views of view_total rows
            Vt = max(1, c.view_total)
            self.view_k = torch.zeros((Vt, D), dtype=dt, **kw)
            self.view_v = torch.zeros((Vt, D), dtype=dt, **kw)
            self.view_pos = torch.full((Vt,), -1, dtype=torch.int32, **kw)
        else:
            self.view_k = torch.zeros((B, H, V, D), dtype=dt, **kw)
            self.view_v = torch.zeros((B, H, V, D), dtype=dt, **kw)
            self.view_pos = torch.full((B, H, V), -1, dtype=torch.int32, **kw)
        self.view_off = torch.zeros((B * H + 1,), dtype=torch.int32, **kw)
        self.tau_fit = torch.zeros((B, H), dtype=torch.float32, **kw)
        self.sink_k = torch.zeros((B, H, max(1, c.sink), D), dtype=dt, **kw)  # sink position p in row p
        self.sink_v = torch.zeros((B, H, max(1, c.sink), D), dtype=dt, **kw)
        self.cond_kn = torch.zeros((B, H, Cs, D), dtype=torch.float32, **kw)
        self.cond_vn = torch.zeros((B, H, Cs, D), dtype=torch.float32, **kw)
        self.cond_omega = torch.zeros((B, H, Cs), dtype=torch.float32, **kw)
        self.cond_n = torch.zeros((B, H, Cs), dtype=torch.int32, **kw)
        self.cond_cursor = torch.zeros((B, H), dtype=torch.int32, **kw)
        self.seq_len = torch.zeros((B,), dtype=torch.int64, **kw)
        self.pool_head = torch.zeros((B, H), dtype=torch.int64, **kw)
        self.scores = torch.zeros((B, H, P * BLOCK), dtype=torch.float32, **kw)
        self.weights = torch.zeros((B, H, P * BLOCK), dtype=torch.int32, **kw)   # uint32 bits
        self.mask = torch.zeros((B, H, P), dtype=torch.int64, **kw)               # uint64 bits
        self.budget = torch.zeros((B, H), dtype=torch.int32, **kw)
        self.n_condense = torch.zeros((B, H), dtype=torch.int32, **kw)
        self.w_all = torch.zeros((B, H), dtype=torch.int64, **kw)
        self.w_u = torch.zeros((B, H), dtype=torch.int64, **kw)
        self.thresh = torch.zeros((B, H), dtype=torch.int64, **kw)
        self.regularized = torch.zeros((B, H), dtype=torch.int32, **kw)
        self.error_word = torch.zeros((4,), dtype=torch.int32, **kw)
        self.workspace_bytes = hardkv_workspace_size(cfg)
        self.workspace = torch.zeros((self.workspace_bytes,), dtype=torch.uint8, **kw)
        self._bind()

    def _bind(self):
        self.c = hardkv_state(*[_ptr(getattr(self, n)) for n in _STATE_FIELDS], self.workspace_bytes,
                              *[_ptr(getattr(self, n)) for n in _STATE_POOL_FIELDS])

    # buffers that hold the cache itself, shared by the two states of the pipeline
    SHARED = ("dense_k", "dense_v", "pool_k", "pool_v", "sink_k", "sink_v", "cond_kn", "cond_vn", "cond_omega",
              "cond_n", "cond_cursor", "seq_len", "pool_head", "error_word") + _STATE_POOL_FIELDS

    def twin(self) -> "State":
        """A state for a selection made ahead (hardkv_select_fork / hardkv_select_ahead): the
        same cache buffers, its own selection buffers and workspace."""
        o = State.__new__(State)
        o.cfg = self.cfg
        for n in _STATE_PTRS:
            t = getattr(self, n)
            setattr(o, n, t if (n in self.SHARED or t is None) else torch.zeros_like(t))
        o.view_pos.fill_(-1)
        o.workspace_bytes = self.workspace_bytes
        o._bind()
        return o

    def tensors(self):
        return {n: getattr(self, n) for n in _STATE_PTRS if getattr(self, n) is not None}


# ---- entry points ----------------------------------------------------------------------------
def hardkv_prefill(cfg: Config, st: State, k_ctx: torch.Tensor, v_ctx: torch.Tensor,
                   ctx_len: torch.Tensor, stream=None) -> None:
    _check("hardkv_prefill", lib().hardkv_prefill(C.byref(cfg.c), C.byref(st.c), _ptr(k_ctx), _ptr(v_ctx),
                                                  _ptr(ctx_len), int(k_ctx.shape[2]), _stream(stream)))


def hardkv_append(cfg: Config, st: State, k_new, v_new, stream=None) -> None:
    _check("hardkv_append", lib().hardkv_append(C.byref(cfg.c), C.byref(st.c), _ptr(k_new), _ptr(v_new),
                                                _stream(stream)))


def hardkv_select(cfg: Config, st: State, q, stream=None) -> None:
    _check("hardkv_select", lib().hardkv_select(C.byref(cfg.c), C.byref(st.c), _ptr(q), _stream(stream)))


def hardkv_regularize(cfg: Config, st: State, stream=None) -> None:
    _check("hardkv_regularize", lib().hardkv_regularize(C.byref(cfg.c), C.byref(st.c), _stream(stream)))


def hardkv_condense(cfg: Config, st: State, stream=None) -> None:
    _check("hardkv_condense", lib().hardkv_condense(C.byref(cfg.c), C.byref(st.c), _stream(stream)))


def hardkv_attend(cfg: Config, st: State, q, out, stream=None) -> None:
    _check("hardkv_attend", lib().hardkv_attend(C.byref(cfg.c), C.byref(st.c), _ptr(q), _ptr(out),
                                                _stream(stream)))


def hardkv_attend_sparse(cfg: Config, st: State, q, out, stream=None) -> None:
    _check("hardkv_attend_sparse", lib().hardkv_attend_sparse(C.byref(cfg.c), C.byref(st.c), _ptr(q),
                                                              _ptr(out), _stream(stream)))


def hardkv_step(cfg: Config, st: State, q, k_new, v_new, out, stream=None) -> None:
    _check("hardkv_step", lib().hardkv_step(C.byref(cfg.c), C.byref(st.c), _ptr(q), _ptr(k_new),
                                            _ptr(v_new), _ptr(out), _stream(stream)))


def hardkv_step_reuse(cfg: Config, st: State, q, k_new, v_new, out, stream=None) -> None:
    _check("hardkv_step_reuse", lib().hardkv_step_reuse(C.byref(cfg.c), C.byref(st.c), _ptr(q), _ptr(k_new),
                                                        _ptr(v_new), _ptr(out), _stream(stream)))


def hardkv_step_noalloc(cfg: Config, st: State, q, k_new, v_new, out, stream=None) -> None:
    """hardkv_step with the library's static scratch in place of the state's workspace."""
    _check("hardkv_step_noalloc", lib().hardkv_step_noalloc(C.byref(cfg.c), C.byref(st.c), _ptr(q), _ptr(k_new),
                                                            _ptr(v_new), _ptr(out), _stream(stream)))


def hardkv_step_stage(cfg: Config, st: State, q, k_new, v_new, out, stage: int, stream=None) -> None:
    _check("hardkv_step_stage", lib().hardkv_step_stage(C.byref(cfg.c), C.byref(st.c), _ptr(q), _ptr(k_new),
                                                        _ptr(v_new), _ptr(out), int(stage), _stream(stream)))


def hardkv_mti_thresholds(cfg: Config, n_survivors: int):
    """(L_lower, L_upper) of the memory-time controller for a head of n_survivors survivors."""
    lo, hi = C.c_int32(0), C.c_int32(0)
    _check("hardkv_mti_thresholds", lib().hardkv_mti_thresholds(C.byref(cfg.c), int(n_survivors), C.byref(lo),
                                                                C.byref(hi)))
    return int(lo.value), int(hi.value)


def hardkv_mti_period(cfg: Config, n_pool: int, n_survivors: int, kstar: int, max_period: int) -> int:
    """Steps per selection with the least memory time per step (the controller's reselect period)."""
    r = C.c_int32(0)
    _check("hardkv_mti_period", lib().hardkv_mti_period(C.byref(cfg.c), int(n_pool), int(n_survivors), int(kstar),
                                                        int(max_period), C.byref(r)))
    return int(r.value)


def hardkv_shared_pool_blocks(cfg: Config, ctx_len, steps: int = 0) -> int:
    """Physical blocks a SHARED pool needs for a prefill of ctx_len (host lengths) and `steps`
    appends without a condensation."""
    lens = [int(x) for x in (ctx_len.tolist() if hasattr(ctx_len, "tolist") else ctx_len)]
    arr = (C.c_int64 * max(1, len(lens)))(*lens)
    n = C.c_int64(0)
    _check("hardkv_shared_pool_blocks", lib().hardkv_shared_pool_blocks(C.byref(cfg.c), arr, int(steps), C.byref(n)))
    return int(n.value)


def hardkv_select_fork(cfg: Config, st_next: State, st_cur: State, stream=None) -> None:
    _check("hardkv_select_fork", lib().hardkv_select_fork(C.byref(cfg.c), C.byref(st_next.c), C.byref(st_cur.c),
                                                          _stream(stream)))


def hardkv_select_ahead(cfg: Config, st_next: State, q, stream=None, unit_begin: int = 0,
                        unit_count: Optional[int] = None) -> None:
    n = cfg.c.batch * cfg.c.num_kv_heads if unit_count is None else int(unit_count)
    _check("hardkv_select_ahead", lib().hardkv_select_ahead(C.byref(cfg.c), C.byref(st_next.c), _ptr(q),
                                                            int(unit_begin), n, _stream(stream)))


def hardkv_step_num_stages() -> int:
    return int(lib().hardkv_step_num_stages())


def hardkv_step_stage_name(stage: int) -> str:
    return lib().hardkv_step_stage_name(stage).decode()


def require_gpu() -> None:
    """Raise unless a GPU is visible and the library is built: there is no CPU path."""
    lib()
    if not torch.cuda.is_available():
        raise RuntimeError("libhardkv needs an AMD GPU (gfx950); none is visible")
