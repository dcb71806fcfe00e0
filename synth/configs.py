"""Workload definitions for the HARD-KV decode step.

Each workload fixes the shapes of one decode layer (batch, query/KV heads,
head_dim), the tier capacities (dense window W, pool ring blocks, sparse cap,
view cap, condensed slots C), the top-p threshold, the condensation mode, the
prefilled context lengths, the number of decode steps and the seed.  The
values that the pages leave open (block size 64, tau = 1, sparse caps, the
condensed tier of the streaming case) are readings; they are listed with the
input recipe in the design notes.

Block size is 64 tokens everywhere: one wavefront, one 64-bit mask word.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

BLOCK = 64

COND_OFF, COND_EVICT, COND_MERGE = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    dtype: str = "bf16"              # storage/compute type of q, K, V: "bf16" or "f32"
    dense_window: int = 512          # W
    sparse_cap: int = 15872          # S_cap (multiple of 64)
    condensed_slots: int = 256       # C
    cond_mode: int = COND_MERGE
    top_p: float = 0.9
    tau: float = 1.0                 # calibration temperature, same for every KV head
    layers: int = 1
    steps: int = 1                   # decode steps taken from the prefilled state
    ctx_len: int = 16384             # prefilled length (or the maximum of a mixed draw)
    ctx_min: Optional[int] = None    # mixed lengths: L_b ~ U{ctx_min .. ctx_len}
    heavy: Tuple[int, int] = (0, 0)  # planted heavy keys per (b, h): U{lo .. hi}
    heavy_scale: float = 4.0
    tau_gen: Optional[Tuple[float, float]] = None  # per-(b,h) query temperature, log-uniform
    seed: int = 0
    sink: int = 0                      # S: sink prefix tokens (a multiple of 64, or 0)
    pool_blocks: Optional[int] = None  # P_blk; derived when None
    view_cap: Optional[int] = None     # V_cap; derived when None
    top_p_sweep: Tuple[float, ...] = field(default_factory=tuple)

    # ---- derived sizes -------------------------------------------------------------
    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def P_blk(self) -> int:
        """Pool ring blocks per (b, h).

        The ring must hold the prefilled pool [0, L - W + 1) before the first
        condensation and, in steady state, at most S_cap + 1 live tokens.
        """
        if self.pool_blocks is not None:
            return self.pool_blocks
        first = -(-(self.ctx_len - self.dense_window + 1 - self.sink) // BLOCK)
        steady = self.sparse_cap // BLOCK + 1
        if self.cond_mode == COND_OFF:
            steady = -(-(self.ctx_len - self.dense_window + self.steps - self.sink) // BLOCK) + 1
        return max(first, steady, 1)

    @property
    def V_cap(self) -> int:
        if self.view_cap is not None:
            return self.view_cap
        if self.cond_mode == COND_OFF:
            return self.P_blk * BLOCK
        return self.sparse_cap

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# ---- the five benchmark workloads --------------------------------------------------
WORKLOADS: Dict[str, Workload] = {
    # batch 1, fp32, 4096-token context, 16 heavy keys per head, one step
    "c1": Workload(
        name="c1_b1_ctx4k_f32_p0.9", batch=1, dtype="f32", dense_window=256,
        sparse_cap=3840, condensed_slots=64, top_p=0.9, ctx_len=4096,
        heavy=(16, 16), seed=1001),
    # Llama-3-8B-shaped layer, batch 16, 16k context, per-head query temperature
    "c2": Workload(
        name="c2_b16_ctx16k_bf16_p0.95", batch=16, dense_window=512, sparse_cap=15872,
        condensed_slots=256, top_p=0.95, ctx_len=16384, tau_gen=(0.3, 3.0), seed=1002),
    # batch 64, mixed lengths 8k..32k, 0..64 heavy keys per head, p swept
    "c3": Workload(
        name="c3_b64_ctx8k-32k_bf16", batch=64, dense_window=512, sparse_cap=8192,
        condensed_slots=256, top_p=0.9, ctx_len=32768, ctx_min=8192, heavy=(0, 64),
        seed=1003, top_p_sweep=(0.8, 0.9, 0.99)),
    # streaming: batch 4, 128k context, 256 decode steps, 512 condensed slots
    "c4": Workload(
        name="c4_b4_ctx128k_bf16_256steps", batch=4, dense_window=512, sparse_cap=130560,
        condensed_slots=512, top_p=0.9, ctx_len=131072, steps=256, seed=1004),
    # full 32-layer step, batch 32, 16k context
    "c5": Workload(
        name="c5_32layers_b32_ctx16k_bf16", batch=32, dense_window=512, sparse_cap=15872,
        condensed_slots=256, top_p=0.9, ctx_len=16384, layers=32, seed=1005),
}


def get_workload(key: str) -> Workload:
    if key in WORKLOADS:
        return WORKLOADS[key]
    for w in WORKLOADS.values():
        if w.name == key:
            return w
    raise KeyError(f"unknown workload {key!r}; known: {sorted(WORKLOADS)}")


def workload_keys() -> List[str]:
    return list(WORKLOADS)
