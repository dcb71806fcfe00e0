"""Seeded input generator for the HARD-KV decode step.

Recipe (one layer of one workload):

* Small per-sequence metadata comes from numpy ``PCG64(SeedSequence([seed,
  layer, stream]))`` and is therefore the same on every machine: mixed context
  lengths ``L_b ~ U{ctx_min..ctx_len}``, per-(b, KV head) query temperatures
  ``tau_gen = exp(U[ln lo, ln hi])``, and the planted heavy positions (count
  ``~ U{lo..hi}``, positions uniform without replacement in ``[0, L_b - W)``).
* Bulk tensors are float32 N(0, 1) draws from a ``torch.Generator`` on the
  target device, seeded from the same seed sequence: queries for every step,
  the prefilled K/V context, and the K/V of every appended token.  Draws on
  the CPU and on the GPU differ, so a parity test generates once on its device
  and copies what the CPU side needs.
* Queries are divided by their head's ``tau_gen`` (when the workload has one).
* A heavy key is rotated onto the mean query of its GQA group at the first
  step: with ``u = qbar / |qbar|``, ``k <- k - (k.u) u + scale |qbar| u``.
* Everything is finally rounded to the storage type (bf16 round-to-nearest-even
  via torch, or kept as float32).

Nothing here computes any part of the decode step itself.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import COND_EVICT, Workload

_STREAM_LEN, _STREAM_TAU, _STREAM_HEAVY = 1, 2, 3
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_KN, _STREAM_VN = 10, 11, 12, 13, 14


def _np_rng(seed: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, stream])))


def _torch_gen(seed: int, layer: int, stream: int, device) -> torch.Generator:
    st = np.random.SeedSequence([seed, layer, stream]).generate_state(2, np.uint32)
    s = (int(st[0]) << 31) ^ int(st[1])
    g = torch.Generator(device=device)
    g.manual_seed(s & ((1 << 62) - 1))
    return g


def storage_dtype(wl: Workload) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


@dataclass
class Inputs:
    """One layer's inputs, all on ``device``.

    ctx_len : int64 [B]              prefilled length per sequence
    k_ctx   : [B][Hkv][Lmax][D]      prefilled keys (rows >= L_b are zero)
    v_ctx   : [B][Hkv][Lmax][D]      prefilled values
    q       : [steps][B][Hq][D]      decode queries
    k_new   : [steps][B][Hkv][D]     appended keys
    v_new   : [steps][B][Hkv][D]     appended values
    tau     : float32 [Hkv]          calibration temperature per KV head
    heavy   : list of int64 arrays per (b, h) with the planted positions
    tau_gen : float64 [B][Hkv] or None
    """

    wl: Workload
    layer: int
    ctx_len: torch.Tensor
    k_ctx: torch.Tensor
    v_ctx: torch.Tensor
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    tau: torch.Tensor
    heavy: list
    tau_gen: Optional[np.ndarray]

    @property
    def max_len(self) -> int:
        return int(self.k_ctx.shape[2])

    def unit(self, b: int, h: int) -> "Inputs":
        """The inputs of one (sequence, KV head) unit as a batch-1, one-KV-head layer."""
        G = self.wl.group
        return Inputs(
            wl=self.wl.with_(batch=1, num_kv_heads=1, num_q_heads=G),
            layer=self.layer,
            ctx_len=self.ctx_len[b:b + 1].clone(),
            k_ctx=self.k_ctx[b:b + 1, h:h + 1].clone(),
            v_ctx=self.v_ctx[b:b + 1, h:h + 1].clone(),
            q=self.q[:, b:b + 1, h * G:(h + 1) * G].clone(),
            k_new=self.k_new[:, b:b + 1, h:h + 1].clone(),
            v_new=self.v_new[:, b:b + 1, h:h + 1].clone(),
            tau=self.tau[h:h + 1].clone(),
            heavy=[self.heavy[b * self.wl.num_kv_heads + h]],
            tau_gen=None if self.tau_gen is None else self.tau_gen[b:b + 1, h:h + 1].copy(),
        )

    def to(self, device) -> "Inputs":
        return Inputs(self.wl, self.layer, self.ctx_len.to(device), self.k_ctx.to(device),
                      self.v_ctx.to(device), self.q.to(device), self.k_new.to(device),
                      self.v_new.to(device), self.tau.to(device), self.heavy, self.tau_gen)


def make_inputs(wl: Workload, layer: int = 0, device="cpu", steps: Optional[int] = None) -> Inputs:
    """Draw one layer of ``wl`` on ``device`` (see the module docstring for the recipe)."""
    device = torch.device(device)
    B, Hq, Hkv, D, G, W = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group, wl.dense_window
    steps = wl.steps if steps is None else steps
    dt = storage_dtype(wl)

    # ---- small metadata (device independent) ----------------------------------------
    if wl.ctx_min is not None:
        lens = _np_rng(wl.seed, layer, _STREAM_LEN).integers(wl.ctx_min, wl.ctx_len + 1, size=B)
    else:
        lens = np.full(B, wl.ctx_len, dtype=np.int64)
    lens = lens.astype(np.int64)
    Lmax = int(lens.max())

    tau_gen = None
    if wl.tau_gen is not None:
        lo, hi = wl.tau_gen
        u = _np_rng(wl.seed, layer, _STREAM_TAU).uniform(np.log(lo), np.log(hi), size=(B, Hkv))
        tau_gen = np.exp(u)

    heavy = []
    hr = _np_rng(wl.seed, layer, _STREAM_HEAVY)
    for b in range(B):
        pool_len = max(0, int(lens[b]) - W)
        for h in range(Hkv):
            lo, hi = wl.heavy
            cnt = int(hr.integers(lo, hi + 1)) if hi > 0 else 0
            cnt = min(cnt, pool_len)
            pos = np.sort(hr.choice(pool_len, size=cnt, replace=False)) if cnt > 0 else np.zeros(0, np.int64)
            heavy.append(pos.astype(np.int64))

    # ---- bulk draws --------------------------------------------------------------------
    gq = _torch_gen(wl.seed, layer, _STREAM_Q, device)
    q32 = torch.randn((steps, B, Hq, D), generator=gq, device=device, dtype=torch.float32)
    if tau_gen is not None:
        scale = torch.from_numpy(1.0 / tau_gen).to(device=device, dtype=torch.float32)  # [B][Hkv]
        q32 = q32 * scale.repeat_interleave(G, dim=1)[None, :, :, None]
    q = q32.to(dt)

    gk = _torch_gen(wl.seed, layer, _STREAM_K, device)
    gv = _torch_gen(wl.seed, layer, _STREAM_V, device)
    k_ctx = torch.zeros((B, Hkv, Lmax, D), device=device, dtype=dt)
    v_ctx = torch.zeros((B, Hkv, Lmax, D), device=device, dtype=dt)
    qbar_all = q[0].float().view(B, Hkv, G, D).mean(dim=2)  # [B][Hkv][D]
    for b in range(B):
        L = int(lens[b])
        kb = torch.randn((Hkv, L, D), generator=gk, device=device, dtype=torch.float32)
        vb = torch.randn((Hkv, L, D), generator=gv, device=device, dtype=torch.float32)
        for h in range(Hkv):
            pos = heavy[b * Hkv + h]
            if pos.size == 0:
                continue
            qbar = qbar_all[b, h]
            nrm = torch.linalg.vector_norm(qbar)
            u = qbar / nrm
            idx = torch.from_numpy(pos).to(device)
            kk = kb[h, idx]                                   # [n][D]
            proj = (kk @ u)[:, None] * u[None, :]
            kb[h, idx] = kk - proj + (wl.heavy_scale * nrm) * u[None, :]
        k_ctx[b, :, :L] = kb.to(dt)
        v_ctx[b, :, :L] = vb.to(dt)
        del kb, vb

    gkn = _torch_gen(wl.seed, layer, _STREAM_KN, device)
    gvn = _torch_gen(wl.seed, layer, _STREAM_VN, device)
    k_new = torch.randn((steps, B, Hkv, D), generator=gkn, device=device, dtype=torch.float32).to(dt)
    v_new = torch.randn((steps, B, Hkv, D), generator=gvn, device=device, dtype=torch.float32).to(dt)

    tau = torch.full((Hkv,), float(wl.tau), dtype=torch.float32)
    return Inputs(wl, layer, torch.from_numpy(lens).to(device), k_ctx, v_ctx, q, k_new, v_new,
                  tau, heavy, tau_gen)


def tiny_workload(**kw) -> Workload:
    """A small layer that still spans several 64-token blocks and ends on a ragged block.

    Used by the parity tests at sizes the oracle finishes in well under a second.
    """
    base = dict(name="tiny", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                dense_window=32, sparse_cap=256, condensed_slots=4, cond_mode=COND_EVICT,
                top_p=0.9, ctx_len=400, ctx_min=300, heavy=(0, 3), seed=7, steps=1)
    base.update(kw)
    return Workload(**base)
