"""Benchmark of the HARD-KV decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c5] [--extra-configs ...] [--gpus 1]

The headline (value, roofline, cpu_baseline) is the 32-layer workload, the largest that
fits one GPU; the other workloads (the batch-1, batch-16 and mixed-length layers, the
last at each p of its sweep, and the streaming one) are measured the same way in child
processes and reported under "configs".

One step is hardkv_step on one batch: append, score + calibrate + top-p, rewrite
(with the view attention fused), condense, tier attention and combine, for every
(sequence, KV head) of the workload (all layers of it for the 32-layer workload).
Inputs are seeded synthetic caches generated on the GPU and resident in HBM
before the timed region.  Prints one JSON line.

Timing:
  * Single-step workloads (one decode step from the prefilled context): the step is
    captured into a HIP graph and replayed K times between two events, each time from
    the prefilled state restored outside the timed region; every kernel of the step is
    also timed on its own on exactly that state (hardkv_step_stage, same stream): the
    ones that only read what earlier kernels wrote R times back to back in one graph, the append and
    the condensation (which advance the state) as the difference of two graphs, R times
    (put back what the kernel changes, run it) against R times the put-back alone.
  * The streaming workload: W warmup steps run eagerly, then the K steps are captured
    into one HIP graph and replayed once between two events; kernels that only read
    what earlier ones wrote are timed again on the post-step state.
  * The dominant kernel is the longest one that moves algorithmic bytes; those bytes
    per launch over its duration give roofline.achieved.  roofline.copy_reference times
    the rewrite's copy alone in the same run (layer 0's kept rows gathered from the pool
    and written contiguously): one 16-byte piece per thread, wavefronts that loop over 64
    rows with the next batch in flight (the pattern a kernel that also consumes the rows
    must take), and a plain device copy of the same bytes; the rates a kernel that reads
    and writes equally can practically reach on this part, beside the 8 TB/s peak.
  * Algorithmic bytes per step follow the byte model of the design notes and are
    computed from the per-unit pool sizes, budgets and condensed blocks of the
    timed steps, replayed eagerly from a snapshot after the timed region.
  * cpu_baseline: the CPU oracle timed on one step of the same workload (a sample
    of units when the full step would take too long), repeated from the prefilled
    state for about --cpu-seconds of CPU time, on the host's cores.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from decode_kv_cache_02_amd import hardkv as hk  # noqa: E402
from synth import get_workload, make_inputs  # noqa: E402
from synth.configs import COND_MERGE  # noqa: E402

HBM_PEAK_GBPS = 8000.0
D = 128
STAGE_NAMES = ["append", "score", "select", "condense", "rewrite_attend", "combine"]
REPEATABLE = [1, 2, 4, 5]  # stages that only read what earlier stages wrote
# the workloads measured beside the headline: the three target workloads (the mixed-length
# one at each p of its sweep, and at p = 0.9 in the shared block pool) and the streaming one
# (also with destructive selection); a spec is workload[:p[:pool layout[:selection]]]
EXTRA_DEFAULT = "c1,c2,c3:0.8,c3:0.9,c3:0.99,c3:0.9:shared,c4,c4:::destructive"
POLICY_DEFAULT = "c2,c4,c5"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c5",
                    help="the headline workload (default: the 32-layer step, the largest that fits one GPU)")
    ap.add_argument("--extra-configs", default=EXTRA_DEFAULT,
                    help="workloads also measured (each in a child process, before the headline) and "
                         "reported under 'configs': comma-separated keys, key:p for a top-p override; "
                         "'none' for none")
    ap.add_argument("--top-p", type=float, default=None, help="override p (the mixed-length workload sweeps it)")
    ap.add_argument("--eager", action="store_true", help="no graph (for counter runs)")
    ap.add_argument("--regularize", choices=["rewrite", "sparse", "mti", "mti-auto"], default="rewrite",
                    help="Rewrite Cache for every head (default), Sparse Loading for every head, the "
                         "budget-threshold rule (rewrite iff --mti-lower <= k* <= --mti-upper), or the "
                         "memory-time controller (default costs, horizon --mti-horizon)")
    ap.add_argument("--mti-horizon", type=int, default=-1,
                    help="reused steps the controller plans for (default: --select-every minus one)")
    ap.add_argument("--pipeline", type=int, default=0,
                    help="with --select-every R: also time the asynchronous pipeline, each selection made "
                         "ahead on a second stream and switched in this many steps later (0: off)")
    ap.add_argument("--pipeline-mode", choices=["side", "spread"], default="side",
                    help="the selection made ahead: all of it on a second stream (side), or in --pipeline "
                         "parts of the units, one after each step before the switch, on the main stream (spread)")
    ap.add_argument("--quick", action="store_true",
                    help="step time only (and --select-every): no per-kernel timing, bytes or roofline")
    ap.add_argument("--policy-configs", default=POLICY_DEFAULT,
                    help="workloads on which the headline run also compares Rewrite Cache, Sparse "
                         "Loading and the memory-time controller at one selection every 1 and 8 steps "
                         "(child processes, reported under 'policies'); 'none' for none")
    ap.add_argument("--mti-lower", type=int, default=0)
    ap.add_argument("--mti-upper", type=int, default=1 << 30)
    ap.add_argument("--calibration", choices=["fixed", "entropy"], default="fixed",
                    help="calibration temperature: the workload's tau (default) or fitted per head by entropy")
    ap.add_argument("--view-layout", choices=["maxlen", "sum"], default="maxlen",
                    help="Flatten Index: view_cap rows per head (default) or packed in unit order")
    ap.add_argument("--view-total", type=int, default=0,
                    help="packed view rows for --view-layout sum (0: batch * kv_heads * view_cap)")
    ap.add_argument("--sink", type=int, default=None,
                    help="sink prefix tokens S (a multiple of 64; default: the workload's, 0)")
    ap.add_argument("--pool-layout", choices=["ring", "shared"], default="ring",
                    help="the pool: a ring per (sequence, KV head), or the shared block pool sized for the "
                         "prefilled lengths")
    ap.add_argument("--selection", choices=["view", "destructive"], default="view",
                    help="what a selection does to the survivors it does not keep: nothing, or drop them for good")
    ap.add_argument("--select-every", type=int, default=1,
                    help="also time steps that select once every R steps and reuse the selection in "
                         "between (hardkv_step_reuse), reported under select_every; the pool ring gets "
                         "ceil(R / 64) + 1 more blocks for the positions that accumulate between selections")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=0, help="oracle sample size in units (0: automatic)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time over which the oracle step is timed")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="OUT_TXT COUNTER_CSV",
                    help="summary of rocprofv3 --pmc runs: OUT_TXT then the counter_collection.csv files")
    ap.add_argument("--summarize-kernels", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_TXT"),
                    help="write a text summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV"),
                    help="HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs of "
                         "--config and of --copy-calib MiB; writes profiles/traffic.json and a text "
                         "summary, then exits")
    ap.add_argument("--cmd", action="append", default=[], help="command recorded in a summary")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.selection == "destructive" and (args.calibration == "entropy" or args.pipeline):
        ap.error("--selection destructive needs the fixed temperature and no --pipeline")
    return args


# ---- layers ------------------------------------------------------------------------------
# the shared pool's allocation state, changed by appends (a block taken) and condensations
# (blocks returned)
POOL_STATE = ("block_table", "free_list", "free_top")
POLICY = {"rewrite": hk.HARDKV_REG_REWRITE, "sparse": hk.HARDKV_REG_SPARSE, "mti": hk.HARDKV_REG_MTI,
          "mti-auto": hk.HARDKV_REG_MTI_AUTO}


class Layer:
    def __init__(self, wl, layer, steps, top_p=None, policy=("rewrite", 0, 0, 0), view=("maxlen", 0),
                 calibration="fixed", pool_layout="ring", selection="view"):
        self.wl = wl
        self.inp = make_inputs(wl, layer=layer, device="cuda", steps=steps)
        total = view[1] or wl.batch * wl.num_kv_heads * wl.V_cap
        kw = dict(top_p=top_p, regularize=POLICY[policy[0]], mti_lower=policy[1], mti_upper=policy[2],
                  mti=dict(mti_horizon=policy[3]),
                  view_layout=hk.HARDKV_VIEW_SUM if view[0] == "sum" else hk.HARDKV_VIEW_MAXLEN, view_total=total,
                  calibration=hk.HARDKV_CAL_ENTROPY if calibration == "entropy" else hk.HARDKV_CAL_FIXED,
                  selection=hk.HARDKV_SEL_DESTRUCTIVE if selection == "destructive" else hk.HARDKV_SEL_VIEW)
        self.cfg = hk.Config.from_workload(wl, **kw)
        self.shared = pool_layout == "shared"
        if self.shared:
            # the shared block pool, sized for the prefilled lengths and the steps taken
            nb = max(1, hk.hardkv_shared_pool_blocks(self.cfg, self.inp.ctx_len.cpu(), steps))
            self.cfg = hk.Config.from_workload(wl, pool_layout=hk.HARDKV_POOL_SHARED, pool_total_blocks=nb, **kw)
            self.MUTABLE = Layer.MUTABLE + POOL_STATE
            self.MUTATES = {0: Layer.MUTATES[0] + POOL_STATE, 3: Layer.MUTATES[3] + POOL_STATE}
        self.st = hk.State(self.cfg)
        self.pool_bytes = 2 * self.st.pool_k.numel() * self.st.pool_k.element_size()
        hk.hardkv_prefill(self.cfg, self.st, self.inp.k_ctx, self.inp.v_ctx, self.inp.ctx_len)
        self.out = torch.zeros((wl.batch, wl.num_q_heads, D), dtype=torch.float32, device="cuda")

    def drop_context(self):
        self.inp.k_ctx = self.inp.v_ctx = None

    def step(self, s):
        hk.hardkv_step(self.cfg, self.st, self.inp.q[s], self.inp.k_new[s], self.inp.v_new[s], self.out)

    def reuse(self, s):
        hk.hardkv_step_reuse(self.cfg, self.st, self.inp.q[s], self.inp.k_new[s], self.inp.v_new[s], self.out)

    def stage(self, s, k):
        hk.hardkv_step_stage(self.cfg, self.st, self.inp.q[s], self.inp.k_new[s], self.inp.v_new[s],
                             self.out, k)

    # What a step changes beyond what it rewrites from scratch: counters, the dense ring
    # (whose slots the append overwrites) and the condensed tier (merged into).  Pool rows
    # written by the append are rewritten with the same values on a replay.
    MUTABLE = ("seq_len", "pool_head", "dense_k", "dense_v", "cond_kn", "cond_vn", "cond_omega",
               "cond_n", "cond_cursor", "error_word")

    # what each state-advancing kernel changes
    MUTATES = {0: ("seq_len", "dense_k", "dense_v", "error_word"),
               3: ("pool_head", "cond_kn", "cond_vn", "cond_omega", "cond_n", "cond_cursor")}

    def snapshot(self):
        return {n: getattr(self.st, n).clone() for n in self.MUTABLE}

    def time_mutating_stage(self, s, k, reps, trials=5):
        """Duration of kernel k (append or condense) on the current state: a graph of
        `reps` times (put back the state it changes, run it) against a graph of the
        put-backs alone, both replayed between events; the median difference per
        launch, in us."""
        names = self.MUTATES[k]
        snap = {n: getattr(self.st, n).clone() for n in names}

        def put():
            for n in names:
                getattr(self.st, n).copy_(snap[n])

        ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(ga):
            for _ in range(reps):
                put()
                self.stage(s, k)
        with torch.cuda.graph(gb):
            for _ in range(reps):
                put()
        torch.cuda.synchronize()
        diffs = []
        for _ in range(trials):
            ta, tb = [], []
            for g, acc in ((ga, ta), (gb, tb)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                acc.append(e0.elapsed_time(e1))
            diffs.append((ta[0] - tb[0]) * 1e3 / reps)
        put()
        torch.cuda.synchronize()
        return float(np.median(diffs))

    def restore(self, snap):
        for n in self.MUTABLE:
            getattr(self.st, n).copy_(snap[n])


def in_step_stage_times(layers, restore, timed, reps):
    """Each kernel's cost inside the step, in us per layer: the step as its six kernels
    (hardkv_step_stage 0..5 for every layer, one graph) against the same graph without
    kernel k, both replayed from the restored state, interleaved, `reps` times; the
    difference of the medians.  Beside the back-to-back durations of stage_us, this keeps
    each kernel between the kernels it really follows and precedes (a kernel that keeps
    the vector ALUs busy runs at a lower clock when repeated back to back)."""
    graphs = {}
    for skip in [None] + list(range(len(STAGE_NAMES))):
        restore()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for L in layers:
                for j in range(len(STAGE_NAMES)):
                    if j != skip:
                        L.stage(0, j)
        graphs[skip] = g
    times = {k: [] for k in graphs}
    for _ in range(max(5, reps)):
        for k, g in graphs.items():
            restore()
            torch.cuda.synchronize()
            times[k].append(timed(g.replay))
    full = float(np.median(times[None]))
    return {STAGE_NAMES[k]: round((full - float(np.median(times[k]))) * 1e3 / len(layers), 2)
            for k in range(len(STAGE_NAMES))}


def time_repeatable_stage(layers, s, k, reps, eager):
    """Duration per launch of a kernel that only reads what earlier kernels wrote: `reps`
    launches per layer back to back, captured into one graph (eagerly with --eager) and
    replayed between events; the median of three replays, in us."""
    run = lambda: [L.stage(s, k) for _ in range(reps) for L in layers]  # noqa: E731
    run()
    torch.cuda.synchronize()
    g = None
    if not eager:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay() if g is not None else run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)) * 1e3 / (reps * len(layers))


def select_every(layers, R, restore_mode, snaps, Wm, K, timed, eager):
    """Steps that select once every R steps and keep that selection in between
    (hardkv_step_reuse): single-step workloads replay [a step with selection, R - 1 steps
    without] from the prefilled state; the streaming one runs its K timed steps with a
    selection at every R-th.  Returns the mean time per step and what the R - 1 steps
    without selection cost each."""
    def restore():
        for L, sn in zip(layers, snaps):
            L.restore(sn)

    steps = list(range(R)) if restore_mode else list(range(Wm, Wm + K))
    first = steps[0]

    def run(mark=lambda: None):
        for s in steps:
            for L in layers:
                L.step(s) if (s - first) % R == 0 else L.reuse(s)
            mark()

    restore()
    run()
    restore()
    torch.cuda.synchronize()
    g = None
    if not eager:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
    times = []
    for _ in range(3 if not restore_mode else max(3, K // R)):
        restore()
        torch.cuda.synchronize()
        times.append(timed(g.replay if g is not None else run))
    err = int(max(int(L.st.error_word[0].item()) for L in layers))
    restore()
    lat = step_latencies(run, len(steps))
    restore()
    torch.cuda.synchronize()
    ms_step = float(np.mean(times)) / len(steps)
    return {"R": R, "ms_per_step": ms_step, "steps_per_s": 1e3 / ms_step, "error_word": err,
            "eager_step_latency": lat,
            "timing": ("graph of one step with selection and R - 1 without, from the prefilled state"
                       if restore_mode else "graph of the K streaming steps, a selection at every R-th")}


def step_latencies(run_steps, nsteps):
    """Per-step latency of a schedule run eagerly: an event on the main stream after each step
    (run_steps(mark) calls mark() after each); the time between consecutive marks, in ms (the
    host stays ahead of the device, so the gaps are the device's time per step)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    i = [0]

    def mark():
        evs[i[0]].record()
        i[0] += 1
    mark()
    run_steps(mark)
    torch.cuda.synchronize()
    lat = [evs[k].elapsed_time(evs[k + 1]) for k in range(i[0] - 1)]
    return {"p50_ms": float(np.median(lat)), "max_ms": float(np.max(lat)), "min_ms": float(np.min(lat))}


def pipeline_every(layers, R, lag, restore_mode, snaps, Wm, timed, eager, mode="side"):
    """Steps with one selection every R steps made ahead: at the first step of each period the
    main stream takes a step on the current selection and forks; a second stream makes the
    selection for that step (hardkv_select_ahead); `lag` steps later the main stream waits for
    it, condenses by its plan and goes on with it.  Two periods (the two states swap roles)
    are captured in one graph with the cross-stream waits; each replay starts from a step
    with selection made the usual way (outside the timing).  Returns the mean time per step."""
    assert 1 <= lag < R
    side = torch.cuda.Stream()
    twins = [L.st.twin() for L in layers]
    first = 0 if restore_mode else Wm
    steps = list(range(first + 1, first + 1 + 2 * R))

    def restore():
        for L, sn in zip(layers, snaps):
            L.restore(sn)

    def setup():
        restore()
        for L in layers:
            L.step(first)  # the selection the first period starts from

    def run(mark=lambda: None):
        main = torch.cuda.current_stream()  # (the capture stream while a graph is captured)
        cur = [L.st for L in layers]
        nxt = list(twins)
        done = None
        for i, s in enumerate(steps):
            k = i % R
            if k == lag and done is not None:  # the switch
                if done != "spread":
                    main.wait_event(done)
                for j, L in enumerate(layers):
                    hk.hardkv_condense(L.cfg, nxt[j], main)
                cur, nxt = nxt, cur
                done = None
            for j, L in enumerate(layers):
                hk.hardkv_step_reuse(L.cfg, cur[j], L.inp.q[s], L.inp.k_new[s], L.inp.v_new[s], L.out, main)
            if k == 0:  # the fork and the selection made ahead
                for j, L in enumerate(layers):
                    hk.hardkv_select_fork(L.cfg, nxt[j], cur[j], main)
                q_fork = s
                if mode == "side":
                    ev = torch.cuda.Event()
                    ev.record(main)
                    side.wait_event(ev)
                    for j, L in enumerate(layers):
                        hk.hardkv_select_ahead(L.cfg, nxt[j], L.inp.q[s], side)
                    done = torch.cuda.Event()
                    done.record(side)
            if mode == "spread" and k < lag:  # part k of the selection, behind this step
                nl = len(layers)
                if nl >= lag:  # whole layers per part (every launch as wide as the step's)
                    for j in range(k * nl // lag, (k + 1) * nl // lag):
                        L = layers[j]
                        hk.hardkv_select_ahead(L.cfg, nxt[j], L.inp.q[q_fork], main)
                else:  # a range of every layer's units per part
                    for j, L in enumerate(layers):
                        n = L.cfg.c.batch * L.cfg.c.num_kv_heads
                        u0, u1 = k * n // lag, (k + 1) * n // lag
                        hk.hardkv_select_ahead(L.cfg, nxt[j], L.inp.q[q_fork], main, u0, u1 - u0)
                done = "spread"
            mark()
        if done is not None and done != "spread":
            main.wait_event(done)

    setup()
    run()
    torch.cuda.synchronize()
    g = None
    if not eager:
        setup()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
    times = []
    for _ in range(3):
        setup()
        torch.cuda.synchronize()
        times.append(timed(g.replay if g is not None else run))
    err = int(max(int(L.st.error_word[0].item()) for L in layers))
    setup()
    lat = step_latencies(run, len(steps))
    restore()
    torch.cuda.synchronize()
    ms_step = float(np.mean(times)) / len(steps)
    return {"R": R, "lag": lag, "mode": mode, "ms_per_step": ms_step, "steps_per_s": 1e3 / ms_step,
            "error_word": err, "eager_step_latency": lat,
            "timing": "graph of two periods of R steps, each selection made ahead " +
                      ("on a second stream" if mode == "side" else
                       f"in {lag} parts behind the steps before the switch") + ", switched in lag steps later"}


def device_copy_reference(nbytes, reps=10):
    """What a plain device copy moving the same bytes (half read, half written) achieves in
    this run, in GB/s: the practical ceiling of a kernel that reads and writes equally,
    beside the data-sheet peak."""
    half = int(nbytes) // 2 // 16 * 16
    if half <= 0:
        return None
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * half * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GBps": gbps, "frac": gbps / HBM_PEAK_GBPS, "what": "torch device copy of the same bytes, this run"}


def gather_copy_reference(L, reps=10):
    """The rewrite's copy alone, in the two access patterns of the copy probes (one 16-byte
    piece per thread, or wavefronts looping over 64 rows with the next batch in flight), and
    torch's device copy of the same bytes: the kept rows of layer 0's last selection (K and
    V) gathered from the pool and written contiguously, timed in this run, in GB/s of bytes
    read plus written."""
    import ctypes as C
    wl, st = L.wl, L.st
    if wl.dtype != "bf16":
        return None
    lib = C.CDLL(os.path.join(ROOT, "decode_kv_cache_02_amd", "libhardkv_probe.so"))
    lib.hardkv_probe_gather_copy.argtypes = [C.c_void_p] * 5 + [C.c_int64, C.c_int32, C.c_void_p]
    lib.hardkv_probe_gather_copy.restype = C.c_int32
    BH, P = wl.batch * wl.num_kv_heads, wl.P_blk
    bits = (st.mask.reshape(BH, P, 1) >> torch.arange(64, device="cuda")) & 1
    u, ring_row = bits.reshape(BH, P * 64).nonzero(as_tuple=True)
    if L.shared:
        rows = st.block_table.reshape(BH, P)[u, ring_row // 64].long() * 64 + ring_row % 64
    else:
        rows = u * (P * 64) + ring_row
    n = int(rows.numel())
    pool_rows = st.pool_k.numel() // D
    if n == 0 or int(rows.min()) < 0 or int(rows.max()) >= pool_rows:
        return None
    rows = rows.to(torch.int32).contiguous()
    dk = torch.empty((n, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    stream = torch.cuda.current_stream()
    nbytes = 2 * 2 * n * D * 2  # K and V, read and written

    def launch(mode):
        rc = lib.hardkv_probe_gather_copy(st.pool_k.data_ptr(), st.pool_v.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                          rows.data_ptr(), n, mode, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"copy probe failed: {rc}")

    res = {"rows": n, "bytes": nbytes}
    for name, mode in (("one_shot_GBps", 0), ("looping_GBps", 1)):
        launch(mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch(mode)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    ok = torch.equal(dk[:: max(1, n // 1000)], st.pool_k.reshape(-1, D)[rows[:: max(1, n // 1000)].long()])
    del dk, dv, rows
    torch.cuda.empty_cache()
    plain = device_copy_reference(nbytes)
    res["torch_copy_GBps"] = plain["GBps"] if plain else None
    res["copy_checked"] = bool(ok)
    res["what"] = ("the kept rows of layer 0 (K and V) gathered from the pool into contiguous rows: one piece "
                   "per thread, wavefronts looping over 64 rows, and a plain device copy of the same bytes")
    return res


def unit_bytes(wl, N, kstar, E, t, c_occ, rw):
    """Algorithmic bytes per stage for arrays of per-unit values (one step).

    score: the pool keys; rewrite_attend: the kept rows read once, and written once for the
    heads that are rewritten (rw), the dense
    window, the sink rows and the occupied condensed slots read, q in; condense (merge): the keys and
    values of the condensing blocks read and the slot read-modify-write (eviction moves
    nothing); append: the leaving dense row read and written to the pool, the new token
    read and written to the dense window, keys and values; combine: the output.  The
    select stage only moves scores and weights (scratch), which the byte model does not
    count."""
    e, G, S = wl.elem_bytes, wl.group, wl.sink
    dense_rows = np.clip(t - S, 0, wl.dense_window)
    sink_rows = np.minimum(t, S)
    merge = wl.cond_mode == COND_MERGE
    cond = (2 * e * D * 64 * E + 2 * (8 * D + 8) * np.minimum(E, wl.condensed_slots)) if merge else 0 * E
    return {
        "append": 8 * e * D * np.ones_like(N),
        "score": e * D * N,
        "select": 0 * N,
        "condense": cond,
        "rewrite_attend": (2 + 2 * rw) * e * D * kstar + 2 * e * D * (dense_rows + sink_rows) + (8 * D + 8) * c_occ + G * D * e,
        "combine": G * D * 4 * np.ones_like(N),
    }


def rows_in_play(L, c, pend):
    """Per unit, the pool rows [c, pend) that the last selection weighed: every survivor, or
    under destructive selection the rows in play (they all weigh at least 1)."""
    wl = L.wl
    P, BH = wl.P_blk, wl.batch * wl.num_kv_heads
    dev = L.st.weights.device
    c = torch.as_tensor(c.reshape(BH), device=dev)
    pend = torch.as_tensor(np.broadcast_to(pend, (wl.batch, wl.num_kv_heads)).reshape(BH), device=dev)
    ring = torch.arange(P * 64, device=dev)
    blk_off = (ring[None, :] // 64 - ((c // 64) % P)[:, None]) % P
    pos = c[:, None] + blk_off * 64 + ring[None, :] % 64
    w = L.st.weights.reshape(BH, P * 64)
    n = ((w != 0) & (pos < pend[:, None])).sum(1)
    return n.cpu().numpy().astype(np.int64).reshape(wl.batch, wl.num_kv_heads)


def step_accounting(layers, s):
    """Runs step s of every layer eagerly and returns (bytes per stage, pool tokens scanned).
    Under destructive selection the score pass reads only the rows in play."""
    tot = {k: 0.0 for k in STAGE_NAMES}
    scanned = 0
    for L in layers:
        wl = L.wl
        t = L.st.seq_len.cpu().numpy().astype(np.int64)
        c = L.st.pool_head.cpu().numpy().astype(np.int64)
        t1 = (t + 1)[:, None]
        pend = np.maximum(wl.sink, t1 - wl.dense_window)
        N = pend - c
        L.step(s)
        torch.cuda.synchronize()
        if L.cfg.c.selection == hk.HARDKV_SEL_DESTRUCTIVE:
            N = rows_in_play(L, c, pend)
        kstar = L.st.budget.cpu().numpy().astype(np.int64)
        E = L.st.n_condense.cpu().numpy().astype(np.int64)
        c_occ = (L.st.cond_n.cpu().numpy() > 0).sum(-1)
        rw = L.st.regularized.cpu().numpy().astype(np.int64)
        ub = unit_bytes(wl, N, kstar, E, np.broadcast_to(t1, N.shape), c_occ, rw)
        for k in tot:
            tot[k] += float(ub[k].sum())
        scanned += int(N.sum())
    return tot, scanned


def copy_calibration(mib):
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}))


# ---- profile summaries -------------------------------------------------------------------
KERNEL_STAGE = {"hardkv_rewrite": "rewrite_attend", "hardkv_score": "score", "hardkv_select": "select",
                "hardkv_condense": "condense", "hardkv_append": "append", "hardkv_combine": "combine",
                "hardkv_attend_tiers": "attend_tiers", "hardkv_prefill": "prefill",
                "probe_one_shot": "copy_one_shot", "probe_loop": "copy_loop",
                "hardkv_fit": "select", "hardkv_fit_prep": "select", "hardkv_fit_round": "select",
                "hardkv_fit_final": "select", "hardkv_sel_weigh": "select", "hardkv_sel_cut": "select",
                "hardkv_sel_count": "select", "hardkv_sel_finish": "select", "hardkv_flatten": "select",
                "hardkv_fork": "select", "hardkv_prefill_alloc": "prefill", "hardkv_prefill_clear": "prefill"}
KERNEL_SOURCES = sorted(
    [os.path.join("decode_kv_cache_02_amd", "csrc", f)
     for f in os.listdir(os.path.join(ROOT, "decode_kv_cache_02_amd", "csrc"))
     if f.endswith((".hip", ".h"))] + [os.path.join("include", "hardkv.h")])


def kernel_key(name):
    for k in sorted(KERNEL_STAGE, key=len, reverse=True):
        if k + "<" in name or k + "(" in name or name.endswith(k) or (k + " ") in name:
            return k
    return None


def summarize_kernels(src, dst, cmds, title):
    import csv
    rows = list(csv.DictReader(open(src)))
    with open(dst, "w") as f:
        f.write(f"# {title}\n\nCommands (repository root R, one MI355X):\n\n")
        for c in cmds:
            f.write(f"    {c}\n")
        f.write("\nrocprofv3 kernel statistics (kernel_stats.csv), all dispatches of the run:\n\n")
        f.write(f"{'kernel':<58} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}\n")
        for r in rows:
            name = r["Name"]
            if kernel_key(name) is None and float(r["Percentage"]) < 1.0:
                continue
            name = (name.replace("void hardkv::(anonymous namespace)::", "")
                    .replace("hardkv::(anonymous namespace)::", "").replace("(hardkv::Args)", "")
                    .replace("hardkv::", ""))
            f.write(f"{name[:58]:<58} {r['Calls']:>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                    f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                    f"{float(r['Percentage']):>6.2f}\n")
    print(open(dst).read())


def _short(name):
    return (name.replace("void hardkv::(anonymous namespace)::", "").replace("hardkv::(anonymous namespace)::", "")
            .replace("(hardkv::Args)", "").replace("hardkv::", "").replace("(anonymous namespace)::", ""))


def summarize_counters(dst, srcs, cmds, title):
    """Per kernel instance: dispatches, mean duration and the mean of every counter per
    dispatch over the counter runs (rocprofv3 --pmc CSVs), with derived ratios whose
    formulas are printed beside them."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for src in srcs:
        for r in csv.DictReader(open(src)):
            name = _short(r["Kernel_Name"])
            if kernel_key(r["Kernel_Name"]) is None:
                continue
            key = (src, r["Dispatch_Id"])
            acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[name][key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    xcd, simds = 8, 1024
    with open(dst, "w") as f:
        f.write(f"# {title}\n\nCommands (repository root R, one MI355X; each counter set in its own run):\n\n")
        for c in cmds:
            f.write(f"    {c}\n")
        f.write("\nMeans per dispatch (durations are those of the counter runs, which serialise dispatches).\n"
                "Derived: clock GHz = GRBM_GUI_ACTIVE / 8 XCDs / duration; VALU busy = SQ_ACTIVE_INST_VALU x 4 /\n"
                "(1024 SIMDs x GRBM_GUI_ACTIVE / 8); VALU instr per wave = SQ_INSTS_VALU / SQ_WAVES; TA busy =\n"
                "TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8).  GRBM_GUI_ACTIVE also counts the dispatch around the\n"
                "kernel, so the clock reads high for kernels shorter than a few tens of us.\n\n")
        for name in sorted(acc, key=lambda n: -np.mean(list(dur[n].values()))):
            c = {k: float(np.mean(v)) for k, v in acc[name].items()}
            d = float(np.mean(list(dur[name].values())))
            f.write(f"## {name}\n\ndispatches {len(dur[name])}, mean duration {d:.2f} us\n\n")
            for k in sorted(c):
                f.write(f"    {k:<26} {c[k]:>18.1f}\n")
            gui = c.get("GRBM_GUI_ACTIVE")
            der = []
            if gui:
                der.append(("clock GHz", gui / xcd / (d * 1e3)))
                if "SQ_ACTIVE_INST_VALU" in c:
                    der.append(("VALU busy", c["SQ_ACTIVE_INST_VALU"] * 4 / (simds * gui / xcd)))
                if "TA_BUSY_avr" in c:
                    der.append(("TA busy", c["TA_BUSY_avr"] / (gui / xcd)))
            if c.get("SQ_WAVES") and "SQ_INSTS_VALU" in c:
                der.append(("VALU instr per wave", c["SQ_INSTS_VALU"] / c["SQ_WAVES"]))
            if der:
                f.write("\n")
                for k, v in der:
                    f.write(f"    {k:<26} {v:>18.3f}\n")
            f.write("\n")
    print(open(dst).read())


def run_options(args, wl):
    """The options that change what the kernels of a run do: counter traffic taken under
    one set of them is reported only for runs with the same set."""
    return {"top_p": args.top_p, "regularize": args.regularize,
            "mti": [args.mti_lower, args.mti_upper] if args.regularize == "mti" else None,
            "calibration": args.calibration, "view_layout": args.view_layout,
            "view_total": args.view_total if args.view_layout == "sum" else None, "sink": wl.sink,
            "pool_layout": args.pool_layout, "select_every": max(1, args.select_every),
            "selection": args.selection}


def summarize_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, calib_mib, wl, cmds, options):
    """Per kernel: the counter's KiB per dispatch, averaged over the run's dispatches and
    scaled by what it reads for a plain device copy of calib_mib MiB (read and written
    once).  The counter runs are taken with the options given here (run_options)."""
    import csv
    import collections

    def per_kernel(path):
        out = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return out

    res = {}
    scale = {}
    for ctr, path, cal in (("FETCH_SIZE", fetch_csv, cal_fetch_csv), ("WRITE_SIZE", write_csv, cal_write_csv)):
        calk = per_kernel(cal)
        copy_kib = max(max(v) for n, v in calk.items() if "copyBuffer" in n or "copy" in n.lower())
        scale[ctr] = calib_mib * 1024 / copy_kib
        for n, v in per_kernel(path).items():
            k = kernel_key(n)
            if k is None:
                continue
            ent = res.setdefault(KERNEL_STAGE[k], {"launches": 0})
            ent["launches"] = max(ent["launches"], len(v))
            ent[ctr] = sum(v) / len(v) * scale[ctr] * 1024  # bytes per dispatch
    digest = source_digest(KERNEL_SOURCES)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec[wl.name] = {st: {"fetch_bytes_per_launch": e.get("FETCH_SIZE", 0.0),
                         "write_bytes_per_launch": e.get("WRITE_SIZE", 0.0),
                         "hbm_bytes_per_launch": e.get("FETCH_SIZE", 0.0) + e.get("WRITE_SIZE", 0.0),
                         "launches": e["launches"], "sources": KERNEL_SOURCES, "source_digest": digest,
                         "options": options}
                    for st, e in res.items()}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    dst = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.txt")
    with open(dst, "w") as f:
        f.write(f"# HBM traffic per launch, workload {wl.name} (counter runs)\n\n")
        f.write("Commands (repository root R, one MI355X; each counter in its own run):\n\n")
        for c in cmds:
            f.write(f"    {c}\n")
        f.write(f"\nCalibration: a {calib_mib} MiB device copy reads FETCH_SIZE as "
                f"{calib_mib * 1024 / scale['FETCH_SIZE']:.0f} KiB (scale {scale['FETCH_SIZE']:.3f}) and "
                f"WRITE_SIZE as {calib_mib * 1024 / scale['WRITE_SIZE']:.0f} KiB "
                f"(scale {scale['WRITE_SIZE']:.3f}).\n")
        f.write(f"Kernel sources digest {digest} (bench.py reports this traffic only while it matches).\n\n")
        f.write(f"{'stage kernel':<16} {'launches':>8} {'fetch MB':>10} {'write MB':>10} {'total MB':>10}\n")
        for st, e in sorted(rec[wl.name].items(), key=lambda kv: -kv[1]["hbm_bytes_per_launch"]):
            f.write(f"{st:<16} {e['launches']:>8} {e['fetch_bytes_per_launch'] / 1e6:>10.1f} "
                    f"{e['write_bytes_per_launch'] / 1e6:>10.1f} {e['hbm_bytes_per_launch'] / 1e6:>10.1f}\n")
    print(open(dst).read())


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, options):
    """HBM bytes per launch measured by the counter runs kept under profiles/, if they were
    taken on the current kernel sources with the same run options."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent:
        return None
    if ent.get("source_digest") != source_digest(ent.get("sources", [])):
        return None
    if ent.get("options") != options:
        return None
    return ent.get("hbm_bytes_per_launch")


# ---- CPU baseline -------------------------------------------------------------------------
def cpu_baseline(wl, layers, units_req, seconds):
    from oracle import hardkv_oracle as orc
    L = layers[0]
    inp = L.inp_cpu_source
    B, H = wl.batch, wl.num_kv_heads
    total_units = B * H * len(layers)
    # whole sequences (all KV heads) of the first layer, as many as the sample needs
    per_seq = H
    if units_req > 0:
        nb = max(1, min(B, units_req // per_seq))
    else:
        nb = B if wl.batch * wl.ctx_len <= 16 * 16384 else max(1, B // 8)
    sub = wl.with_(batch=nb)
    k_ctx = inp["k_ctx"][:nb].cpu()
    v_ctx = inp["v_ctx"][:nb].cpu()
    lens = inp["ctx_len"][:nb].cpu()
    o = orc.Oracle(sub, top_p=L.cfg.c.top_p)
    assert o.prefill(k_ctx, v_ctx, lens) == 0
    q = L.inp.q[0][:nb].cpu()
    kn = L.inp.k_new[0][:nb].cpu()
    vn = L.inp.v_new[0][:nb].cpu()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1))
    # the sampled step, repeated from the prefilled state until about `seconds` of CPU
    # time have been measured (the prefill is outside the timed part)
    total, reps = 0.0, 0
    while total < seconds and reps < 20000:
        if reps:
            assert o.prefill(k_ctx, v_ctx, lens) == 0
        t0 = time.perf_counter()
        o.step(q, kn, vn, attend=True, nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    units = nb * H
    step_s = total / reps * total_units / units
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} repetitions of one step of {units} of the {total_units} (sequence, KV "
                      f"head) units ({nb} sequences x {H} KV heads of layer 0, same inputs), "
                      f"{total:.1f} s in all, scaled to the whole step",
            "seconds": total}


# ---- main ---------------------------------------------------------------------------------
def run_extras(args):
    """Each extra workload in a child process of its own (so that its device memory is
    freed before the next one): the same timing, no CPU baseline; a summary per workload."""
    import subprocess
    out = []
    if not args.extra_configs or args.extra_configs == "none":
        return out
    for spec in args.extra_configs.split(","):
        key, _, rest = spec.partition(":")
        p, _, rest = rest.partition(":")
        layout, _, selection = rest.partition(":")
        cmd = [sys.executable, os.path.abspath(__file__), "--child", "--config", key, "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--no-cpu-baseline", "--extra-configs", "none"]
        if p:
            cmd += ["--top-p", p]
        if layout:
            cmd += ["--pool-layout", layout]
        if selection:
            cmd += ["--selection", selection]
        t0 = time.perf_counter()
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        wall = time.perf_counter() - t0
        if r.returncode != 0:
            raise RuntimeError(f"bench child {spec} failed ({r.returncode}):\n{r.stderr[-2000:]}")
        d = json.loads(r.stdout.strip().splitlines()[-1])
        rf = d["roofline"]
        out.append({"workload": d["config"]["workload"], "top_p": d["config"]["top_p"],
                    "pool_layout": d["config"]["pool_layout"], "selection": d["config"]["selection"],
                    "pool_bytes": d["pool_bytes"],
                    "ms_per_step": d["ms_per_step"], "steps_per_s": d["value"],
                    "kv_tokens_scanned_per_s": d["kv_tokens_scanned_per_s"],
                    "algorithmic_bytes_per_step": d["algorithmic_bytes_per_step"],
                    "step_hbm_GBps": d["step_hbm_GBps"], "step_hbm_frac": d["step_hbm_frac"],
                    "dominant_kernel": rf["kernel"], "dominant_GBps": rf["achieved"], "dominant_frac": rf["frac"],
                    "copy_reference": rf.get("copy_reference"),
                    "stage_us": d["stage_us"], "stage_us_in_step": d.get("stage_us_in_step"),
                    "timing": d["config"]["timing"], "wall_s": round(wall, 1)})
        print(f"bench: {spec} {d['ms_per_step']:.4f} ms/step, step {d['step_hbm_frac']:.3f} of HBM peak "
              f"({wall:.0f} s)", file=sys.stderr, flush=True)
    return out


def shared_pool_summary(extras):
    """The shared block pool beside the rings on the same workload and p (the first such pair
    among the extra workloads): pool memory, and the score, rewrite and step times."""
    for sh in extras:
        if sh["pool_layout"] != "shared":
            continue
        for rg in extras:
            if (rg["pool_layout"] == "ring" and rg["workload"] == sh["workload"] and rg["top_p"] == sh["top_p"]
                    and rg.get("selection") == sh.get("selection")):
                def pair(x, y):
                    return {"ring": x, "shared": y, "shared_over_ring": y / x if x else None}
                return {"workload": sh["workload"], "top_p": sh["top_p"],
                        "pool_bytes": pair(rg["pool_bytes"], sh["pool_bytes"]),
                        "score_us": pair(rg["stage_us"]["score"], sh["stage_us"]["score"]),
                        "rewrite_attend_us": pair(rg["stage_us"]["rewrite_attend"], sh["stage_us"]["rewrite_attend"]),
                        "ms_per_step": pair(rg["ms_per_step"], sh["ms_per_step"])}
    return None


def run_policies(args):
    """Rewrite Cache, Sparse Loading and the memory-time controller (default costs, horizon =
    the steps that reuse a selection) on each workload, with a selection every step and every
    8 steps, each in a child process; step times only."""
    import subprocess
    out = []
    if not args.policy_configs or args.policy_configs == "none":
        return out
    for key in args.policy_configs.split(","):
        for R in (1, 8):
            row = {"workload": get_workload(key).name, "select_every": R}
            for pol in ("rewrite", "sparse", "mti-auto"):
                cmd = [sys.executable, os.path.abspath(__file__), "--child", "--quick", "--config", key, "--steps",
                       str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline", "--extra-configs", "none",
                       "--policy-configs", "none", "--regularize", pol, "--select-every", str(R)]
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
                if r.returncode != 0:
                    raise RuntimeError(f"bench policy child {key} {pol} R={R} failed ({r.returncode}):\n{r.stderr[-2000:]}")
                d = json.loads(r.stdout.strip().splitlines()[-1])
                ms = d["select_every"]["ms_per_step"] if R > 1 else d["ms_per_step"]
                row[pol] = {"ms_per_step": ms, "steps_per_s": 1e3 / ms, "rewritten_heads": d["rewritten_heads"]}
            best_fixed = max(row["rewrite"]["steps_per_s"], row["sparse"]["steps_per_s"])
            row["controller_vs_best_fixed"] = row["mti-auto"]["steps_per_s"] / best_fixed
            # Rewrite Cache with each selection made ahead: all of it on a second stream and
            # switched in 2 steps later, or in R - 1 parts behind the steps before the switch
            for mode, lag in (("side", 2), ("spread", R - 1)) if R > 1 else ():
                cmd = [sys.executable, os.path.abspath(__file__), "--child", "--quick", "--config", key, "--steps",
                       str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline", "--extra-configs", "none",
                       "--policy-configs", "none", "--select-every", str(R), "--pipeline", str(lag),
                       "--pipeline-mode", mode]
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
                if r.returncode != 0:
                    raise RuntimeError(f"bench pipeline child {key} R={R} failed ({r.returncode}):\n{r.stderr[-2000:]}")
                d = json.loads(r.stdout.strip().splitlines()[-1])
                pl = d["pipeline"]
                row[f"rewrite_pipelined_{mode}"] = {
                    "ms_per_step": pl["ms_per_step"], "steps_per_s": pl["steps_per_s"], "lag": pl["lag"],
                    "eager_step_latency": pl["eager_step_latency"],
                    "same_run_without": {"ms_per_step": d["select_every"]["ms_per_step"],
                                         "eager_step_latency": d["select_every"]["eager_step_latency"]}}
                print(f"bench: pipeline {key} R={R} {mode} lag {lag}: {pl['ms_per_step']:.4f} ms/step, max step "
                      f"{pl['eager_step_latency']['max_ms']:.3f} ms (without: {d['select_every']['ms_per_step']:.4f}, "
                      f"max {d['select_every']['eager_step_latency']['max_ms']:.3f})", file=sys.stderr, flush=True)
            print(f"bench: policies {key} R={R}: " + ", ".join(f"{p} {row[p]['ms_per_step']:.4f} ms"
                                                              for p in ("rewrite", "sparse", "mti-auto")),
                  file=sys.stderr, flush=True)
            out.append(row)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.cmd,
                           f"Counters, workload {get_workload(args.config).name}")
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels, args.cmd, f"Kernel trace, workload {get_workload(args.config).name}")
        return
    if args.summarize_traffic:
        wl = get_workload(args.config)
        if args.sink is not None:
            wl = dataclasses.replace(wl, sink=args.sink)
        summarize_traffic(*args.summarize_traffic, args.copy_calib or 1024, wl, args.cmd, run_options(args, wl))
        return
    extras = [] if (args.child or args.copy_calib) else run_extras(args)
    policies = [] if (args.child or args.copy_calib) else run_policies(args)
    hk.require_gpu()
    torch.cuda.set_device(0)
    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    wl = get_workload(args.config)
    if args.sink is not None:
        wl = dataclasses.replace(wl, sink=args.sink)
    R = max(1, args.select_every)
    if R > 1:
        wl = dataclasses.replace(wl, pool_blocks=wl.P_blk + (R + 63) // 64 + 1)
    top_p = args.top_p
    # single-step workloads: every timed step is the step from the prefilled context
    restore_mode = wl.steps == 1
    K, Wm = args.steps, args.warmup
    nsteps = R if restore_mode else Wm + K
    if args.pipeline:
        nsteps = max(nsteps, (0 if restore_mode else Wm) + 1 + 2 * R)

    layers = []
    for layer in range(wl.layers):
        horizon = args.mti_horizon if args.mti_horizon >= 0 else R - 1
        L = Layer(wl, layer, nsteps, top_p=top_p,
                  policy=(args.regularize, args.mti_lower, args.mti_upper, horizon),
                  view=(args.view_layout, args.view_total), calibration=args.calibration,
                  pool_layout=args.pool_layout, selection=args.selection)
        if layer == 0 and not args.no_cpu_baseline:
            L.inp_cpu_source = {"k_ctx": L.inp.k_ctx, "v_ctx": L.inp.v_ctx, "ctx_len": L.inp.ctx_len}
        else:
            L.drop_context()
        layers.append(L)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    stage_us = {}
    stage_in_step = None
    if restore_mode:
        # the workload is one decode step from the prefilled context: capture that step,
        # then replay it K times, each from the restored state
        snaps = [L.snapshot() for L in layers]

        def restore():
            for L, sn in zip(layers, snaps):
                L.restore(sn)

        for _ in range(max(1, Wm)):
            for L in layers:
                L.step(0)
            restore()
        torch.cuda.synchronize()
        g = None
        if not args.eager:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for L in layers:
                    L.step(0)
            torch.cuda.synchronize()
        times = []
        for _ in range(K):
            restore()
            torch.cuda.synchronize()
            times.append(timed(g.replay if g is not None else (lambda: [L.step(0) for L in layers])))
        ms_per_step = float(np.mean(times))
        graph_out = layers[-1].out.clone()
        # every kernel of the step timed on the state it really sees: kernels that only
        # read what earlier ones wrote run R times back to back; the append and the
        # condensation (which advance the state) run once per restore
        for k in range(0 if args.quick else len(STAGE_NAMES)):
            restore()
            for j in range(k):
                for L in layers:
                    L.stage(0, j)
            torch.cuda.synchronize()
            if k in REPEATABLE:
                stage_us[STAGE_NAMES[k]] = time_repeatable_stage(layers, 0, k, args.stage_reps, args.eager)
            else:
                stage_us[STAGE_NAMES[k]] = layers[0].time_mutating_stage(0, k, args.stage_reps)
        if not args.quick and not args.eager:
            stage_in_step = in_step_stage_times(layers, restore, timed, K)
        restore()
        torch.cuda.synchronize()
        snap_after = snaps
        acc_steps = [0]
    else:
        for s in range(Wm):
            for L in layers:
                L.step(s)
        torch.cuda.synchronize()
        snap_after = [L.snapshot() for L in layers]
        if args.eager:
            ms = timed(lambda: [L.step(s) for s in range(Wm, Wm + K) for L in layers])
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(Wm, Wm + K):
                    for L in layers:
                        L.step(s)
            # capture does not run the kernels; the state is still the post-warmup one
            torch.cuda.synchronize()
            ms = timed(g.replay)
        ms_per_step = ms / K
        graph_out = layers[-1].out.clone()
        acc_steps = list(range(Wm, Wm + K))
        # per-kernel durations of the stages that only read what earlier stages wrote,
        # repeated on the post-step state
        # (the append and the condensation are not re-run here: an append on the post-step
        # state would write the next pool row, which may hold a live row of the ring)
        s_last = acc_steps[-1]
        for k in ([] if args.quick else REPEATABLE):
            stage_us[STAGE_NAMES[k]] = time_repeatable_stage(layers, s_last, k, args.stage_reps, args.eager)

    if args.quick:
        res = {"workload": wl.name, "regularize": args.regularize, "ms_per_step": ms_per_step,
               "steps_per_s": 1e3 / ms_per_step,
               "rewritten_heads": float(np.mean([L.st.regularized.float().mean().item() for L in layers]))}
        if R > 1:
            res["select_every"] = select_every(layers, R, restore_mode, snaps if restore_mode else snap_after, Wm, K,
                                               timed, args.eager)
            res["select_every"]["mti_horizon"] = horizon
            if args.pipeline:
                res["pipeline"] = pipeline_every(layers, R, args.pipeline, restore_mode,
                                                 snaps if restore_mode else snap_after, Wm, timed, args.eager,
                                                 args.pipeline_mode)
        print(json.dumps(res))
        return

    # exact algorithmic bytes of the timed steps, replayed eagerly from the snapshot
    for L, sn in zip(layers, snap_after):
        L.restore(sn)
    torch.cuda.synchronize()
    bytes_tot = {k: 0.0 for k in STAGE_NAMES}
    scanned_tot = 0
    for s in acc_steps:
        b, n = step_accounting(layers, s)
        for k in b:
            bytes_tot[k] += b[k]
        scanned_tot += n
    nacc = len(acc_steps)
    replay_matches = bool(torch.equal(graph_out, layers[-1].out))
    bytes_step = {k: v / nacc for k, v in bytes_tot.items()}
    algo_step = sum(bytes_step.values())
    scanned_step = scanned_tot / nacc

    # the dominant kernel: the longest of the repeatable stages that move algorithmic bytes
    dom = max((k for k in stage_us if bytes_step[k] > 0), key=stage_us.get)
    dom_bytes_launch = bytes_step[dom] / len(layers)
    achieved = dom_bytes_launch / (stage_us[dom] * 1e-6) / 1e9
    traffic = load_traffic(dom, wl.name, run_options(args, wl))

    steps_per_s = 1e3 / ms_per_step
    res = {
        "metric": "hardkv_step decode steps/s + KV tokens scanned/s; % of HBM peak GB/s",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "batch": wl.batch,
                   "ctx_len": wl.ctx_len, "ctx_min": wl.ctx_min, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "dense_window": wl.dense_window,
                   "sink": wl.sink, "sparse_cap": wl.sparse_cap, "condensed_slots": wl.condensed_slots,
                   "top_p": float(layers[0].cfg.c.top_p), "cond_mode": "merge",
                   "regularize": args.regularize if args.regularize != "mti" else
                   f"mti [{args.mti_lower}, {args.mti_upper}]",
                   "mti_horizon": horizon if args.regularize == "mti-auto" else None,
                   "view_layout": args.view_layout, "calibration": args.calibration,
                   "pool_layout": args.pool_layout, "selection": args.selection,
                   "timing": ("one-step graph replay from the prefilled state" if restore_mode else
                              "graph of the K streaming steps") + (" (eager)" if args.eager else "")},
        "kv_tokens_scanned_per_s": scanned_step * steps_per_s,
        "algorithmic_bytes_per_step": algo_step,
        "step_hbm_GBps": algo_step / (ms_per_step * 1e-3) / 1e9,
        "step_hbm_frac": algo_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stage_us_in_step": stage_in_step,
        "stage_algorithmic_bytes": {k: round(v) for k, v in bytes_step.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": dom_bytes_launch, "us_per_launch": stage_us[dom],
                     "copy_reference": gather_copy_reference(layers[0])},
        "graph_replay_matches_eager": replay_matches,
        # device bytes of the pools' K and V (all layers): the rings' worst case, or the
        # shared pool sized for the prefilled lengths
        "pool_bytes": sum(L.pool_bytes for L in layers),
    }
    if R > 1:
        res["select_every"] = select_every(layers, R, restore_mode, snaps if restore_mode else snap_after, Wm, K,
                                           timed, args.eager)
        res["config"]["pool_blocks"] = wl.P_blk
        if args.pipeline:
            res["pipeline"] = pipeline_every(layers, R, args.pipeline, restore_mode,
                                             snaps if restore_mode else snap_after, Wm, timed, args.eager,
                                             args.pipeline_mode)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, layers, args.cpu_units, args.cpu_seconds)
    if extras:
        res["configs"] = extras
        res["shared_pool"] = shared_pool_summary(extras)
    if policies:
        res["policies"] = policies
    print(json.dumps(res))


if __name__ == "__main__":
    main()
