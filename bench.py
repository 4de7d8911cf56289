"""Benchmark: MoE dispatch + combine, forward + backward, per layer, on one GPU.

One step is one pass of the whole hot path over one layer's synthetic input.
The expert in between is the identity, so there is no GEMM: the path is
HBM-bound and is measured against the HBM roofline.

* Standard layers (the default Qwen3-30B-A3B-shaped one, the skewed and the
  DeepSeek-V3-shaped ones): layout (counts, offsets, stable positions) ->
  dispatch (with per-row scores) -> combine (top-k weighted) -> combine
  backward (rows + router-weight gradient) -> dispatch backward.
* The DiffusionGemma-shaped layer (router scores absorbed before W2): three
  forward passes with independent routings (layout, scaled dispatch, plain
  combine); passes 1 and 3 then replay layout + dispatch (activation
  checkpointing; the combine is never replayed) and run the combine backward
  (a copy) and the scaled dispatch backward (rows + score gradient).

Cold HBM: the step rotates over buffer sets that together span at least
12 GiB (``--sets`` overrides the count), and the combine backward reads its
own copy of the expert output, so the 256 MB Infinity Cache cannot serve a
buffer from one use to the next.  A shallow rotation is not enough: the
token rows are read with ordinary loads, while the receive rows move with
non-temporal accesses that leave the cache alone, so three sets of the
Qwen3-30B-A3B shape (33 MB of token rows each) kept the token rows resident.
That step measured 140.4 us with 3 sets, 146.8 with 8, 150.0 with 16 and
150.2-150.6 with 24 to 48.  ``--warm`` chains the real tensors instead
(combine reads what dispatch wrote) as a secondary figure.

Timing: set-up runs one untimed step on every buffer set, then the warmup
steps; the headline is K steps of plain launches bracketed by
synchronisations (wall clock, no event inside).  An event pass of K more
steps in the same rotation then takes the dominant kernel's own start and
stop events and the step distribution; it never feeds `value`.

Prints ONE JSON line.  ``--gpus N`` with N > 1 is not supported (the path is
one GPU's share of the exchange).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
COLD_SPAN_BYTES = 12 << 30  # the rotating buffer sets span at least this much
MAX_SETS = 64
METRIC = "dispatch+combine fwd+bwd GB/s per layer and % of MI355X HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_30b_a3b")
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating buffer sets (cold HBM); 0: enough to span COLD_SPAN_BYTES, at least 3")
    ap.add_argument("--warm", action="store_true", help="chain tensors: combine reads dispatch's output")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--chunks-per-lane", type=int, default=0)
    ap.add_argument("--nontemporal", type=int, default=2)
    ap.add_argument("--waves-per-block", type=int, default=0)
    ap.add_argument("--layout-pairs", type=int, default=0)
    ap.add_argument("--gather-mode", type=int, default=0,
                    help="receive rows of the gathers: 0 by row width (LDS-staged from 4 KiB), "
                         "1 staged in LDS, 2 in registers")
    ap.add_argument("--events", choices=["kernel", "all", "none"], default="kernel",
                    help="HIP events of the event pass, which repeats the timed steps after the "
                         "headline loop (the headline loop itself records no event). kernel: the "
                         "dominant kernel's own start and stop on every --kernel-every-th step, and a "
                         "stop event bound to each step's last kernel (step times; it idles the queue "
                         "about 4.5 us); all: also "
                         "hipEventRecord around every call, and the dominant kernel timed on every "
                         "step (per-call diagnostics; the records cost GPU time); none: no event pass")
    ap.add_argument("--kernel-every", type=int, default=2,
                    help="in the event pass, time the dominant kernel on every n-th step (its start "
                         "event is a stream marker, about 3 us of GPU time; step times are taken "
                         "over the other steps)")
    ap.add_argument("--staged", action="store_true",
                    help="staged exchange: send buffer per destination partition, receiver-side "
                         "expansion, two-level combine")
    ap.add_argument("--pad-multiple", type=int, default=1,
                    help="pad every expert's receive segment to a multiple of this (zero rows)")
    ap.add_argument("--overlap", action="store_true",
                    help="the step beside a stand-in expert GEMM: alone, concurrent on two streams, and "
                         "with the step on a CU-masked stream of each --budgets size")
    ap.add_argument("--budgets", default="32,64,96,128,160,192",
                    help="CU budgets of the exchange for --overlap")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the 1 GiB copy that measures the achievable HBM ceiling")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps as captured HIP graphs (no per-call events)")
    ap.add_argument("--graph-steps", type=int, default=1,
                    help="with --graph, consecutive steps of the rotation per captured graph (a divisor "
                         "of --steps and --warmup)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# The step: a list of calls, each with its algorithmic row bytes
# --------------------------------------------------------------------------

# calls that write receive rows: with a padded layout they also write the
# zero padding rows of every expert segment
PADDING_WRITERS = ("dispatch", "dispatch_scaled", "combine_bwd", "combine_bwd_plain",
                   "expand_x", "expand_x_scaled", "expand_g", "expand_g_w")


def step_calls(cfg, staged=False, n_send=None, pad_rows=None):
    """[(name, kind, pass, algorithmic row bytes)] of one step, in order.

    Row bytes only (index and weight traffic, about 4-12 bytes per (t,k)
    pair per call, are reported apart): TH = T*H*b token-row bytes, RH =
    T*K*H*b receive-row bytes, NS = N_send*H*b send-buffer bytes (one row
    per (token, destination partition) pair; n_send[p] for pass p).  With a
    padded layout, pad_rows[p] zero rows are added to each write of
    receive rows.
    """
    TH = cfg.T * cfg.H * cfg.esize
    RH = cfg.R * cfg.H * cfg.esize
    if staged:
        calls = _staged_calls(cfg, TH, RH, [n * cfg.H * cfg.esize for n in n_send])
    elif not cfg.absorbed:
        calls = [("layout", "layout", 0, 0),
                 ("dispatch", "dispatch", 0, TH + RH),
                 ("combine", "combine", 0, RH + TH),
                 ("combine_bwd", "combine_bwd", 0, TH + 2 * RH),
                 ("dispatch_bwd", "dispatch_bwd", 0, RH + TH)]
    else:
        calls = []
        for p in range(3):
            calls += [(f"layout.{p}", "layout", p, 0),
                      (f"dispatch.{p}", "dispatch_scaled", p, TH + RH),
                      (f"combine.{p}", "combine_plain", p, RH + TH)]
        for p in (0, 2):
            calls += [(f"replay_layout.{p}", "layout", p, 0),
                      (f"replay_dispatch.{p}", "dispatch_scaled", p, TH + RH),
                      (f"combine_bwd.{p}", "combine_bwd_plain", p, TH + RH),
                      (f"dispatch_bwd.{p}", "dispatch_bwd_scaled", p, RH + 2 * TH)]
    if pad_rows:
        calls = [(n, k, p, b + (pad_rows[p] * cfg.H * cfg.esize if k in PADDING_WRITERS else 0))
                 for n, k, p, b in calls]
    return calls


def _staged_calls(cfg, TH, RH, NS):
    """The same step through the staged exchange: every dispatch is send +
    expand, every combine is reduce_partitions + combine_partitions ("merge"),
    and a router-side gradient is a row-free dot call of its own."""
    if not cfg.absorbed:
        n = NS[0]
        return [("layout", "layout", 0, 0),
                ("dispatch:send", "send_x", 0, TH + n),
                ("dispatch:expand", "expand_x", 0, n + RH),
                ("combine:reduce", "reduce_y_w", 0, RH + n),
                ("combine:merge", "merge_out", 0, n + TH),
                ("combine_bwd:send", "send_g", 0, TH + n),
                ("combine_bwd:expand", "expand_g_w", 0, n + RH),
                ("combine_bwd:dot", "dot_w", 0, TH + RH),
                ("dispatch_bwd:reduce", "reduce_gr", 0, RH + n),
                ("dispatch_bwd:merge", "merge_gx", 0, n + TH)]
    calls = []
    for p in range(3):
        n = NS[p]
        calls += [(f"layout.{p}", "layout", p, 0),
                  (f"dispatch.{p}:send", "send_x", p, TH + n),
                  (f"dispatch.{p}:expand", "expand_x_scaled", p, n + RH),
                  (f"combine.{p}:reduce", "reduce_y", p, RH + n),
                  (f"combine.{p}:merge", "merge_out", p, n + TH)]
    for p in (0, 2):
        n = NS[p]
        calls += [(f"replay_layout.{p}", "layout", p, 0),
                  (f"replay_dispatch.{p}:send", "send_x", p, TH + n),
                  (f"replay_dispatch.{p}:expand", "expand_x_scaled", p, n + RH),
                  (f"combine_bwd.{p}:send", "send_g", p, TH + n),
                  (f"combine_bwd.{p}:expand", "expand_g", p, n + RH),
                  (f"dispatch_bwd.{p}:reduce", "reduce_gr_w", p, RH + n),
                  (f"dispatch_bwd.{p}:merge", "merge_gx", p, n + TH),
                  (f"dispatch_bwd.{p}:dot", "dot_s", p, RH + TH)]
    return calls


def index_bytes(cfg, staged=False, n_send=None, pad_rows=None):
    """Index, weight and score traffic per step (reported apart from `value`)."""
    R, T = cfg.R, cfg.T
    per = {"layout": R * 4 * 2 + R * 4 * 3 + T * cfg.P * 5 + T * 8 * 2 + T * 8,
           "dispatch": R * 4 * 3, "dispatch_scaled": R * 4 * 3, "combine": R * 4 * 2,
           "combine_plain": R * 4, "combine_bwd": R * 4 * 3, "combine_bwd_plain": R * 4,
           "dispatch_bwd": R * 4, "dispatch_bwd_scaled": R * 4 * 3}
    # staged calls: per token its partition mask and send slots; per pair its
    # receive row, weight and score as used; per send row its token
    tok = T * (8 + cfg.P * 4)
    per.update(send_x=tok, send_g=tok, merge_out=tok, merge_gx=tok, dot_w=R * 4 * 3, dot_s=R * 4 * 3)
    ns = max(n_send) * 4 if n_send else 0
    for kind, words in (("expand_x", 3), ("expand_x_scaled", 3), ("expand_g", 1), ("expand_g_w", 2),
                        ("reduce_y_w", 2), ("reduce_y", 1), ("reduce_gr", 1), ("reduce_gr_w", 2)):
        per[kind] = R * 4 * words + ns
    return sum(per[kind] for _, kind, _, _ in step_calls(cfg, staged, n_send, pad_rows))


# The call whose kernel the roofline reports, the step's longest launch
# measured cold: the dispatch's row scatter on every direct shape
# (Qwen3-30B-A3B 29.0 us against 27.3 for the combine's gather; DeepSeek-V3
# 110.0 against 97.2; the
# DiffusionGemma scaled dispatch 78.6 us, five times a step), and on the
# staged path the dispatch's expansion (39.5 us, beside the combine
# backward's scaled expansion at 40.6 and the partition reduce at 37.4).
DOMINANT = {False: "dispatch", True: "dispatch:expand"}
DOMINANT_KERNEL = {False: "scatter_kernel: token row to its K receive rows",
                   True: "expand_kernel: send row to its pairs' receive rows"}
# what the committed traffic counters describe: the dominant kernel's
# function, its launcher, and the device headers it uses
KERNEL_SOURCES = {False: ("row_kernels.hip", ("scatter_kernel", "go_scatter"), ("device_common.h", "pad_fill.h")),
                  True: ("staged_kernels.hip", ("expand_kernel", "go_expand"), ("device_common.h", "pad_fill.h"))}


def rotation(nsets, warmup, steps):
    """Buffer-set indices of each phase of a run: set-up (every set once),
    warmup, the headline steps and the event-pass steps.  The timed phases
    continue the warmup's rotation, so a set used by a timed step was last
    used nsets - 1 steps earlier (with at least as many steps run before it)."""
    first = warmup % nsets
    return {"setup": list(range(nsets)),
            "warmup": [i % nsets for i in range(warmup)],
            "headline": [(first + i) % nsets for i in range(steps)],
            "event": [(first + steps + i) % nsets for i in range(steps)]}


def dominant_call(cfg, staged=False):
    name = DOMINANT[staged]
    if not cfg.absorbed:
        return name
    return name.replace("dispatch", "dispatch.0", 1)


def function_text(src, name):
    """Source text of the function `name` in `src`: from the template line
    before its definition to the closing brace in column 0."""
    m = re.search(r"^template <[^\n]*>\n(?:__global__[^\n]*|hipError_t) %s\(" % re.escape(name), src, re.M)
    if m is None:
        raise ValueError(f"{name} not found")
    end = src.index("\n}\n", m.start())
    return src[m.start():end + 3]


def kernel_source_hash(staged=False):
    """Hash of the dominant kernel's source (the counters' subject): its
    function, its launcher and the device headers it uses."""
    csrc = os.path.join(ROOT, "combine_moe_layout_04_amd", "csrc")
    path, funcs, headers = KERNEL_SOURCES[staged]
    src = open(os.path.join(csrc, path)).read()
    h = hashlib.sha256()
    for f in funcs:
        h.update(function_text(src, f).encode())
    for name in headers:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def sources_hash():
    """Hash of every library source and the public header: which code a result
    line measured (the repository's history does not travel with the tree)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_moe_layout_04_amd", "csrc")
    paths = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    inc = os.path.join(ROOT, "include")
    headers = sorted(os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h"))
    for path in paths + headers:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(cfg, staged=False):
    """HBM bytes per launch of the dominant call's kernel from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, calibrated on a copy of known
    size), or None when its sources have changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    call = DOMINANT[staged]
    m = re.search(r"^source_hash\.%s: (\w+)$" % re.escape(call), text, re.M)
    if m is None or m.group(1) != kernel_source_hash(staged):
        return None
    m = re.search(r"^traffic_bytes_per_launch\.%s: (\d+)$" % re.escape(call), text, re.M)
    return None if m is None else int(m.group(1))


class HipEvents:
    """Timing-only HIP events on torch's current stream, created with
    hipEventDisableSystemFence so that recording one does not write back and
    invalidate the caches (a default event's system-scope fence adds about
    3 us to the interval it brackets).  Uses the HIP runtime instance torch
    and the library already share in this process."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import torch

        torch.cuda.init()
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.L = L = ctypes.CDLL(path)
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if L.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)
        self._ms = ctypes.c_float()

    def record(self, i, stream):
        if self.L.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        if self.L.hipEventElapsedTime(ctypes.byref(self._ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return self._ms.value

    def close(self):
        for e in self.ev:
            self.L.hipEventDestroy(e)
        self.ev = []


# --------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the same step
# --------------------------------------------------------------------------

def cpu_baseline(cfg, budget_s, staged=False, pad_multiple=1):
    import numpy as np

    import workloads as W
    from oracle import moe_oracle as O

    dt = cfg.dtype
    m = pad_multiple
    passes = 3 if cfg.absorbed else 1
    inps = [W.layer_inputs(cfg, seed=0, pss=p) for p in range(passes)]
    if m > 1:  # receive-row inputs span the padded capacity
        extra = cfg.E * (m - 1)
        inps = [i.__class__(i.cfg, i.topk_idx, i.topk_weights, i.x,
                            np.concatenate([i.y, np.zeros((extra, cfg.H), i.y.dtype)]), i.g,
                            np.concatenate([i.grad_recv, np.zeros((extra, cfg.H), i.y.dtype)]))
                for i in inps]
    lays = [O.layout(inp.topk_idx, cfg.E, cfg.P, m) for inp in inps]
    calls = step_calls(cfg, staged, [l.n_send for l in lays],
                       [int(l.expert_offset[-1]) - cfg.R for l in lays])
    step_b = sum(b for _, _, _, b in calls)
    lay = {}
    st = {}  # staged: the last send buffer and partial rows of each pass
    n_calls, moved = 0, 0
    t0 = time.perf_counter()
    out_of_time = False
    # the step's calls in order, step after step, until the budget is spent
    while not out_of_time and n_calls < 50 * len(calls):
        for name, kind, p, b in calls:
            inp = inps[p]
            w = inp.topk_weights
            if kind == "layout":
                lay[p] = L = O.layout(inp.topk_idx, cfg.E, cfg.P, m)
            L = lay[p]
            if kind == "dispatch":
                O.dispatch(L, inp.x, dt, w)
            elif kind == "dispatch_scaled":
                O.dispatch(L, inp.x, dt, w, scale_rows=True)
            elif kind == "combine":
                O.combine(L, inp.y, dt, w)
            elif kind == "combine_plain":
                O.combine(L, inp.y, dt)
            elif kind == "combine_bwd":
                O.combine_bwd(L, inp.g, dt, w, inp.y)
            elif kind == "combine_bwd_plain":
                O.combine_bwd(L, inp.g, dt)
            elif kind == "dispatch_bwd":
                O.dispatch_bwd(L, inp.grad_recv, dt)
            elif kind == "dispatch_bwd_scaled":
                O.dispatch_bwd(L, inp.grad_recv, dt, w, inp.x)
            elif kind in ("send_x", "send_g"):
                st[p, "S"] = O.send(L, inp.x if kind == "send_x" else inp.g)
            elif kind in ("expand_x", "expand_x_scaled", "expand_g", "expand_g_w"):
                O.expand(L, st[p, "S"], dt, None if kind == "expand_g" else w,
                         kind in ("expand_x_scaled", "expand_g_w"))
            elif kind in ("reduce_y_w", "reduce_y", "reduce_gr", "reduce_gr_w"):
                rows = inp.y if kind.startswith("reduce_y") else inp.grad_recv
                st[p, "Q"] = O.reduce_partitions(L, rows, dt, w if kind.endswith("_w") else None)
            elif kind in ("merge_out", "merge_gx"):
                O.combine_partitions(L, st[p, "Q"], dt)
            elif kind == "dot_w":
                O.canonical_dot(np.repeat(inp.g, cfg.K, axis=0), inp.y[L.recv_pos.reshape(-1)], dt)
            elif kind == "dot_s":
                O.canonical_dot(inp.grad_recv[L.recv_pos.reshape(-1)], np.repeat(inp.x, cfg.K, axis=0), dt)
            elif kind != "layout":
                raise ValueError(kind)
            n_calls += 1
            moved += b
            if time.perf_counter() - t0 >= budget_s:
                out_of_time = True
                break
    done_steps = n_calls // len(calls)
    el = time.perf_counter() - t0
    return {
        "value": round(moved / el / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "host_cpus": os.cpu_count(),
        "cpu_affinity": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{done_steps} whole steps + {n_calls - done_steps * len(calls)} calls of the "
                  f"{cfg.name} {'staged ' if staged else ''}step (T={cfg.T}, H={cfg.H}, {dt}; "
                  f"{step_b / 1e6:.1f} MB of rows per step), numpy single-threaded, {el:.1f} s",
    }


# --------------------------------------------------------------------------
# Overlap with a stand-in expert GEMM, and the exchange's CU budget
# --------------------------------------------------------------------------

# Qwen3-30B-A3B's expert FFN width: the stand-in GEMM is the layer's gate+up
# projection, [T*K, H] x [H, 2*768], in bf16.
EXPERT_FFN = 768


def overlap_run(args, cfg, step, sets, nsets, calls, n_send, pad_rows):
    """Exchange steps and stand-in GEMMs, K of each: alone on the full GPU,
    concurrent on two ordinary streams, and for every CU budget N concurrent
    with the exchange on CUs [0, N) and the GEMM on the other CUs (each
    also timed alone on its CUs).  Wall time for all K of both."""
    import torch

    import combine_moe_layout_04_amd as M

    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    R, H, F2 = cfg.R, cfg.H, 2 * EXPERT_FFN
    A = [torch.randn((R, H), device=dev).to(torch.bfloat16) for _ in range(2)]
    B = torch.randn((H, F2), device=dev).to(torch.bfloat16).contiguous()
    C = [torch.empty((R, F2), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    K = args.steps
    gemm_flop = 2.0 * R * H * F2

    def gemm(i):
        torch.matmul(A[i % 2], B, out=C[i % 2])

    def xstep(i):
        step(sets[i % nsets])

    def timed(parts):
        """parts: [(stream or None, fn(i))], enqueued interleaved so that both
        streams stay fed; wall us per iteration (K of each)."""
        cur = torch.cuda.current_stream()

        def run(n):
            for i in range(n):
                for st, fn in parts:
                    with torch.cuda.stream(st if st is not None else cur):
                        fn(i)

        run(max(2, args.warmup // 4))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(K)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / K

    t_x = timed([(None, xstep)])
    t_g = timed([(None, gemm)])
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    t_both = timed([(sa, xstep), (sb, gemm)])
    rows = []
    for n in [int(b) for b in args.budgets.split(",") if b]:
        if not 0 < n < ncu:
            continue
        xs, gs = M.CuBudgetStream(0, n), M.CuBudgetStream(n, ncu - n)
        try:
            tx = timed([(xs.stream, xstep)])
            tg = timed([(gs.stream, gemm)])
            tb = timed([(xs.stream, xstep), (gs.stream, gemm)])
            # only the exchange confined: the GEMM may use every CU
            tbf = timed([(xs.stream, xstep), (sb, gemm)])
        finally:
            xs.close()
            gs.close()
        rows.append({"exchange_cus": n, "gemm_cus": ncu - n, "exchange_alone_us": round(tx, 2),
                     "gemm_alone_us": round(tg, 2), "concurrent_us": round(tb, 2),
                     "speedup_vs_serial": round((t_x + t_g) / tb, 3),
                     "concurrent_gemm_unmasked_us": round(tbf, 2),
                     "speedup_gemm_unmasked": round((t_x + t_g) / tbf, 3)})
    best = min(rows, key=lambda r: min(r["concurrent_us"], r["concurrent_gemm_unmasked_us"])) if rows else None
    step_b = sum(b for *_, b in calls)
    line = {
        "metric": "exchange step beside a stand-in expert GEMM: wall us per (step + GEMM)",
        "value": round(min(best["concurrent_us"], best["concurrent_gemm_unmasked_us"]) if best else t_both, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "higher_is_better": False,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: T={cfg.T} H={H} {cfg.dtype} E={cfg.E} P={cfg.P} K={cfg.K}; "
                        f"stand-in GEMM [{R},{H}]x[{H},{F2}] bf16 (gate+up projection of the experts)",
            "exchange_alone_us": round(t_x, 2),
            "exchange_TBps": round(step_b / (t_x * 1e-6) / 1e12, 3),
            "gemm_alone_us": round(t_g, 2),
            "gemm_TFLOPs": round(gemm_flop / (t_g * 1e-6) / 1e12, 1),
            "serial_us": round(t_x + t_g, 2),
            "concurrent_two_streams_us": round(t_both, 2),
            "speedup_two_streams": round((t_x + t_g) / t_both, 3),
            "cu_budgets": rows,
            "best_budget_cus": best["exchange_cus"] if best else None,
            "cus": ncu,
        },
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the exchange; --gpus {args.gpus} is not "
              "supported (this path has no collectives and runs on one GPU).", file=sys.stderr)
        sys.exit(2)
    G = args.graph_steps
    if G < 1 or (G > 1 and (not args.graph or args.steps % G or args.warmup % G)):
        print("--graph-steps needs --graph and must divide --steps and --warmup", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    import combine_moe_layout_04_amd as M
    from combine_moe_layout_04_amd._lib import lib

    lib()  # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = W.get_config(args.config)
    dt = cfg.dtype
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    passes = 3 if cfg.absorbed else 1

    def dev_rows(a):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # inputs: per pass a routing and token rows; expert outputs and
    # gradients are shared by the passes
    base = W.layer_inputs(cfg, seed=0)
    y0, g0, gr0 = (dev_rows(a) for a in (base.y, base.g, base.grad_recv))
    m = args.pad_multiple
    RC = cfg.R + cfg.E * (m - 1)  # receive rows: T*K plus the padding capacity
    if RC > cfg.R:
        y0, gr0 = (torch.cat([a, torch.zeros((RC - cfg.R, cfg.H), dtype=a.dtype, device=dev)])
                   for a in (y0, gr0))
    per_pass = []
    for p in range(passes):
        inp = base if p == 0 else W.layer_inputs(cfg, seed=0, pss=p, with_rows=False)
        x = dev_rows(base.x if p == 0 else W.normal_rows(cfg, cfg.T, 1, seed=0, pss=p))
        per_pass.append((torch.from_numpy(inp.topk_idx).to(dev), torch.from_numpy(inp.topk_weights).to(dev), x))
    del base

    def empty_rows(n):
        return torch.empty((n, cfg.H), dtype=tdt, device=dev)

    ws_bytes = M.moe_workspace_size(cfg.T, cfg.K, cfg.E, cfg.P, m)
    sets = []

    def set_bytes(s):
        n = sum(t.numel() * t.element_size() for k, t in s.items() if torch.is_tensor(t))
        return n + sum(t.numel() * t.element_size() for q in s["pass"] for t in q.values() if torch.is_tensor(t))

    nsets = 1 if args.warm else max(1, args.sets)
    while len(sets) < nsets:
        s = {"pass": [], "y": y0.clone(), "g": g0.clone()}
        if not args.warm:
            s["y_bwd"] = y0.clone()      # the backward's own copy of the expert output
            s["grad_recv"] = gr0.clone()
        for idx, w, x in per_pass:
            s["pass"].append(dict(
                idx=idx.clone(), w=w.clone(), x=x.clone(),
                recv=empty_rows(RC), scores=torch.empty(RC, dtype=torch.float32, device=dev),
                out=empty_rows(cfg.T),
                ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
                h=M.Handle(args.chunks_per_lane, args.nontemporal, args.waves_per_block, args.layout_pairs,
                           pad_multiple=m, gather_mode=args.gather_mode)))
        s["grad_y"] = empty_rows(RC)
        s["grad_w"] = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device=dev)
        s["grad_x"] = empty_rows(cfg.T)
        sets.append(s)
        if not args.warm and args.sets <= 0 and len(sets) == 1:
            nsets = min(MAX_SETS, max(3, -(-COLD_SPAN_BYTES // max(1, set_bytes(s)))))
    del y0, g0, gr0, per_pass

    # padding rows of each pass's routing (the same in every buffer set)
    pad_rows = []
    for q in sets[0]["pass"]:
        M.moe_layout(q["idx"], cfg.E, cfg.P, handle=q["h"], workspace=q["ws"])
        pad_rows.append(int(q["h"].field("expert_offset")[-1].item()) - cfg.R)

    n_send = None
    if args.staged:
        # Send buffers and partial rows.  A transport would carry each sent
        # buffer (S_out, Q_out) into the peer's receive buffer (S_in, Q_in);
        # cold, the receive buffers are separate ones, filled once here with
        # valid rows and last touched a full buffer rotation ago; warm, they
        # are the buffers just written.
        n_send = []
        for s in sets:
            for p, q in enumerate(s["pass"]):
                M.moe_layout(q["idx"], cfg.E, cfg.P, handle=q["h"], workspace=q["ws"])
                cap = M.moe_send_capacity(q["h"])
                q["S_out"], q["Q_out"] = empty_rows(cap), empty_rows(cap)
                M.moe_send(q["h"], q["x"], send=q["S_out"])
                M.moe_reduce_partitions(q["h"], s["y"], q["w"], partial=q["Q_out"])
                if args.warm:
                    q["S_in"], q["Q_in"] = q["S_out"], q["Q_out"]
                else:
                    q["S_in"], q["Q_in"] = q["S_out"].clone(), q["Q_out"].clone()
                if s is sets[0]:
                    n_send.append(int(q["h"].field("send_offset")[-1].item()))
    torch.cuda.synchronize()

    calls = step_calls(cfg, args.staged, n_send, pad_rows)
    names = [c[0] for c in calls]
    ncall = len(calls)
    dom = dominant_call(cfg, args.staged)

    def run_call(s, kind, p):
        q = s["pass"][p]
        h = q["h"]
        if kind == "layout":
            M.moe_layout(q["idx"], cfg.E, cfg.P, handle=h, workspace=q["ws"])
        elif kind == "dispatch":
            M.moe_dispatch(h, q["x"], q["w"], recv=q["recv"], recv_scores=q["scores"])
        elif kind == "dispatch_scaled":
            M.moe_dispatch(h, q["x"], q["w"], scale_rows=True, recv=q["recv"], recv_scores=q["scores"])
        elif kind in ("combine", "combine_plain"):
            y = q["recv"] if args.warm else s["y"]
            M.moe_combine(h, y, q["w"] if kind == "combine" else None, out=q["out"])
        elif kind == "combine_bwd":
            yb = q["recv"] if args.warm else s["y_bwd"]
            M.moe_combine_bwd(h, s["g"], q["w"], yb, grad_y=s["grad_y"], grad_w=s["grad_w"])
        elif kind == "combine_bwd_plain":
            M.moe_combine_bwd(h, s["g"], grad_y=s["grad_y"])
        elif kind == "dispatch_bwd":
            gr = s["grad_y"] if args.warm else s["grad_recv"]
            M.moe_dispatch_bwd(h, gr, grad_x=s["grad_x"])
        elif kind == "dispatch_bwd_scaled":
            gr = s["grad_y"] if args.warm else s["grad_recv"]
            M.moe_dispatch_bwd(h, gr, q["w"], q["x"], grad_x=s["grad_x"], grad_s=s["grad_w"])
        # staged exchange
        elif kind in ("send_x", "send_g"):
            M.moe_send(h, q["x"] if kind == "send_x" else s["g"], send=q["S_out"])
        elif kind in ("expand_x", "expand_x_scaled"):
            M.moe_expand(h, q["S_in"], q["w"], scale_rows=kind == "expand_x_scaled",
                         recv=q["recv"], recv_scores=q["scores"])
        elif kind in ("expand_g", "expand_g_w"):
            M.moe_expand(h, q["S_in"], q["w"] if kind == "expand_g_w" else None,
                         scale_rows=kind == "expand_g_w", recv=s["grad_y"])
        elif kind in ("reduce_y", "reduce_y_w"):
            y = q["recv"] if args.warm else s["y"]
            M.moe_reduce_partitions(h, y, q["w"] if kind == "reduce_y_w" else None, partial=q["Q_out"])
        elif kind in ("reduce_gr", "reduce_gr_w"):
            gr = s["grad_y"] if args.warm else s["grad_recv"]
            M.moe_reduce_partitions(h, gr, q["w"] if kind == "reduce_gr_w" else None, partial=q["Q_out"])
        elif kind in ("merge_out", "merge_gx"):
            M.moe_combine_partitions(h, q["Q_in"], out=q["out"] if kind == "merge_out" else s["grad_x"])
        elif kind == "dot_w":
            yb = q["recv"] if args.warm else s["y_bwd"]
            M.moe_combine_bwd(h, s["g"], q["w"], yb, grad_y=False, grad_w=s["grad_w"])
        elif kind == "dot_s":
            gr = s["grad_y"] if args.warm else s["grad_recv"]
            M.moe_dispatch_bwd(h, gr, q["w"], q["x"], grad_x=False, grad_s=s["grad_w"])
        else:
            raise ValueError(kind)

    def step(s, ev=None, i=None):
        # ev: the event pass's events, i: its step index.  The dominant
        # call's kernel may record its own start and stop, the last call's
        # kernel binds the step's stop event, and with --events all every
        # call is bracketed by records.  The headline loop passes no events.
        for j, (_, kind, p, _) in enumerate(calls):
            slot = None
            if ev is not None:
                h = s["pass"][p]["h"]
                if j == d and i in ev["kslot"]:
                    r = ev["kslot"][i]
                    M.moe_time_next_kernel(h, ev["kev"].ev[2 * r].value, ev["kev"].ev[2 * r + 1].value)
                if j == ncall - 1 and ev["bev"] is not None:
                    M.moe_time_next_kernel(h, None, ev["bev"].ev[i].value)
                slot = ev["slot_of"].get(j)
                if slot is not None:
                    ev["hev"].record(ev["per_step"] * i + 2 * slot, stream)
            run_call(s, kind, p)
            if slot is not None:
                ev["hev"].record(ev["per_step"] * i + 2 * slot + 1, stream)

    d = names.index(dom)
    assert d != ncall - 1, "the step's last call carries the step-boundary event"
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # Set-up, untimed: every buffer set runs one step, so that no set is
    # first touched inside a timed region.  Then the warmup steps, and the
    # timed steps continue the same rotation: every set is last touched
    # nsets - 1 steps before its next use.
    order = rotation(nsets, args.warmup, args.steps)
    for j in order["setup"]:
        step(sets[j])
    for j in order["warmup"]:
        step(sets[j])
    for s in sets:
        for q in s["pass"]:
            assert q["h"].check() == 0
    first = args.warmup % nsets

    def set_of(i):  # timed step i (headline, then event pass) of the rotation
        return sets[(first + i) % nsets]

    if args.overlap:
        overlap_run(args, cfg, step, sets, nsets, calls, n_send, pad_rows)
        return

    graphs = None
    if args.graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for s in sets:
                step(s)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for j in range(nsets):  # graph j: the G steps of the rotation from set j on
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for u in range(G):
                    step(sets[(j + u) % nsets])
            graphs.append(g)
        for g in graphs:
            g.replay()
        for i in range(0, args.warmup, G):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()
    eager = graphs is None

    def run_steps(K, start, ev=None):
        # steps start .. start+K-1 of the rotation
        if not eager:  # one replay runs G steps
            for i in range(0, K, G):
                if ev is not None:
                    ev["sev"].record(i // G, stream)
                graphs[(first + start + i) % nsets].replay()
            if ev is not None:
                ev["sev"].record(K // G, stream)
            return
        for i in range(K):
            step(set_of(start + i), ev, i)

    # The headline: K steps of plain launches (or graph replays), bracketed
    # by synchronisations, wall clock only.  No event is recorded or bound
    # inside it.
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(K, 0)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    host_us = (t_enq - t0) * 1e6 / K

    # The event pass: K more steps of the same rotation, with
    # HIP events on the stream the library launches on.  It gives the
    # dominant kernel's own duration (its start and stop events, on every
    # other step) and the step distribution (a stop event bound to each
    # step's last kernel (it idles the queue about 4.5 us before the next
    # kernel); taken over the steps without a start marker,
    # which costs about 3 us).  Its wall time is reported beside the
    # headline's, never as it.
    events = args.events if eager else ("none" if args.events == "none" else "graph")
    ev = None
    ev_ms_per_step = None
    kern_us, call_ms, st = None, {}, None
    ksteps = []
    if events != "none":
        timed = list(range(ncall)) if events == "all" else []  # --events all: records around every call
        every = 1 if events == "all" else max(1, args.kernel_every)
        ksteps = [i for i in range(K) if i % every == 0] if events in ("kernel", "all") else []
        ev = {"slot_of": {j: r for r, j in enumerate(timed)}, "per_step": 2 * len(timed),
              "kslot": {i: r for r, i in enumerate(ksteps)}}
        ev["hev"] = HipEvents(ev["per_step"] * K)
        ev["kev"] = HipEvents(2 * len(ksteps))
        ev["bev"] = HipEvents(K) if eager else None
        ev["sev"] = HipEvents(K // G + 1 if not eager else 0)
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        run_steps(K, K, ev)  # the rotation continues where the headline left it
        torch.cuda.synchronize()
        ev_ms_per_step = (time.perf_counter() - e0) * 1e3 / K
        call_ms = {names[j]: [ev["hev"].elapsed_ms(ev["per_step"] * i + 2 * r, ev["per_step"] * i + 2 * r + 1)
                              for i in range(K)] for r, j in enumerate(timed)}
        kern_us = [ev["kev"].elapsed_ms(2 * r, 2 * r + 1) * 1e3 for r in range(len(ksteps))] or None
        if eager and K > 1:   # end of step i-1's last kernel to end of step i's
            clean = [i for i in range(1, K) if i not in ev["kslot"]] or list(range(1, K))
            st = np.array([ev["bev"].elapsed_ms(i - 1, i) for i in clean]) * 1e3
        elif not eager:  # per replay, divided over its G steps
            st = np.array([ev["sev"].elapsed_ms(i, i + 1) for i in range(K // G)]) * 1e3 / G
        for k in ("hev", "kev", "bev", "sev"):
            if ev[k] is not None:
                ev[k].close()

    avg_us = {n: float(np.mean(v)) * 1e3 for n, v in call_ms.items()}
    med_us = {n: float(np.median(v)) * 1e3 for n, v in call_ms.items()}
    step_us = None if st is None else {
        "median": round(float(np.median(st)), 2), "p10": round(float(np.percentile(st, 10)), 2),
        "p90": round(float(np.percentile(st, 90)), 2), "n": int(len(st))}
    per_pass = None
    if cfg.absorbed and len(avg_us) == ncall:
        # each forward pass, and each replay + backward
        def of_pass(n, p):
            return n.endswith(f".{p}") or f".{p}:" in n

        per_pass = {f"fwd.{p}": round(sum(v for n, v in avg_us.items()
                                          if n.startswith(("layout.", "dispatch.", "combine.")) and of_pass(n, p)), 2)
                    for p in range(3)}
        per_pass.update({f"replay_bwd.{p}": round(sum(v for n, v in avg_us.items()
                                                      if n.startswith(("replay_", "combine_bwd", "dispatch_bwd"))
                                                      and of_pass(n, p)), 2)
                         for p in (0, 2)})

    # the achievable ceiling: a plain device copy of 1 GiB (2 GiB moved), median of 5
    ceiling = None
    if not args.no_ceiling:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        cev = HipEvents(12)
        for i in range(6):
            cev.record(2 * i, stream)
            M.moe_bench_copy(dst, src)
            cev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        cus = sorted(cev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(1, 6))
        cev.close()
        del src, dst
        ceiling = round(2.0 * (1 << 30) / (cus[2] * 1e-6) / 1e9, 1)

    # the copy kernel of known size, untimed: calibrates the traffic counters
    cbuf = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(cbuf)
    M.moe_bench_copy(cdst, cbuf)
    torch.cuda.synchronize()
    del cbuf, cdst

    row_bytes = {n: b for n, _, _, b in calls}
    step_b = sum(row_bytes.values())
    value = step_b / (ms_per_step * 1e-3) / 1e9
    # the dominant kernel's duration: its own start and stop events
    # (hipExtLaunchKernel), which leave out the launch latency that the events
    # around the call include
    dom_us = None if kern_us is None else float(np.mean(kern_us))
    achieved = None if dom_us is None else row_bytes[dom] / (dom_us * 1e-6) / 1e9
    traffic = traffic_from_profiles(cfg, args.staged)
    direct_b = sum(b for _, _, _, b in step_calls(cfg))

    protocol = ("layout+dispatch+combine+combine_bwd+dispatch_bwd per step" if not cfg.absorbed else
                "3 forward passes (layout, scaled dispatch, plain combine) + replay of layout and "
                "dispatch and backward (combine_bwd copy, scaled dispatch_bwd with score gradient) "
                "for passes 1 and 3, per step")
    if args.staged:
        protocol += ("; staged exchange: dispatch = send + expand, combine = reduce_partitions + "
                     "combine_partitions, router-side gradients as row-free dot calls")
    if m > 1:
        protocol += f"; expert segments padded to a multiple of {m} (zero rows and scores)"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: T={cfg.T} H={cfg.H} {dt} E={cfg.E} P={cfg.P} K={cfg.K}, {protocol}",
            "cache": ("warm (chained tensors)" if args.warm else
                      f"cold ({nsets} rotating buffer sets, {nsets * set_bytes(sets[0]) / 1e9:.1f} GB)"),
            "bytes_per_step": step_b,
            "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
            "us_per_step": round(ms_per_step * 1e3, 2),
            **({} if not avg_us else {  # --events all: per-call intervals, records included
                "call_avg_us": {n: round(v, 2) for n, v in avg_us.items()},
                "call_median_us": {n: round(v, 2) for n, v in med_us.items()},
                "call_GBps": {n: round(row_bytes[n] / (avg_us[n] * 1e-6) / 1e9, 1) for n in avg_us if row_bytes[n]},
            }),
            "index_bytes_per_step": index_bytes(cfg, args.staged, n_send, pad_rows),
            **({} if m == 1 else {"pad_multiple": m, "padding_rows": pad_rows}),
            "host_enqueue_us_per_step": round(host_us, 1),
            "event_pass_us_per_step": None if ev_ms_per_step is None else round(ev_ms_per_step * 1e3, 2),
            "step_us": step_us,
            **({} if per_pass is None else {"per_pass_us": per_pass}),
            "timing": (f"hip graph replays, {G} step(s) per graph" if graphs is not None else "eager launches") +
                      f"; headline loop without events, set-up touches all {nsets} sets first; event pass "
                      f"(same {K} steps): {events}" +
                      (f", dominant kernel timed on {len(ksteps)} of {K} steps" if ksteps else ""),
            **({} if not args.staged else {
                "exchange": "staged",
                "n_send": n_send,
                # rows a transport would move per exchange: one per (token,
                # partition) pair here, one per (token, k) pair when direct
                "exchange_bytes_per_step": sum(n_send[p] for _, kind, p, _ in calls
                                               if kind.startswith(("send", "reduce"))) * cfg.H * cfg.esize,
                "direct_exchange_bytes_per_step": sum(1 for _, kind, _, _ in calls
                                                      if kind.startswith(("send", "reduce")))
                                                  * cfg.R * cfg.H * cfg.esize,
                "direct_step_bytes_per_s_GBps": round(direct_b / (ms_per_step * 1e-3) / 1e9, 2),
            }),
            "tuning": {"chunks_per_lane": args.chunks_per_lane, "nontemporal": args.nontemporal,
                       "waves_per_block": args.waves_per_block, "layout_pairs": args.layout_pairs,
                       "gather_mode": args.gather_mode},
            "sources_sha256": sources_hash(),
        },
        "roofline": None if achieved is None else {
            "bound": "hbm",
            "kernel": f"{dom} ({DOMINANT_KERNEL[args.staged]})",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": row_bytes[dom],
            "avg_launch_us": round(dom_us, 2),
            "median_launch_us": round(float(np.median(kern_us)), 2),
            "launch_timing": f"the kernel's own start and stop events (hipExtLaunchKernel), on {len(ksteps)} "
                             f"of the {K} steps of the event pass",
            **({} if dom not in avg_us else {"call_interval_avg_us": round(avg_us[dom], 2)}),
            "achievable_copy_GBps": ceiling,
            "frac_of_achievable": None if ceiling is None else round(achieved / ceiling, 4),
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(cfg, args.cpu_seconds, args.staged, m),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
