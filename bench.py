"""Benchmark: MoE dispatch + combine, forward + backward, per layer, on one GPU.

One step is one pass of the whole hot path over one layer's synthetic input:
layout (counts, offsets, stable positions) -> dispatch (with per-row scores)
-> combine (top-k weighted) -> combine backward (rows + router-weight
gradient) -> dispatch backward.  The expert in between is the identity, so
there is no GEMM: the path is HBM-bound and is measured against the HBM
roofline.

Cold HBM: every kernel of a step reads buffers that were last touched more
than 1 GB of traffic earlier (several rotating buffer sets, and the combine
backward reads its own copy of the expert output), so the 256 MB Infinity
Cache cannot serve them.  ``--warm`` chains the real tensors instead
(combine reads what dispatch wrote) as a secondary figure.

Prints ONE JSON line.  ``--gpus N`` with N > 1 is not supported (the path is
one GPU's share of the exchange).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_30b_a3b")
    ap.add_argument("--sets", type=int, default=3, help="rotating buffer sets (cold HBM)")
    ap.add_argument("--warm", action="store_true", help="chain tensors: combine reads dispatch's output")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--chunks-per-lane", type=int, default=0)
    ap.add_argument("--nontemporal", type=int, default=1)
    ap.add_argument("--waves-per-block", type=int, default=0)
    ap.add_argument("--layout-pairs", type=int, default=0)
    ap.add_argument("--events", choices=["all", "dominant", "none"], default="dominant",
                    help="HIP events in the timed region: around every call, around the "
                         "dominant kernel's call only, or none")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (no per-call events)")
    return ap.parse_args()


def layer_bytes(cfg):
    """Algorithmic payload bytes per kernel (rows only; index traffic apart)."""
    TH = cfg.T * cfg.H * cfg.esize
    RH = cfg.R * cfg.H * cfg.esize
    R, T, K = cfg.R, cfg.T, cfg.K
    rows = {
        "dispatch": TH + RH,
        "combine": RH + TH,
        "combine_bwd": TH + 2 * RH,
        "dispatch_bwd": RH + TH,
        "layout": 0,
    }
    # index / weight traffic: recv_pos reads, weights, scores, grad_w; layout
    # reads topk_idx and writes the handle arrays
    index = {
        "dispatch": R * 4 * 3,            # recv_pos, weights, recv_scores
        "combine": R * 4 * 2,             # recv_pos, weights
        "combine_bwd": R * 4 * 3,         # recv_pos, weights, grad_w
        "dispatch_bwd": R * 4,            # recv_pos
        "layout": R * 4 * 2 + R * 4 * 3 + T * cfg.P * 5 + T * 8 * 2,
    }
    return rows, index


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("row_kernels.hip", "device_common.h", "layout_kernels.hip"):
        with open(os.path.join(ROOT, "combine_moe_layout_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, calibrated on a copy of known size), or None
    when the kernels have changed since the counters were taken."""
    import re

    path = os.path.join(ROOT, "profiles", "traffic_qwen3_30b_a3b.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_hash: (\w+)$", text, re.M)
    if m is None or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"^traffic_bytes_per_launch\.%s: (\d+)$" % re.escape(kernel), text, re.M)
    return None if m is None else int(m.group(1))


class HipEvents:
    """Timing-only HIP events on torch's current stream, created with
    hipEventDisableSystemFence so that recording one does not write back and
    invalidate the caches (a default event's system-scope fence adds about
    3 us to the interval it brackets).  Uses the HIP runtime instance torch
    and the library already share in this process."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
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
        self._byref = ctypes.byref

    def record(self, i, stream):
        if self.L.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        if self.L.hipEventElapsedTime(self._byref(self._ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return self._ms.value

    def close(self):
        for e in self.ev:
            self.L.hipEventDestroy(e)
        self.ev = []


def cpu_baseline(cfg, budget_s):
    """The oracle, untuned, on a bounded sample: whole layers of the same shape."""
    import numpy as np

    import workloads as W
    from oracle import moe_oracle as O

    inp = W.layer_inputs(cfg, seed=0)
    dt = cfg.dtype
    w = inp.topk_weights
    rows, _ = layer_bytes(cfg)
    per_layer = sum(rows.values())
    n = 0
    t0 = time.perf_counter()
    while True:
        lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
        O.dispatch(lay, inp.x, dt, w)
        O.combine(lay, inp.y, dt, w)
        O.combine_bwd(lay, inp.g, dt, w, inp.y)
        O.dispatch_bwd(lay, inp.grad_recv, dt)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    return {
        "value": round(per_layer * n / el / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{n} full {cfg.name} layers (T={cfg.T}, H={cfg.H}, {dt}) fwd+bwd, "
                  f"numpy single-threaded, {el:.1f} s, {el / n * 1e3:.0f} ms/layer",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the exchange; --gpus {args.gpus} is not "
              "supported (this path has no collectives and runs on one GPU).", file=sys.stderr)
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

    def dev_rows(a):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    inp = W.layer_inputs(cfg, seed=0)
    idx0 = torch.from_numpy(inp.topk_idx).to(dev)
    w0 = torch.from_numpy(inp.topk_weights).to(dev)
    x0, y0, g0, gr0 = (dev_rows(a) for a in (inp.x, inp.y, inp.g, inp.grad_recv))
    del inp

    nsets = 1 if args.warm else max(1, args.sets)
    sets = []
    for _ in range(nsets):
        s = dict(idx=idx0.clone(), w=w0.clone(), x=x0.clone(), y=y0.clone(), g=g0.clone())
        if not args.warm:
            s["y_bwd"] = y0.clone()      # the backward's own copy of the expert output
            s["grad_recv"] = gr0.clone()
        s["recv"] = torch.empty((cfg.R, cfg.H), dtype=tdt, device=dev)
        s["scores"] = torch.empty(cfg.R, dtype=torch.float32, device=dev)
        s["out"] = torch.empty((cfg.T, cfg.H), dtype=tdt, device=dev)
        s["grad_y"] = torch.empty((cfg.R, cfg.H), dtype=tdt, device=dev)
        s["grad_w"] = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device=dev)
        s["grad_x"] = torch.empty((cfg.T, cfg.H), dtype=tdt, device=dev)
        s["ws"] = torch.empty(M.moe_workspace_size(cfg.T, cfg.K, cfg.E, cfg.P), dtype=torch.uint8, device=dev)
        s["h"] = M.Handle(args.chunks_per_lane, args.nontemporal, args.waves_per_block, args.layout_pairs)
        sets.append(s)
    del x0, y0, g0, gr0
    torch.cuda.synchronize()

    names = ["layout", "dispatch", "combine", "combine_bwd", "dispatch_bwd"]
    DOMINANT = "combine"  # the longest single kernel (a K-row gather-reduce)

    def step_call(s, ev=None, only=None):
        def mark(i):
            if ev is not None and (only is None or i in only):
                hev.record(ev + i, stream)
        mark(0)
        h = M.moe_layout(s["idx"], cfg.E, cfg.P, handle=s["h"], workspace=s["ws"])
        mark(1)
        M.moe_dispatch(h, s["x"], s["w"], recv=s["recv"], recv_scores=s["scores"])
        mark(2)
        y = s["recv"] if args.warm else s["y"]
        M.moe_combine(h, y, s["w"], out=s["out"])
        mark(3)
        yb = s["recv"] if args.warm else s["y_bwd"]
        M.moe_combine_bwd(h, s["g"], s["w"], yb, grad_y=s["grad_y"], grad_w=s["grad_w"])
        mark(4)
        gr = s["grad_y"] if args.warm else s["grad_recv"]
        M.moe_dispatch_bwd(h, gr, None, None, grad_x=s["grad_x"])
        mark(5)

    for i in range(args.warmup):
        step_call(sets[i % nsets])
    for s in sets:
        assert s["h"].check() == 0

    graphs = None
    if args.graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for s in sets:
                step_call(s)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(s)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()

    K = args.steps
    d = names.index(DOMINANT)
    only = None if args.events == "all" else ({d, d + 1} if args.events == "dominant" else set())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hev = HipEvents(6 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if graphs is not None:
            graphs[i % nsets].replay()
        else:
            step_call(sets[i % nsets], 6 * i, only)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    host_us = (t_enq - t0) * 1e6 / K

    # per-call event times (only the calls bracketed in the timed region)
    timed = [n for j, n in enumerate(names)
             if graphs is None and (only is None or (j in only and j + 1 in only))]
    call_ms = {n: [hev.elapsed_ms(6 * i + names.index(n), 6 * i + names.index(n) + 1) for i in range(K)]
               for n in timed}
    hev.close()
    avg_us = {n: float(np.mean(v)) * 1e3 for n, v in call_ms.items()}
    med_us = {n: float(np.median(v)) * 1e3 for n, v in call_ms.items()}

    # the copy kernel of known size, untimed: calibrates the traffic counters
    cbuf = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(cbuf)
    M.moe_bench_copy(cdst, cbuf)
    torch.cuda.synchronize()
    del cbuf, cdst

    rows, index = layer_bytes(cfg)
    step_bytes = sum(rows.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom = DOMINANT
    dom_us = avg_us.get(dom)
    achieved = None if dom_us is None else rows[dom] / (dom_us * 1e-6) / 1e9
    traffic = traffic_from_profiles(dom)

    line = {
        "metric": "dispatch+combine fwd+bwd GB/s per layer and % of MI355X HBM peak",
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
            "workload": f"{cfg.name}: T={cfg.T} H={cfg.H} {dt} E={cfg.E} P={cfg.P} K={cfg.K}, "
                        "layout+dispatch+combine+combine_bwd+dispatch_bwd per step",
            "cache": "warm (chained tensors)" if args.warm else f"cold ({nsets} rotating buffer sets)",
            "bytes_per_step": step_bytes,
            "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
            "us_per_layer": round(ms_per_step * 1e3, 2),
            "call_avg_us": {n: round(v, 2) for n, v in avg_us.items()},
            "call_median_us": {n: round(v, 2) for n, v in med_us.items()},
            "call_GBps": {n: round(rows[n] / (avg_us[n] * 1e-6) / 1e9, 1) for n in avg_us if rows[n]},
            "index_bytes_per_step": sum(index.values()),
            "host_enqueue_us_per_step": round(host_us, 1),
            "timing": ("hip graph replay" if graphs is not None else "eager launches") +
                      f", events: {args.events if graphs is None else 'none'}",
            "tuning": {"chunks_per_lane": args.chunks_per_lane, "nontemporal": args.nontemporal,
                       "waves_per_block": args.waves_per_block, "layout_pairs": args.layout_pairs},
        },
        "roofline": None if achieved is None else {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": rows[dom],
            "avg_launch_us": round(dom_us, 2),
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(cfg, args.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
