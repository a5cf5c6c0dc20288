#!/usr/bin/env python3
"""Benchmark of the AWQ per-layer hot path on one MI355X.

One step = the whole path on one linear group with its inputs resident in HBM:
activation statistics -> candidate scales -> grid search over alpha (20
points) -> selection -> INT4 quantize + pack of the winner.  The default
workload is a Qwen3-8B q_proj-shaped linear (W 4096 x 4096 fp16, X 4096
tokens x 4096 bf16, group size 128, weight-domain activation-weighted error).

Prints ONE JSON line.  `value` is weight-elements x grid-points per second of
the whole step, timed over K steps with nothing else on the stream; per-kernel
times come from a second pass over the same K steps in which the library
records HIP events around its main kernels on the stream they run on (an event
record costs microseconds of GPU timeline, so it stays out of the step time);
`roofline` describes the dominant kernel (traffic from committed counter runs,
null once its sources change); `cpu_baseline` times the CPU oracle on a
bounded sample.

Other workloads (--workload) measure the remaining rows: the output-score
search on the matrix cores (fused QKV, MLP with clip search) and the full
Qwen3-8B-shaped sweep of 144 linear groups.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scale-search weight-elems×grid-pts/s + pack GB/s; % of HBM roofline, 1 MI355X"
# MI355X published peaks and unit counts
HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
# fp32 vector: 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 lane-ops per clock x 2 flops
# (FMA) x 2.4 GHz, i.e. 78.6 T lane-operations/s; a SIMD issues up to two
# wave64 VALU instructions per 4 clocks when they come from different classes
VALU_LANE_OPS_PEAK_T = 256 * 4 * 32 * 2.4e9 / 1e12   # 78.64 T fp32 lane-ops/s
# fp32 lane operations that one element x candidate needs in the weight score:
# scale (mul), group max (max), v / step (mul by reciprocal), round (rndne),
# residual v - q*step (fma), square-accumulate (fma)
SEARCH_OPS_PER_ELEM_PT = 6
# the asymmetric grid adds a second running extremum (max(-v), half an op with
# the max3 pairing, plus the max of v no longer folding |.|) and the clamp of
# the code to [-z, 15 - z] (med3): 7
SEARCH_OPS_PER_ELEM_PT_ASYM = 7
# HBM bytes per launch of the dominant kernels, from `rocprofv3 --pmc FETCH_SIZE`
# and `--pmc WRITE_SIZE` runs of this script (commands and tables in
# profiles/search_weight_q_proj_4096x4096.md and
# profiles/gemm_sq_qkv_6144x4096_output.md): KiB per dispatch, scaled by what
# the same counters read for a plain copy of known size
# (profiles/copy_512MiB_calibration.md).  Each entry records the sha256 of the
# sources its kernel is built from; once those change, the counters describe
# another kernel and traffic is reported as null.
FETCH_CAL, WRITE_CAL = 2.0, 1.0
PMC_TRAFFIC = {
    ("search_weight_kernel", "q_proj_4096x4096"): {
        "fetch_kib": 16758.4, "write_kib": 640.0,
        "sources": ("csrc/search_weight.hip", "csrc/awq_device.h"),
        "sha256": "defe0c2e9940a8e54a9e9e972d928a3348712ea21d6d59d02dfc4e145d6bede3"},
    ("gemm_sq_kernel", "qkv_6144x4096_output"): {
        "fetch_kib": 11797680.2, "write_kib": 30720.0,
        "sources": ("csrc/output_score.hip", "csrc/awq_device.h"),
        "sha256": "694cb7a3b501509768c9ce468c13db421cf19ad44e50f1b2f92caf9c141469fb"},
}


def pmc_traffic(kernel: str, workload: str, args=None):
    """Calibrated HBM bytes per launch, or None (no counters for this kernel and
    workload, or sources changed since they were taken).  The counters were
    taken on the symmetric-grid instantiation; the asymmetric one has none."""
    if args is not None and getattr(args, "asym", False):
        return None
    e = PMC_TRAFFIC.get((kernel, workload))
    if e is None:
        return None
    h = hashlib.sha256()
    for rel in e["sources"]:
        with open(os.path.join(ROOT, "post_weight_quantization_awq_amd", rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != e["sha256"]:
        return None
    return 1024.0 * (FETCH_CAL * e["fetch_kib"] + WRITE_CAL * e["write_kib"])


class HipEvents:
    """Raw hipEvent_t pairs through the HIP runtime already loaded by torch."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(self.ev[b]) == 0
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def h(self, i: int) -> int:
        return self.ev[i].value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def pack_bytes(d_out: int, d_in: int, G: int) -> int:
    n = d_out * d_in
    return 2 * n + n // 2 + 2 * n // G + n // (2 * G) + 4 * d_in


def cpu_baseline_weight(W, X, G, budget_s: float, duo: bool = False, asym: bool = False):
    """Times the CPU oracle on the same group: statistics over all tokens, then
    search (20 points) + pack on consecutive row chunks until the time budget
    or the rows run out; the step time is scaled to all rows."""
    from oracle import awq_oracle as O
    d_out, d_in = W.shape
    t0, c0 = time.perf_counter(), time.process_time()
    xm = O.act_stats(X)
    t_stats = time.perf_counter() - t0
    done, t_rows, chunk = 0, 0.0, 256
    while done < d_out and t_stats + t_rows < budget_s:
        Wr = W[done:done + chunk]
        t1 = time.perf_counter()
        _, _, s = O.search_scales([Wr], xm, G, 20, duo=duo, asym=asym)
        if asym:
            O.quantize_pack_asym(Wr, s, G)
        else:
            O.quantize_pack(Wr, s, G)
        t_rows += time.perf_counter() - t1
        done += Wr.shape[0]
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    step_s = t_stats + t_rows * d_out / done
    return {
        "value": d_out * d_in * 20 / step_s,
        "unit": "weight-elem*grid-pt/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"act_stats over all {X.shape[0]} tokens, search (20 points) + pack of {done} of {d_out} "
                  f"rows, step time scaled to all rows ({wall:.1f} s wall)",
    }


def bench_weight(args, wl_name: str):
    import numpy as np
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS[wl_name]
    grp = wl.groups[0]
    G = args.group_size or wl.group_sizes[0]
    parts_h, X_h = WL.host_group_inputs(wl, 0, 0)
    W_h = np.concatenate(parts_h, axis=0)
    dev = torch.device("cuda:0")
    Ws = [torch.from_numpy(p).to(dev) for p in parts_h]
    if X_h.dtype == np.uint16:
        X = torch.from_numpy(X_h.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X = torch.from_numpy(X_h).to(dev)
    d_out, d_in, T = grp.d_out, grp.d_in, X.shape[0]
    n_w = d_out * d_in

    # preallocated outputs and workspaces: the timed step allocates nothing
    xm = torch.empty(d_in, dtype=torch.float32, device=dev)
    ws_stats = A.workspace(A.act_stats_workspace_bytes(T, d_in), dev)
    ws_search = A.workspace(A.search_workspace_bytes(d_out, d_in, 1, group_size=G, duo=args.duo, asym=args.asym),
                            dev)
    res = A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                         torch.empty(d_in, device=dev), None, None)
    packs = [(torch.empty((d_in, p.shape[0] // 8), dtype=torch.int32, device=dev),
              torch.empty((d_in // G, p.shape[0]), dtype=torch.float16, device=dev),
              torch.empty((d_in // G, p.shape[0] // 8), dtype=torch.int32, device=dev)) for p in Ws]
    K = args.steps
    ev = HipEvents(6 * K)

    stats_plan = A.ActStatsPlan(X, x_mean=xm, ws=ws_stats)
    search_plan = A.SearchPlan(Ws, xm, group_size=G, ws=ws_search, out=res, duo=args.duo, asym=args.asym)
    pack_plans = [A.PackPlan(p, G, res.best_s, out=o, asym=args.asym) for p, o in zip(Ws, packs)]

    def step(i: int = -1):
        if i >= 0:
            A.set_timing_events(ev.h(6 * i), ev.h(6 * i + 1))
        stats_plan.launch()
        if i >= 0:
            A.set_timing_events(ev.h(6 * i + 2), ev.h(6 * i + 3))
        search_plan.launch()
        if i >= 0:
            A.set_timing_events(ev.h(6 * i + 4), ev.h(6 * i + 5))
        for pp in pack_plans:
            pp.launch()
        if i >= 0:
            A.set_timing_events(None, None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # step time: K steps with nothing else on the stream (an event record
    # costs several microseconds of GPU timeline, which would be charged to
    # the method)
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    # kernel durations: the same K steps again, events around each kernel
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    k_ms = {"act_stats": 0.0, "search_weight": 0.0, "quantize_pack": 0.0}
    for i in range(K):
        k_ms["act_stats"] += ev.ms(6 * i, 6 * i + 1) / K
        k_ms["search_weight"] += ev.ms(6 * i + 2, 6 * i + 3) / K
        k_ms["quantize_pack"] += ev.ms(6 * i + 4, 6 * i + 5) / K
    ev.close()
    # unpack + dequantize (verification path, not part of the step): the first member's
    # packed output back to fp16 W, K calls between two events on torch's stream
    qw0, sc0, qz0 = packs[0]
    d0 = Ws[0].shape[0]
    w_back = torch.empty((d0, d_in), dtype=torch.float16, device=dev)
    unpack_args = (qw0.data_ptr(), sc0.data_ptr(), qz0.data_ptr(), d0, d_in, G, res.best_s.data_ptr(),
                   w_back.data_ptr(), A.AWQ_F16, torch.cuda.current_stream().cuda_stream)
    unpack_ms = []
    for a in (unpack_args, unpack_args[:6] + (None,) + unpack_args[7:]):  # W domain (/ s), scaled domain
        A._check(A.lib().awq_unpack_dequant(*a))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            A.lib().awq_unpack_dequant(*a)
        e1.record()
        torch.cuda.synchronize()
        unpack_ms.append(e0.elapsed_time(e1) / K)
    unpack_bytes = d0 * d_in // 2 + 2 * d0 * (d_in // G) + d0 * (d_in // G) // 2 + 4 * d_in + 2 * d0 * d_in

    elem_pts = n_w * 20
    t_search = k_ms["search_weight"] * 1e-3
    ops = SEARCH_OPS_PER_ELEM_PT_ASYM if args.asym else SEARCH_OPS_PER_ELEM_PT
    achieved_ops = ops * elem_pts / t_search / 1e12
    pk_bytes = sum(pack_bytes(p.shape[0], d_in, G) for p in Ws)
    out = {
        "metric": METRIC,
        "value": elem_pts / (ms_step * 1e-3),
        "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl_name, "d_out": d_out, "d_in": d_in, "tokens": T, "group_size": G,
                   "n_grid": 20, "score": "weight", "x_dtype": grp.x_dtype, "duo": args.duo,
                   "asym": args.asym},
        "search_elem_pts_per_s": elem_pts / t_search,
        "search_hbm_equiv_GBps": 2.0 * elem_pts / t_search / 1e9,
        "pack_GBps": pk_bytes / (k_ms["quantize_pack"] * 1e-3) / 1e9,
        "act_stats_GBps": (2 * T * d_in + 4 * d_in) / (k_ms["act_stats"] * 1e-3) / 1e9,
        "kernel_us": {k: v * 1e3 for k, v in k_ms.items()},
        "unpack_us": unpack_ms[0] * 1e3, "unpack_GBps": unpack_bytes / (unpack_ms[0] * 1e-3) / 1e9,
        "unpack_scaled_domain_us": unpack_ms[1] * 1e3,
        "roofline": {"bound": "alu", "achieved": achieved_ops, "peak": VALU_LANE_OPS_PEAK_T, "unit": "TOP/s",
                     "frac": achieved_ops / VALU_LANE_OPS_PEAK_T,
                     "traffic": pmc_traffic("search_weight_kernel", wl_name, args),
                     "kernel": "search_weight_kernel",
                     "ops_per_elem_pt": ops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_weight(W_h, X_h, G, args.cpu_seconds, args.duo, args.asym)
    return out


def bench_output(args, wl_name: str):
    import numpy as np
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS[wl_name]
    G = args.group_size or wl.group_sizes[0]
    dev = torch.device("cuda:0")
    groups = []
    for gi, grp in enumerate(wl.groups):
        parts = [WL.torch_weight(wl.seed(0, gi, 1 + 1000 * p), r, grp.d_in, dev) for p, r in enumerate(grp.parts)]
        if grp.x_from == "mlp_down":
            Xsrc = groups[gi - 1][1]
            X = WL.torch_down_input(Xsrc, groups[gi - 1][0][0], groups[gi - 1][0][1])
        else:
            X = WL.torch_activations(wl.seed(0, gi, 2), grp.T, grp.d_in, dev)
        groups.append((parts, X, grp))
    torch.cuda.synchronize()
    plans = []
    for parts, X, grp in groups:
        d_out = grp.d_out
        xm = torch.empty(grp.d_in, dtype=torch.float32, device=dev)
        ws_stats = A.workspace(A.act_stats_workspace_bytes(X.shape[0], grp.d_in), dev)
        ws = A.workspace(A.search_workspace_bytes(d_out, grp.d_in, X.shape[0], group_size=G, score="output",
                                                  n_clip=wl.n_clip, duo=args.duo, asym=args.asym), dev)
        res = A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                             torch.empty(grp.d_in, device=dev),
                             torch.empty(d_out, device=dev) if wl.n_clip else None, None)
        packs = [(torch.empty((grp.d_in, p.shape[0] // 8), dtype=torch.int32, device=dev),
                  torch.empty((grp.d_in // G, p.shape[0]), dtype=torch.float16, device=dev),
                  torch.empty((grp.d_in // G, p.shape[0] // 8), dtype=torch.int32, device=dev)) for p in parts]
        sp = A.ActStatsPlan(X, x_mean=xm, ws=ws_stats)
        qp = A.SearchPlan(parts, xm, group_size=G, score="output", X=X, n_clip=wl.n_clip, ws=ws, out=res,
                          duo=args.duo, asym=args.asym)
        pps, off = [], 0
        for p, o in zip(parts, packs):
            clip = res.clip[off:off + p.shape[0]] if res.clip is not None else None
            pps.append(A.PackPlan(p, G, res.best_s, clip, out=o, asym=args.asym))
            off += p.shape[0]
        plans.append((parts, X, grp, sp, qp, pps))
    K = args.steps
    n_pl = len(plans)
    ev = HipEvents(2 * n_pl * K)

    def step(k: int = -1):
        for i, (parts, X, grp, sp, qp, pps) in enumerate(plans):
            sp.launch()
            if k >= 0:
                A.set_timing_events(ev.h(2 * (k * n_pl + i)), ev.h(2 * (k * n_pl + i) + 1))
            qp.launch()
            if k >= 0:
                A.set_timing_events(None, None)
            for pp in pps:
                pp.launch()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / K
    for k in range(K):  # GEMM durations: same steps again with events around the GEMMs
        step(k)
    torch.cuda.synchronize()
    gemm_ms = [sum(ev.ms(2 * (k * n_pl + i), 2 * (k * n_pl + i) + 1) for k in range(K)) / K for i in range(n_pl)]
    ev.close()
    n_elem_pts = sum(g.d_out * g.d_in for _, _, g, *_ in plans) * 20
    flops_alpha = [2.0 * X.shape[0] * g.d_out * g.d_in * 20 for _, X, g, *_ in plans]
    # the events bracket the alpha-search GEMMs (with their dW builds when chunked)
    tflops = sum(flops_alpha) / (sum(gemm_ms) * 1e-3) / 1e12
    n_gemm = 20 + (wl.n_clip or 0)
    total_flops = sum(2.0 * X.shape[0] * g.d_out * g.d_in * n_gemm for _, X, g, *_ in plans)
    return {
        "metric": METRIC,
        "value": n_elem_pts / (ms_step * 1e-3),
        "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16-mfma/f32", "data": "synthetic",
        "config": {"workload": wl_name, "groups": [[g.name, g.d_out, g.d_in, X.shape[0]] for _, X, g, *_ in plans],
                   "group_size": G, "n_grid": 20, "score": "output", "n_clip": wl.n_clip, "duo": args.duo,
                   "asym": args.asym},
        "step_TFLOPs_algorithmic": total_flops / (ms_step * 1e-3) / 1e12,
        "gemm_ms": gemm_ms,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_FP16_PEAK_TFLOPS, "traffic": pmc_traffic("gemm_sq_kernel", wl_name, args),
                     "kernel": "gemm_sq_kernel"},
    }


def bench_sweep(args):
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS["qwen3_8b_sweep"]
    dev = torch.device("cuda:0")
    blocks = args.blocks
    # one calibration input per group kind (the 36 blocks share their statistics' shape)
    Xs = [WL.torch_activations(wl.seed(0, gi, 2), g.T, g.d_in, dev) for gi, g in enumerate(wl.groups)]
    Ws = []
    for b in range(blocks):
        Ws.append([[WL.torch_weight(wl.seed(b, gi, 1 + 1000 * p), r, g.d_in, dev) for p, r in enumerate(g.parts)]
                   for gi, g in enumerate(wl.groups)])
    torch.cuda.synchronize()
    out_all = {}
    for G in wl.group_sizes:
        xms = [torch.empty(g.d_in, device=dev) for g in wl.groups]
        ws_stats = [A.workspace(A.act_stats_workspace_bytes(g.T, g.d_in), dev) for g in wl.groups]
        ws = [A.workspace(A.search_workspace_bytes(g.d_out, g.d_in, 1, group_size=G, duo=args.duo, asym=args.asym), dev)
              for g in wl.groups]
        res = [A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                              torch.empty(g.d_in, device=dev), None, None) for g in wl.groups]
        packs = [[(torch.empty((g.d_in, r // 8), dtype=torch.int32, device=dev),
                   torch.empty((g.d_in // G, r), dtype=torch.float16, device=dev),
                   torch.empty((g.d_in // G, r // 8), dtype=torch.int32, device=dev)) for r in g.parts]
                 for g in wl.groups]
        K = args.steps
        per = 6 * 4 * blocks
        ev = HipEvents(per * K)
        ng = len(wl.groups)
        # The groups of a block are independent chains (own statistics, search and
        # packing; own workspaces and outputs): the timed steps put each group
        # kind on a stream of its own, joined to the main stream at both ends.
        # Kernel durations come from the same steps on the main stream alone.
        main = torch.cuda.current_stream()
        streams = [torch.cuda.Stream() for _ in range(args.streams)]

        def plans(stream_of):
            st = [A.ActStatsPlan(Xs[gi], x_mean=xms[gi], ws=ws_stats[gi], stream=stream_of(gi)) for gi in range(ng)]
            se = [[A.SearchPlan(Ws[b][gi], xms[gi], group_size=G, ws=ws[gi], out=res[gi], stream=stream_of(gi),
                                 duo=args.duo, asym=args.asym)
                   for gi in range(ng)] for b in range(blocks)]
            pk = [[[A.PackPlan(p, G, res[gi].best_s, out=o, stream=stream_of(gi), asym=args.asym)
                    for p, o in zip(Ws[b][gi], packs[gi])]
                   for gi in range(ng)] for b in range(blocks)]
            return st, se, pk

        par = plans(lambda gi: streams[gi % len(streams)])
        ser = plans(lambda gi: main)

        def step(pl, k=-1):
            st_plans, se_plans, pk_plans = pl
            n = k * per
            for b in range(blocks):
                for gi in range(ng):
                    if k >= 0:
                        A.set_timing_events(ev.h(n), ev.h(n + 1))
                    st_plans[gi].launch()
                    if k >= 0:
                        A.set_timing_events(ev.h(n + 2), ev.h(n + 3))
                    se_plans[b][gi].launch()
                    if k >= 0:
                        A.set_timing_events(ev.h(n + 4), ev.h(n + 5))
                    for pp in pk_plans[b][gi]:
                        pp.launch()
                    n += 6
            if k >= 0:
                A.set_timing_events(None, None)

        def step_streams():
            start = torch.cuda.Event()
            start.record(main)
            for s_ in streams:
                s_.wait_event(start)
            step(par)
            for s_ in streams:
                done = torch.cuda.Event()
                done.record(s_)
                main.wait_event(done)

        for _ in range(args.warmup):
            step_streams()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(K):
            step_streams()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t1) * 1e3 / K
        for k in range(K):  # kernel durations: same steps again, one stream, events around each kernel
            step(ser, k)
        torch.cuda.synchronize()
        sums = [0.0, 0.0, 0.0]
        for n in range(0, per * K, 6):
            sums[0] += ev.ms(n, n + 1)
            sums[1] += ev.ms(n + 2, n + 3)
            sums[2] += ev.ms(n + 4, n + 5)
        ev.close()
        sums = [s / args.steps for s in sums]
        n_w = blocks * sum(g.d_out * g.d_in for g in wl.groups)
        pk = blocks * sum(pack_bytes(r, g.d_in, G) for g in wl.groups for r in g.parts)
        xb = blocks * sum(2 * g.T * g.d_in for g in wl.groups)
        out_all[f"G{G}"] = {
            "ms_per_step": ms_step, "elem_pts_per_s": n_w * 20 / (ms_step * 1e-3),
            "search_ms": sums[1], "search_elem_pts_per_s": n_w * 20 / (sums[1] * 1e-3),
            "search_hbm_equiv_GBps": 2.0 * n_w * 20 / (sums[1] * 1e-3) / 1e9,
            "search_alu_frac": (SEARCH_OPS_PER_ELEM_PT_ASYM if args.asym else SEARCH_OPS_PER_ELEM_PT)
            * n_w * 20 / (sums[1] * 1e-3) / 1e12 / VALU_LANE_OPS_PEAK_T,
            "pack_ms": sums[2], "pack_GBps": pk / (sums[2] * 1e-3) / 1e9,
            "act_stats_ms": sums[0], "act_stats_GBps": xb / (sums[0] * 1e-3) / 1e9,
        }
    n_w = blocks * sum(g.d_out * g.d_in for g in wl.groups)
    first = out_all[f"G{wl.group_sizes[0]}"]
    return {
        "metric": METRIC, "value": first["elem_pts_per_s"], "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": first["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_sweep", "blocks": blocks, "weights": n_w, "n_grid": 20,
                   "group_sizes": list(wl.group_sizes), "score": "weight", "streams": args.streams,
                   "duo": args.duo, "asym": args.asym},
        "per_group_size": out_all,
        "roofline": {"bound": "alu", "achieved": first["search_alu_frac"] * VALU_LANE_OPS_PEAK_T,
                     "peak": VALU_LANE_OPS_PEAK_T, "unit": "TOP/s", "frac": first["search_alu_frac"],
                     "traffic": None, "kernel": "search_weight_kernel"},
    }


def bench_export(args):
    """Norm-group export of the 36 blocks ("From-Scratch AWQ INT4 Quantization
    on Qwen3-8B", exporter steps 1-3): per block the statistics of the two
    norm groups' inputs, per-linear weight-score searches of q/k/v and
    gate/up, the two norm folds (shared scale + folded norm), q/k/v and
    gate/up packed with their group's shared scale, o/down packed at RTN."""
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS["qwen3_8b_export"]
    dev = torch.device("cuda:0")
    blocks, G, K = args.blocks, wl.group_sizes[0], args.steps
    grp = wl.groups                      # qkv, o, gate_up, down
    NORMED, RTN = (0, 2), (1, 3)         # groups behind a norm / without one
    Xs = {gi: WL.torch_activations(wl.seed(0, gi, 2), grp[gi].T, grp[gi].d_in, dev) for gi in NORMED}
    Ws = [[[WL.torch_weight(wl.seed(b, gi, 1 + 1000 * p), r, g.d_in, dev) for p, r in enumerate(g.parts)]
           for gi, g in enumerate(grp)] for b in range(blocks)]
    norms = [{gi: WL.torch_norm(wl.seed(b, gi, 3), grp[gi].d_in, dev) for gi in NORMED} for b in range(blocks)]
    torch.cuda.synchronize()
    xms = {gi: torch.empty(grp[gi].d_in, device=dev) for gi in NORMED}
    ws_st = {gi: A.workspace(A.act_stats_workspace_bytes(grp[gi].T, grp[gi].d_in), dev) for gi in NORMED}
    members = [(gi, p) for gi in NORMED for p in range(len(grp[gi].parts))]
    ws_se = {m: A.workspace(A.search_workspace_bytes(grp[m[0]].parts[m[1]], grp[m[0]].d_in, 1, group_size=G), dev)
             for m in members}
    res = {m: A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                             torch.empty(grp[m[0]].d_in, device=dev), None, None) for m in members}
    s_sh = {gi: torch.empty(grp[gi].d_in, device=dev) for gi in NORMED}
    n_out = {gi: torch.empty(grp[gi].d_in, dtype=torch.float16, device=dev) for gi in NORMED}
    packs = {(gi, p): (torch.empty((g.d_in, r // 8), dtype=torch.int32, device=dev),
                       torch.empty((g.d_in // G, r), dtype=torch.float16, device=dev),
                       torch.empty((g.d_in // G, r // 8), dtype=torch.int32, device=dev))
             for gi, g in enumerate(grp) for p, r in enumerate(g.parts)}
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(args.streams)]
    chain_of = {0: 0, 2: 1, 1: 2, 3: 3}  # attention group, MLP group, o_proj, down_proj

    def plans(stream_of):
        """Per block, the calls in order, each tagged with its kernel kind."""
        st = {gi: A.ActStatsPlan(Xs[gi], x_mean=xms[gi], ws=ws_st[gi], stream=stream_of(chain_of[gi])) for gi in NORMED}
        out = []
        for b in range(blocks):
            calls = []
            for gi in NORMED:
                sp = stream_of(chain_of[gi])
                calls.append(("act_stats", st[gi]))
                for p in range(len(grp[gi].parts)):
                    calls.append(("search", A.SearchPlan([Ws[b][gi][p]], xms[gi], group_size=G, ws=ws_se[(gi, p)],
                                                         out=res[(gi, p)], stream=sp)))
                calls.append(("fold", A.FoldPlan([res[(gi, p)].best_s for p in range(len(grp[gi].parts))],
                                                 norms[b][gi], out=n_out[gi], s_shared=s_sh[gi], stream=sp)))
                for p in range(len(grp[gi].parts)):
                    calls.append(("pack", A.PackPlan(Ws[b][gi][p], G, s_sh[gi], out=packs[(gi, p)], stream=sp)))
            for gi in RTN:
                for p in range(len(grp[gi].parts)):
                    calls.append(("pack", A.PackPlan(Ws[b][gi][p], G, None, out=packs[(gi, p)],
                                                     stream=stream_of(chain_of[gi]))))
            out.append(calls)
        return out

    par = plans(lambda c: streams[c % len(streams)])
    ser = plans(lambda c: main)
    n_calls = sum(len(c) for c in ser)
    ev = HipEvents(2 * n_calls * K)

    def step(pl, k=-1):
        n, kinds = k * 2 * n_calls, []
        for calls in pl:
            for kind, c in calls:
                if k >= 0:
                    A.set_timing_events(ev.h(n), ev.h(n + 1))
                    kinds.append((kind, n))
                    n += 2
                c.launch()
        if k >= 0:
            A.set_timing_events(None, None)
        return kinds

    def step_streams():
        start = torch.cuda.Event()
        start.record(main)
        for s_ in streams:
            s_.wait_event(start)
        step(par)
        for s_ in streams:
            done = torch.cuda.Event()
            done.record(s_)
            main.wait_event(done)

    for _ in range(args.warmup):
        step_streams()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(K):
        step_streams()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / K
    tagged = []
    for k in range(K):  # kernel durations: the same steps on one stream, events around each call's main kernel
        tagged += step(ser, k)
    torch.cuda.synchronize()
    sums, counts = {}, {}
    for kind, n in tagged:
        sums[kind] = sums.get(kind, 0.0) + ev.ms(n, n + 1)
        counts[kind] = counts.get(kind, 0) + 1
    ev.close()
    per_step = {kk: v / K for kk, v in sums.items()}
    n_search = blocks * sum(grp[gi].d_out * grp[gi].d_in for gi in NORMED)
    n_all = blocks * sum(g.d_out * g.d_in for g in grp)
    pk = blocks * sum(pack_bytes(r, g.d_in, G) for g in grp for r in g.parts)
    frac = SEARCH_OPS_PER_ELEM_PT * n_search * 20 / (per_step["search"] * 1e-3) / 1e12 / VALU_LANE_OPS_PEAK_T
    return {
        "metric": METRIC, "value": n_search * 20 / (ms_step * 1e-3), "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_export", "blocks": blocks, "searched_weights": n_search,
                   "exported_weights": n_all, "n_grid": 20, "group_size": G, "score": "weight",
                   "streams": args.streams},
        "weights_exported_per_s": n_all / (ms_step * 1e-3),
        "kernel_ms_per_step": per_step,
        "fold_us_per_call": sums["fold"] / counts["fold"] * 1e3,
        "pack_GBps": pk / (per_step["pack"] * 1e-3) / 1e9,
        "roofline": {"bound": "alu", "achieved": frac * VALU_LANE_OPS_PEAK_T, "peak": VALU_LANE_OPS_PEAK_T,
                     "unit": "TOP/s", "frac": frac, "traffic": None, "kernel": "search_weight_kernel"},
    }


def cpu_baseline_w4a16(layers_h, M, budget_s: float):
    """Times the CPU oracle's W4A16 product on the first layers of the step
    (host copies of the same packed tensors) until the budget runs out; the
    rate is packed bytes per second."""
    from oracle import awq_oracle as O
    t0, c0 = time.perf_counter(), time.process_time()
    done_b, done_l = 0, 0
    for qw, sc, qz, x, d_out, G in layers_h:
        O.w4a16_matmul(x, qw, sc, qz, d_out, G)
        done_b += O.w4a16_bytes(d_out, qw.shape[0], G)
        done_l += 1
        if time.perf_counter() - t0 > budget_s:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return {"value": done_b / wall / 1e9, "unit": "GB/s", "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"{done_l} layers of the step at M = {M} ({done_b / 1e9:.2f} GB of packed weights, "
                      f"{wall:.1f} s wall)"}


def bench_w4a16(args):
    import numpy as np
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS["qwen3_8b_decode_w4a16"]
    G = args.group_size or wl.group_sizes[0]
    M = args.tokens
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed_base)
    lo, hi = -2 ** 31, 2 ** 31 - 1
    layers = []
    for b in range(args.blocks):
        for g in wl.groups:
            d_out, d_in = g.d_out, g.d_in
            qw = torch.randint(lo, hi, (d_in, d_out // 8), dtype=torch.int32, device=dev, generator=gen)
            sc = (torch.rand((d_in // G, d_out), device=dev, generator=gen) * 0.028 + 0.002).half()
            qz = torch.randint(lo, hi, (d_in // G, d_out // 8), dtype=torch.int32, device=dev, generator=gen)
            x = torch.randn((M, d_in), device=dev, generator=gen).half()
            y = torch.empty((M, d_out), dtype=torch.float16, device=dev)
            layers.append((qw, sc, qz, x, y, d_out, d_in))
    n, ws_bytes = ctypes.c_size_t(), 0
    for g in wl.groups:   # one workspace for every call of the step (stream-ordered)
        A.lib().awq_w4a16_workspace(M, g.d_out, g.d_in, ctypes.byref(n))
        ws_bytes = max(ws_bytes, n.value)
    ws = A.workspace(ws_bytes, dev)
    # a decode step is a fixed sequence of launches: captured once as a HIP
    # graph (default-priority side stream) and replayed, as a serving loop does
    s = torch.cuda.Stream()
    plans = [A.W4A16Plan(x, qw, sc, qz, d_out, G, out=y, ws=ws, stream=s)
             for qw, sc, qz, x, y, d_out, d_in in layers]
    # fp16 reference: the same shapes through torch's fp16 linear (hipBLASLt)
    w16 = [torch.randn((d_out, d_in), device=dev, generator=gen).half() * 0.02
           for qw, sc, qz, x, y, d_out, d_in in layers]
    y16 = [torch.empty((M, d_out), dtype=torch.float16, device=dev) for *_, d_out, d_in in layers]
    torch.cuda.synchronize()
    K = args.steps

    def step():
        for p in plans:
            p.launch()

    def step16():
        for (qw, sc, qz, x, y, d_out, d_in), w, o in zip(layers, w16, y16):
            torch.mm(x, w.t(), out=o)

    def timed(fn):
        s.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fn()
        s.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            step()
            step16()
        ms_eager = timed(step)
        ms16_eager = timed(step16)
        ref_y = [y.clone() for *_, y, d_out, d_in in layers[:8]]
        g, g16 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        with torch.cuda.graph(g16, stream=s):
            step16()
        for _ in range(args.warmup):
            g.replay()
            g16.replay()
        ms = timed(g.replay)
        ms16 = timed(g16.replay)
        s.synchronize()
        for r, (*_, y, d_out, d_in) in zip(ref_y, layers[:8]):   # replays reproduce the eager results
            if not torch.equal(r, y):
                raise RuntimeError("graph replay differs from the eager W4A16 result")
    # per-call durations (the GEMV and its reduction) with events on the call's stream
    n_l = len(plans)
    ev = HipEvents(2 * n_l * K)
    with torch.cuda.stream(s):
        for k in range(K):
            for i, p in enumerate(plans):
                A.set_timing_events(ev.h(2 * (k * n_l + i)), ev.h(2 * (k * n_l + i) + 1))
                p.launch()
            A.set_timing_events(None, None)
    s.synchronize()
    call_ms = [sum(ev.ms(2 * (k * n_l + i), 2 * (k * n_l + i) + 1) for k in range(K)) / K for i in range(n_l)]
    ev.close()

    def alg_bytes(d_out, d_in):
        return d_out * d_in // 2 + 2 * d_out * (d_in // G) + d_out * (d_in // G) // 2 + 2 * M * (d_in + d_out)

    tot_b = sum(alg_bytes(d_out, d_in) for *_, d_out, d_in in layers)
    achieved = tot_b / (sum(call_ms) * 1e-3) / 1e9
    # 9 tokens or more run the matrix-core GEMM: quoted against the fp16 MFMA peak
    gemm = M >= 9
    tflops = 2.0 * M * sum(d_out * d_in for *_, d_out, d_in in layers) / (sum(call_ms) * 1e-3) / 1e12
    kinds = {}
    for (qw, sc, qz, x, y, d_out, d_in), t in zip(layers, call_ms):
        key = f"{d_out}x{d_in}"
        kb = kinds.setdefault(key, [0.0, 0.0, 0])
        kb[0] += t
        kb[1] += alg_bytes(d_out, d_in)
        kb[2] += 1
    out = {
        "metric": "W4A16 decode through packed linears: weight bytes/s", "value": tot_b / (ms * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16-in/u4-w/f32-acc",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_decode_w4a16", "blocks": args.blocks, "tokens": M, "group_size": G,
                   "linears_per_block": [f"{g.d_out}x{g.d_in}" for g in wl.groups]},
        "fp16_ms_per_step": ms16, "speedup_vs_fp16": ms16 / ms,
        "eager_ms_per_step": ms_eager, "fp16_eager_ms_per_step": ms16_eager,
        "per_shape_GBps": {k: v[1] / (v[0] * 1e-3) / 1e9 for k, v in kinds.items()},
        "per_shape_us": {k: 1e3 * v[0] / v[2] for k, v in kinds.items()},
        "roofline": ({"bound": "mfma", "achieved": tflops, "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": tflops / MFMA_FP16_PEAK_TFLOPS, "traffic": None,
                      "kernel": "w4a16_gemm_kernel (+ w4a16_reduce_kernel where K is split, per call)"}
                     if gemm else
                     {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                      "kernel": "w4a16_gemv_kernel + w4a16_reduce_kernel (per call)"}),
        "step_TFLOPs": 2.0 * M * sum(d_out * d_in for *_, d_out, d_in in layers) / (ms * 1e-3) / 1e12,
        "fp16_step_TFLOPs": 2.0 * M * sum(d_out * d_in for *_, d_out, d_in in layers) / (ms16 * 1e-3) / 1e12,
    }
    if not args.no_cpu_baseline:
        hl = []
        for qw, sc, qz, x, y, d_out, d_in in layers[:8]:
            hl.append((qw.cpu().numpy().view(np.uint32), sc.cpu().numpy(), qz.cpu().numpy().view(np.uint32),
                       x.cpu().numpy(), d_out, G))
        out["cpu_baseline"] = cpu_baseline_w4a16(hl, M, min(args.cpu_seconds, 20.0))
    return out


def bench_copy(args):
    """Plain device copy of 512 MiB (torch), the calibration of the HBM byte counters."""
    import torch
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"metric": "device copy bandwidth (counter calibration)", "value": 2 * n / (ms * 1e-3) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": "copy_512MiB", "bytes_read": n, "bytes_written": n}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q_proj_4096x4096",
                    choices=["single_linear_256x512", "q_proj_4096x4096", "qkv_6144x4096_output",
                             "mlp_output_clip", "qwen3_8b_sweep", "qwen3_8b_export", "qwen3_8b_decode_w4a16",
                             "copy_512MiB"])
    ap.add_argument("--group-size", type=int, default=None)
    ap.add_argument("--blocks", type=int, default=36, help="blocks of the sweep workload")
    ap.add_argument("--streams", type=int, default=4,
                    help="streams the sweep's group kinds are spread over in the timed steps")
    ap.add_argument("--duo", action="store_true",
                    help="duo-scaling candidates (x_mean^r / (w_mean^(1-r) + 1e-4)) in the search workloads")
    ap.add_argument("--asym", action="store_true",
                    help="asymmetric INT4 (zero point per group) in the search and pack of the search workloads")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per decode step of the W4A16 workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the AWQ search and pack run per linear group on a single device; "
              "run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from post_weight_quantization_awq_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from post_weight_quantization_awq_amd import build
        build.build()
    torch.cuda.set_device(0)
    if args.workload in ("single_linear_256x512", "q_proj_4096x4096"):
        out = bench_weight(args, args.workload)
    elif args.workload == "qwen3_8b_sweep":
        out = bench_sweep(args)
    elif args.workload == "qwen3_8b_export":
        out = bench_export(args)
    elif args.workload == "qwen3_8b_decode_w4a16":
        out = bench_w4a16(args)
    elif args.workload == "copy_512MiB":
        out = bench_copy(args)
    else:
        out = bench_output(args, args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
