#!/usr/bin/env python3
"""Benchmark of the AWQ per-layer hot path on one MI355X.

One step = the whole path on every linear group of the workload, inputs
resident in HBM: activation statistics -> candidate scales -> grid search over
alpha (20 points) -> selection -> INT4 quantize + pack of the winner.  The
default workload is the full Qwen3-8B-shaped sweep: 36 blocks x 4
input-sharing groups (QKV 6144 x 4096, o 4096 x 4096, gate/up 24576 x 4096,
down 4096 x 12288; 6.95 G fp16 weights), every group with its own calibration
input of 65536 bf16 tokens, weight-domain activation-weighted error, group
size 128 (the line also reports group size 64).

Prints ONE JSON line.  `value` is weight-elements x grid-points per second of
the whole step, timed over K steps with nothing else on the streams; per-kernel
times come from a second pass over the same K steps in which the library
records HIP events around its main kernels on the stream they run on (an event
record costs microseconds of GPU timeline, so it stays out of the step time);
`roofline` describes the dominant kernel (traffic from committed counter runs,
null once its sources change); `cpu_baseline` times the CPU oracle on a
bounded sample over the host's cores.

Other workloads (--workload) measure the remaining rows: a single q_proj-shaped
linear, the output-score search on the matrix cores (fused QKV, MLP with clip
search), the norm-group export and the W4A16 product on the packed layout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scale-search weight-elems×grid-pts/s + pack GB/s; % of HBM roofline, 1 MI355X"
# MI355X published peaks and unit counts
HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
# fp32 vector: 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 lane-ops per clock x 2 flops
# (FMA) x 2.4 GHz, i.e. 78.6 T lane-operations/s: one wave64 instruction of the
# full-rate class (fma, mul, add) per 2 clocks per SIMD, no dual issue
VALU_LANE_OPS_PEAK_T = 256 * 4 * 32 * 2.4e9 / 1e12   # 78.64 T fp32 lane-ops/s
# The same class as measured on the machine by the issue-rate probe
# (`--workload valu_issue_probe`: v_fma / v_mul / v_add at 8 waves per SIMD,
# one wave64 instruction per 2 clocks at the ~2.1 GHz the chip holds under it)
VALU_LANE_OPS_MEASURED_T = 68.4
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
# profiles/gemm_gram_qkv_mlp_output.md): KiB per dispatch, scaled by what
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
    # the 36-block sweep at G = 128: mean over the 144 search launches of a step
    # (the four group shapes, 36 times each); profiles/sweep_qwen3_8b_36_blocks.md
    ("search_weight_kernel", "qwen3_8b_sweep"): {
        "fetch_kib": 47659.7, "write_kib": 1840.0,
        "sources": ("csrc/search_weight.hip", "csrc/awq_device.h"),
        "sha256": "defe0c2e9940a8e54a9e9e972d928a3348712ea21d6d59d02dfc4e145d6bede3"},
    # the fused QKV output score at 16384 tokens in either form: the
    # second-moment product (gemm_sq_kernel<1>, the default here) and the direct
    # GEMM (gemm_sq_kernel<0>, --out-form direct); profiles/gemm_gram_qkv_mlp_output.md
    ("gemm_sq_kernel<1>", "qkv_6144x4096_output"): {
        "fetch_kib": 1958292.6, "write_kib": 2880.0,
        "sources": ("csrc/output_score.hip", "csrc/awq_device.h"),
        "sha256": "533cb816d98cc45e5f4eda807c2acf4ed616753e493111d3ed9eaa027d8f3369"},
    ("gemm_sq_kernel<0>", "qkv_6144x4096_output"): {
        "fetch_kib": 11891109.2, "write_kib": 20640.0,
        "sources": ("csrc/output_score.hip", "csrc/awq_device.h"),
        "sha256": "533cb816d98cc45e5f4eda807c2acf4ed616753e493111d3ed9eaa027d8f3369"},
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

    def __init__(self, n: int, timing: bool = True):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if timing:
                assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            else:   # hipEventDisableTiming: a plain dependency marker
                assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), 2) == 0
            self.ev.append(e)

    def record(self, i: int, stream) -> None:
        assert self.hip.hipEventRecord(self.ev[i], stream.cuda_stream) == 0

    def wait(self, stream, i: int) -> None:
        """`stream` waits for event i (enqueued; the host does not wait)."""
        assert self.hip.hipStreamWaitEvent(stream.cuda_stream, self.ev[i], 0) == 0

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


class PowerSampler:
    """Socket power and shader clock while the timed steps run (``--power``):
    a thread calls ``amd-smi metric --clock --power`` back to back (about one
    sample per 0.1 s) between start() and stop(); stop() returns the means, or
    None when the option is off or amd-smi is not there.  Use enough steps for
    the timed region to hold a few tens of samples."""

    def __init__(self, enabled: bool, device: int = 0):
        self.cmd = ["amd-smi", "metric", "-g", str(device), "--clock", "--power"]
        self.enabled = enabled and shutil.which("amd-smi") is not None
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    @staticmethod
    def parse(text: str):
        watts, clocks, in_gfx = None, [], False
        for line in text.splitlines():
            f = line.strip()
            if f.startswith("SOCKET_POWER:"):
                try:
                    watts = float(f.split()[1])
                except (IndexError, ValueError):
                    pass
            elif re.fullmatch(r"GFX_\d+:", f):
                in_gfx = True
            elif f.startswith("CLK:") and in_gfx:
                try:
                    clocks.append(float(f.split()[1]))
                except (IndexError, ValueError):
                    pass
                in_gfx = False
            elif f.endswith(":"):
                in_gfx = False
        return (watts, sum(clocks) / len(clocks)) if watts is not None and clocks else None

    def _run(self):
        while not self._stop.is_set():
            try:
                r = subprocess.run(self.cmd, capture_output=True, text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            v = self.parse(r.stdout)
            if v is not None and not self._stop.is_set():
                self.samples.append(v)

    def start(self):
        if self.enabled:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        if not self.samples:
            return None
        n = len(self.samples)
        return {"socket_W": sum(w for w, _ in self.samples) / n, "gfx_MHz": sum(c for _, c in self.samples) / n,
                "gfx_MHz_min": min(c for _, c in self.samples), "samples": n,
                "source": " ".join(self.cmd) + ", sampled during the timed steps"}


def pack_bytes(d_out: int, d_in: int, G: int) -> int:
    n = d_out * d_in
    return 2 * n + n // 2 + 2 * n // G + n // (2 * G) + 4 * d_in


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_workers() -> int:
    """Worker processes for the oracle baseline: the host's CPU share (the
    OMP_NUM_THREADS the machine sets for a job, else every CPU this process
    may run on)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


# Oracle tasks for the worker pool (top-level so that spawned workers can run them).
def _oracle_stats_task(X):
    from oracle import awq_oracle as O
    return O.act_stats(X), X.shape[0]


def _oracle_search_task(W, S, xm, G, asym):
    """Candidate errors of a row chunk of a group (the group's candidate table S)."""
    import numpy as np
    from oracle import awq_oracle as O
    return np.array([O.weight_error(W, S[k], xm, G, asym=asym) for k in range(S.shape[0])])


def _oracle_pack_task(W, s, G, asym):
    from oracle import awq_oracle as O
    out = O.quantize_pack_asym(W, s, G) if asym else O.quantize_pack(W, s, G)
    return out[0].shape


def _noop_task(i):
    return i


class OraclePool:
    """The CPU oracle, unchanged, spread over a pool of worker processes: the
    activation statistics over token chunks, the search over row chunks (a
    group's candidate errors are sums over its rows, so the chunks' errors add
    up to the group's), and the packing over row chunks."""

    def __init__(self, n: int):
        import concurrent.futures as cf
        import multiprocessing as mp
        self.n = n
        # single-threaded numpy in every worker: the pool is the parallelism
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        try:
            self.ex = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))
            list(self.ex.map(_noop_task, range(4 * n)))     # start every worker before any timing
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def act_stats(self, X, chunk_rows: int):
        """x_mean of X from per-chunk means weighted by their token counts."""
        import numpy as np
        futs = [self.ex.submit(_oracle_stats_task, X[t:t + chunk_rows]) for t in range(0, X.shape[0], chunk_rows)]
        tot = np.zeros(X.shape[1], dtype=np.float64)
        for f in futs:
            m, t = f.result()
            tot += m.astype(np.float64) * t
        return (tot / X.shape[0]).astype(np.float32)

    def search(self, groups, G, duo=False, asym=False, chunk_rows=256):
        """groups: list of (W [d_out, d_in] fp16, x_mean).  Returns per group (errors, best index, best s)."""
        import numpy as np
        from oracle import awq_oracle as O
        tables = [O.candidate_scales(xm, 20, w_mean=O.weight_channel_mean([W]) if duo else None)
                  for W, xm in groups]
        futs = [[self.ex.submit(_oracle_search_task, W[r:r + chunk_rows], S, xm, G, asym)
                 for r in range(0, W.shape[0], chunk_rows)] for (W, xm), S in zip(groups, tables)]
        out = []
        for S, fs in zip(tables, futs):
            errs = np.zeros(S.shape[0], dtype=np.float64)
            for f in fs:
                errs += f.result()
            k = O.first_argmin(errs)
            out.append((errs, k, S[k]))
        return out

    def pack(self, jobs, G, asym=False, chunk_rows=256):
        """jobs: list of (W part, s)."""
        futs = [self.ex.submit(_oracle_pack_task, W[r:r + chunk_rows], s, G, asym)
                for W, s in jobs for r in range(0, W.shape[0], chunk_rows)]
        for f in futs:
            f.result()

    def close(self):
        self.ex.shutdown(wait=True)


def cpu_baseline_weight(W_parts, X, G, budget_s: float, duo: bool = False, asym: bool = False):
    """Times the CPU oracle on the same group on the host's cores: statistics
    over all tokens, then search (20 points) + pack of row chunks (the whole
    group when it fits the budget, else as many 256-row chunks as fit, the
    step time scaled to all rows)."""
    import numpy as np
    W = np.concatenate(W_parts, axis=0)
    d_out, d_in = W.shape
    pool = OraclePool(oracle_workers())
    try:
        t0 = time.perf_counter()
        xm = pool.act_stats(X, max(64, -(-X.shape[0] // pool.n)))
        t_stats = time.perf_counter() - t0
        # rows in rounds of one 256-row chunk per worker until the budget runs out
        done, t_rows, rnd = 0, 0.0, 256 * pool.n
        while done < d_out and t_stats + t_rows < budget_s:
            Wr = W[done:done + rnd]
            t1 = time.perf_counter()
            (errs, k, s), = pool.search([(Wr, xm)], G, duo, asym)
            pool.pack([(Wr, s)], G, asym)
            t_rows += time.perf_counter() - t1
            done += Wr.shape[0]
        wall = time.perf_counter() - t0
    finally:
        pool.close()
    step_s = t_stats + t_rows * d_out / done
    return {
        "value": d_out * d_in * 20 / step_s,
        "unit": "weight-elem*grid-pt/s",
        "cores": pool.n, "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"act_stats over all {X.shape[0]} tokens, search (20 points) + pack of {done} of {d_out} "
                  f"rows in 256-row chunks over {pool.n} worker processes, step time scaled to all rows "
                  f"({wall:.1f} s wall)",
    }


def cpu_baseline_sweep(host_blocks, T_full: int, G: int, budget_s: float, duo: bool = False, asym: bool = False,
                       n_blocks: int = 36):
    """Times the CPU oracle on blocks of the sweep (host copies of the same
    device tensors), on the host's cores, block after block until the budget
    runs out: statistics on a token sample of every group's input (scaled to
    all tokens), then the search of every group over all its rows and the
    packing of every part; the per-block time is scaled to all blocks.
    host_blocks: list over blocks of list over groups of (parts, X token sample)."""
    pool = OraclePool(oracle_workers())
    t_stats = t_search = t_pack = 0.0
    done, t_tok = 0, 0
    try:
        t0 = time.perf_counter()
        for groups in host_blocks:
            t1 = time.perf_counter()
            xms = [pool.act_stats(X, max(64, -(-X.shape[0] // pool.n))) for _, X in groups]
            t2 = time.perf_counter()
            res = pool.search([(__import__("numpy").concatenate(parts, axis=0), xm)
                               for (parts, _), xm in zip(groups, xms)], G, duo, asym)
            t3 = time.perf_counter()
            pool.pack([(p, s) for (parts, _), (_, _, s) in zip(groups, res) for p in parts], G, asym)
            t4 = time.perf_counter()
            t_stats += t2 - t1
            t_search += t3 - t2
            t_pack += t4 - t3
            t_tok = groups[0][1].shape[0]
            done += 1
            if t4 - t0 > budget_s:
                break
        wall = time.perf_counter() - t0
    finally:
        pool.close()
    per_block = t_stats * (T_full / t_tok) / done + (t_search + t_pack) / done
    n_w = sum(p.shape[0] * p.shape[1] for parts, _ in host_blocks[0] for p in parts)
    return {
        "value": n_blocks * n_w * 20 / (n_blocks * per_block),
        "unit": "weight-elem*grid-pt/s",
        "cores": pool.n, "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} of {n_blocks} blocks at G = {G}: act_stats on {t_tok} of {T_full} tokens per group "
                  f"(scaled to all tokens), search (20 points) of every group and pack of every part in 256-row "
                  f"chunks over {pool.n} worker processes; per-block time scaled to {n_blocks} blocks "
                  f"({wall:.1f} s wall: stats {t_stats:.1f}, search {t_search:.1f}, pack {t_pack:.1f})",
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
                     "frac": achieved_ops / VALU_LANE_OPS_PEAK_T, "measured_peak": VALU_LANE_OPS_MEASURED_T,
                     "frac_of_measured_peak": achieved_ops / VALU_LANE_OPS_MEASURED_T,
                     "traffic": pmc_traffic("search_weight_kernel", wl_name, args),
                     "kernel": "search_weight_kernel",
                     "ops_per_elem_pt": ops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_weight(parts_h, X_h, G, args.cpu_seconds, args.duo, args.asym)
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
                                                  n_clip=wl.n_clip, duo=args.duo, asym=args.asym,
                                                  out_form=args.out_form), dev)
        res = A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                             torch.empty(grp.d_in, device=dev),
                             torch.empty(d_out, device=dev) if wl.n_clip else None, None)
        packs = [(torch.empty((grp.d_in, p.shape[0] // 8), dtype=torch.int32, device=dev),
                  torch.empty((grp.d_in // G, p.shape[0]), dtype=torch.float16, device=dev),
                  torch.empty((grp.d_in // G, p.shape[0] // 8), dtype=torch.int32, device=dev)) for p in parts]
        sp = A.ActStatsPlan(X, x_mean=xm, ws=ws_stats)
        qp = A.SearchPlan(parts, xm, group_size=G, score="output", X=X, n_clip=wl.n_clip, ws=ws, out=res,
                          duo=args.duo, asym=args.asym, out_form=args.out_form)
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
    pw = PowerSampler(args.power)
    pw.start()
    t1 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / K
    power = pw.stop()
    for k in range(K):  # GEMM durations: same steps again with events around the GEMMs
        step(k)
    torch.cuda.synchronize()
    gemm_ms = [sum(ev.ms(2 * (k * n_pl + i), 2 * (k * n_pl + i) + 1) for k in range(K)) / K for i in range(n_pl)]
    ev.close()
    n_elem_pts = sum(g.d_out * g.d_in for _, _, g, *_ in plans) * 20
    # the form the library takes per group: "direct" contracts X with each
    # candidate's dW (2 T d_in flops per scored row); "gram" forms H = X^T X once
    # and scores each row against it, both on and right of H's diagonal
    # 384-blocks only (H is symmetric): 2 tri(d_in) flops per scored row and
    # 2 T tri(d_in) for H, tri(d) = sum over blocks I of rows(I) (d - 384 I)
    both = [A.search_output_forms(g.d_out, g.d_in, X.shape[0], group_size=G, n_clip=wl.n_clip, duo=args.duo,
                                  asym=args.asym, out_form=args.out_form) for _, X, g, *_ in plans]
    forms = [a for a, _ in both]
    clip_forms = [c for _, c in both]
    n_gemm = 20 + (wl.n_clip or 0)

    def tri(d):
        return float(sum(min(384, d - b) * (d - b) for b in range(0, d, 384)))

    def row_flops(X, g, form, parts=1):  # per scored output row (the clip search's H in `parts` fp16 parts)
        return 2.0 * (parts * tri(g.d_in) if form == "gram" else X.shape[0] * g.d_in)

    # the events bracket the alpha-search products (with their dW builds when chunked)
    flops_alpha = [row_flops(X, g, f) * g.d_out * 20 for (_, X, g, *_), f in zip(plans, forms)]
    tflops = sum(flops_alpha) / (sum(gemm_ms) * 1e-3) / 1e12
    n_clip = wl.n_clip or 0
    total_flops = sum(row_flops(X, g, f) * g.d_out * 20
                      + (row_flops(X, g, cf, 2) * g.d_out * n_clip if n_clip else 0.0)
                      + (2.0 * X.shape[0] * tri(g.d_in) if "gram" in (f, cf) else 0.0)
                      for (_, X, g, *_), f, cf in zip(plans, forms, clip_forms))
    direct_flops = sum(2.0 * X.shape[0] * g.d_out * g.d_in * n_gemm for _, X, g, *_ in plans)
    out = {
        "metric": METRIC,
        "value": n_elem_pts / (ms_step * 1e-3),
        "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16-mfma/f32", "data": "synthetic",
        "config": {"workload": wl_name, "groups": [[g.name, g.d_out, g.d_in, X.shape[0]] for _, X, g, *_ in plans],
                   "group_size": G, "n_grid": 20, "score": "output", "n_clip": wl.n_clip, "duo": args.duo,
                   "asym": args.asym, "out_form": args.out_form},
        "output_forms": forms, "clip_forms": clip_forms if wl.n_clip else None,
        "step_TFLOPs_performed": total_flops / (ms_step * 1e-3) / 1e12,
        "step_TFLOPs_direct_equivalent": direct_flops / (ms_step * 1e-3) / 1e12,
        "gemm_ms": gemm_ms,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_FP16_PEAK_TFLOPS,
                     "traffic": pmc_traffic("gemm_sq_kernel<%d>" % (forms[0] == "gram"), wl_name, args)
                     if len(set(forms)) == 1 else None,
                     "kernel": "gemm_sq_kernel<" + ",".join("1" if f == "gram" else "0" for f in forms) + ">"},
    }
    if power is not None:
        out["power"] = power
    return out


def _sweep_outputs(xmb, res_lane, packs_lane):
    """Copies of a step's outputs: x_mean of every block and group, and the
    search results and packed tensors held by one lane (its last block)."""
    return ([x.clone() for row in xmb for x in row],
            [t.clone() for r in res_lane for t in (r.err, r.best_idx, r.best_s)],
            [t.clone() for grp in packs_lane for o in grp for t in o])


def _same_outputs(a, b) -> bool:
    import torch
    return all(len(x) == len(y) and all(torch.equal(u, v) for u, v in zip(x, y)) for x, y in zip(a, b))


def bench_sweep(args):
    """The full Qwen3-8B-shaped sweep: 36 blocks x 4 input-sharing groups (QKV
    6144 x 4096, o 4096 x 4096, gate/up 24576 x 4096, down 4096 x 12288), each
    block with its own calibration input per group (65536 tokens, bf16), at
    G = 128 and then G = 64.  One step = per group: statistics, candidates,
    search, select, pack of every part."""
    import numpy as np
    import torch
    import post_weight_quantization_awq_amd as A
    import workloads as WL

    wl = WL.WORKLOADS["qwen3_8b_sweep"]
    dev = torch.device("cuda:0")
    blocks = args.blocks
    ng = len(wl.groups)
    # every block has its own weights and its own calibration inputs (108 GiB of
    # bf16 activations for 36 blocks, resident in HBM with the 13.9 GB of weights)
    Xs = [[WL.torch_activations(wl.seed(b, gi, 2), g.T, g.d_in, dev) for gi, g in enumerate(wl.groups)]
          for b in range(blocks)]
    Ws = [[[WL.torch_weight(wl.seed(b, gi, 1 + 1000 * p), r, g.d_in, dev) for p, r in enumerate(g.parts)]
           for gi, g in enumerate(wl.groups)] for b in range(blocks)]
    torch.cuda.synchronize()
    out_all = {}
    for G in wl.group_sizes:
        # one x_mean per block and group: the statistics of later blocks may be
        # taken while earlier blocks are still being searched
        xmb = [[torch.empty(g.d_in, device=dev) for g in wl.groups] for _ in range(blocks)]
        # workspaces and results per lane (a stream of the "blocks" schedule) and group kind
        n_lane = args.streams if args.schedule == "blocks" else (args.search_streams if args.schedule == "pipeline" else 1)
        ws_stats = [[A.workspace(A.act_stats_workspace_bytes(g.T, g.d_in), dev) for g in wl.groups]
                    for _ in range(n_lane)]
        ws = [[A.workspace(A.search_workspace_bytes(g.d_out, g.d_in, 1, group_size=G, duo=args.duo, asym=args.asym),
                           dev) for g in wl.groups] for _ in range(n_lane)]
        res = [[A.SearchResult(torch.empty(20, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                               torch.empty(g.d_in, device=dev), None, None) for g in wl.groups]
               for _ in range(n_lane)]
        packs = [[[(torch.empty((g.d_in, r // 8), dtype=torch.int32, device=dev),
                    torch.empty((g.d_in // G, r), dtype=torch.float16, device=dev),
                    torch.empty((g.d_in // G, r // 8), dtype=torch.int32, device=dev)) for r in g.parts]
                  for g in wl.groups] for _ in range(n_lane)]
        K = args.steps
        per = 6 * ng * blocks
        ev = HipEvents(per * K)
        # Schedules of the timed steps (kernel durations come from the same steps
        # on the main stream alone, events around each kernel).  The side
        # streams are forked from and joined to the main stream at both ends of
        # a step with HIP events:
        # * "pipeline": all statistics on one stream, running ahead; the
        #   searches (with select and pack) on two streams, alternating blocks,
        #   each waiting for its group's statistics through an event; the
        #   HBM-bound statistics of later groups stream while the VALU-bound
        #   searches of earlier ones compute;
        # * "blocks": block b's whole chain on stream b % streams;
        # * "groups": group kind g's chain on stream g % streams.
        main = torch.cuda.current_stream()
        n_side = 1 + args.search_streams if args.schedule == "pipeline" else args.streams
        streams = [torch.cuda.Stream() for _ in range(n_side)]
        # per-group readiness, fork, joins, per-block search completion
        sync = HipEvents(blocks * ng + n_side + 1 + blocks, timing=False)
        E_FORK = blocks * ng
        E_DONE = blocks * ng + n_side + 1

        def plans(stats_stream, work_stream, lane_of):
            st = [[A.ActStatsPlan(Xs[b][gi], x_mean=xmb[b][gi], ws=ws_stats[lane_of(b)][gi], stream=stats_stream(b, gi))
                   for gi in range(ng)] for b in range(blocks)]
            se = [[A.SearchPlan(Ws[b][gi], xmb[b][gi], group_size=G, ws=ws[lane_of(b)][gi], out=res[lane_of(b)][gi],
                                 stream=work_stream(b, gi), duo=args.duo, asym=args.asym)
                   for gi in range(ng)] for b in range(blocks)]
            pk = [[[A.PackPlan(p, G, res[lane_of(b)][gi].best_s, out=o, stream=work_stream(b, gi), asym=args.asym)
                    for p, o in zip(Ws[b][gi], packs[lane_of(b)][gi])]
                   for gi in range(ng)] for b in range(blocks)]
            return st, se, pk

        if args.schedule == "pipeline":
            ns = args.search_streams
            par = plans(lambda b, gi: streams[0], lambda b, gi: streams[1 + b % ns], lambda b: b % ns)
        elif args.schedule == "blocks":
            par = plans(lambda b, gi: streams[b % n_side], lambda b, gi: streams[b % n_side], lambda b: b % n_side)
        else:
            par = plans(lambda b, gi: streams[gi % n_side], lambda b, gi: streams[gi % n_side], lambda b: 0)
        ser = plans(lambda b, gi: main, lambda b, gi: main, lambda b: 0)

        def step(pl, k=-1):
            st_plans, se_plans, pk_plans = pl
            n = k * per
            for b in range(blocks):
                for gi in range(ng):
                    if k >= 0:
                        A.set_timing_events(ev.h(n), ev.h(n + 1))
                    st_plans[b][gi].launch()
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

        def fork():
            sync.record(E_FORK, main)
            for s_ in streams:
                sync.wait(s_, E_FORK)

        def join():
            for j, s_ in enumerate(streams):
                sync.record(E_FORK + 1 + j, s_)
                sync.wait(main, E_FORK + 1 + j)

        def step_pipeline():
            # The statistics of block b + D start once the searches of block
            # b - 1 are done, so they stream from HBM while the searches of
            # blocks b and b + 1 compute, instead of all running first.
            st_plans, se_plans, pk_plans = par
            D = max(1, args.lookahead)

            def stats(b):
                for gi in range(ng):
                    st_plans[b][gi].launch()
                    sync.record(b * ng + gi, streams[0])

            for b in range(min(D, blocks)):
                stats(b)
            for b in range(blocks):
                if b + D < blocks:
                    if b >= 1:
                        sync.wait(streams[0], E_DONE + b - 1)
                    stats(b + D)
                ws_ = streams[1 + b % args.search_streams]
                for gi in range(ng):
                    sync.wait(ws_, b * ng + gi)
                    se_plans[b][gi].launch()
                    for pp in pk_plans[b][gi]:
                        pp.launch()
                sync.record(E_DONE + b, ws_)

        def step_streams():
            fork()
            if args.schedule == "pipeline":
                step_pipeline()
            else:
                step(par)
            join()

        for _ in range(args.warmup):
            step_streams()
        torch.cuda.synchronize()
        pw = PowerSampler(args.power)
        pw.start()
        t1 = time.perf_counter()
        for _ in range(K):
            step_streams()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t1) * 1e3 / K
        power = pw.stop()
        # the multi-stream step must give exactly the one-stream results: every
        # block's statistics and the last block's search results and packed tensors
        last = blocks - 1
        lane_last = {"pipeline": last % args.search_streams, "blocks": last % n_side}.get(args.schedule, 0)
        snap = _sweep_outputs(xmb, res[lane_last], packs[lane_last])
        for k in range(K):  # kernel durations: same steps again, one stream, events around each kernel
            step(ser, k)
        torch.cuda.synchronize()
        if not _same_outputs(snap, _sweep_outputs(xmb, res[0], packs[0])):
            raise RuntimeError("the multi-stream sweep step differs from the one-stream step")
        sums = [0.0, 0.0, 0.0]
        for n in range(0, per * K, 6):
            sums[0] += ev.ms(n, n + 1)
            sums[1] += ev.ms(n + 2, n + 3)
            sums[2] += ev.ms(n + 4, n + 5)
        ev.close()
        sync.close()
        sums = [s / args.steps for s in sums]
        n_w = blocks * sum(g.d_out * g.d_in for g in wl.groups)
        pk = blocks * sum(pack_bytes(r, g.d_in, G) for g in wl.groups for r in g.parts)
        xb = blocks * sum(2 * g.T * g.d_in + 4 * g.d_in for g in wl.groups)
        ops = SEARCH_OPS_PER_ELEM_PT_ASYM if args.asym else SEARCH_OPS_PER_ELEM_PT
        out_all[f"G{G}"] = {
            "ms_per_step": ms_step, "elem_pts_per_s": n_w * 20 / (ms_step * 1e-3),
            "search_ms": sums[1], "search_elem_pts_per_s": n_w * 20 / (sums[1] * 1e-3),
            "search_hbm_equiv_GBps": 2.0 * n_w * 20 / (sums[1] * 1e-3) / 1e9,
            "search_alu_frac": ops * n_w * 20 / (sums[1] * 1e-3) / 1e12 / VALU_LANE_OPS_PEAK_T,
            "pack_ms": sums[2], "pack_GBps": pk / (sums[2] * 1e-3) / 1e9,
            "pack_hbm_frac": pk / (sums[2] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "act_stats_ms": sums[0], "act_stats_GBps": xb / (sums[0] * 1e-3) / 1e9,
            "act_stats_hbm_frac": xb / (sums[0] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        }
        if power is not None:
            out_all[f"G{G}"]["power"] = power
        del par, ser
    n_w = blocks * sum(g.d_out * g.d_in for g in wl.groups)
    G0 = wl.group_sizes[0]
    first = out_all[f"G{G0}"]
    ops = SEARCH_OPS_PER_ELEM_PT_ASYM if args.asym else SEARCH_OPS_PER_ELEM_PT
    wl_key = "qwen3_8b_sweep" if blocks == 36 else f"qwen3_8b_sweep_{blocks}_blocks"
    out = {
        "metric": METRIC, "value": first["elem_pts_per_s"], "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": first["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl_key, "blocks": blocks, "weights": n_w, "n_grid": 20,
                   "group_size": G0, "group_sizes": list(wl.group_sizes), "score": "weight",
                   "calibration_tokens_per_group": wl.groups[0].T, "x_per_block": True,
                   "x_dtype": "bf16", "schedule": args.schedule, "lookahead": args.lookahead,
                   "streams": 1 + args.search_streams if args.schedule == "pipeline" else args.streams,
                   "duo": args.duo, "asym": args.asym},
        "per_group_size": out_all,
        "streams_match_one_stream": True,
        "pack_GBps": first["pack_GBps"], "pack_hbm_frac": first["pack_hbm_frac"],
        "act_stats_GBps": first["act_stats_GBps"], "act_stats_hbm_frac": first["act_stats_hbm_frac"],
        "roofline": {"bound": "alu", "achieved": first["search_alu_frac"] * VALU_LANE_OPS_PEAK_T,
                     "peak": VALU_LANE_OPS_PEAK_T, "unit": "TOP/s", "frac": first["search_alu_frac"],
                     "measured_peak": VALU_LANE_OPS_MEASURED_T,
                     "frac_of_measured_peak": first["search_alu_frac"] * VALU_LANE_OPS_PEAK_T / VALU_LANE_OPS_MEASURED_T,
                     "traffic": pmc_traffic("search_weight_kernel", wl_key, args),
                     "kernel": "search_weight_kernel", "ops_per_elem_pt": ops,
                     "per": "achieved over all 144 launches of one step at G = %d; traffic per launch, "
                            "mean over the 144" % G0},
    }
    if not args.no_cpu_baseline:
        # host copies of the first blocks (weights, and a 4096-token sample of every group's input)
        n_cpu = min(blocks, args.cpu_blocks)
        T_s = min(4096, wl.groups[0].T)
        host_blocks = []
        for b in range(n_cpu):
            gs = []
            for gi in range(ng):
                parts = [w.cpu().numpy() for w in Ws[b][gi]]
                X = Xs[b][gi][:T_s].view(torch.int16).cpu().numpy().view(np.uint16)
                gs.append((parts, X))
            host_blocks.append(gs)
        del Xs, Ws
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline_sweep(host_blocks, wl.groups[0].T, G0, args.cpu_seconds, args.duo,
                                                 args.asym, n_blocks=blocks)
    return out


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
    pw = PowerSampler(args.power)
    pw.start()
    t1 = time.perf_counter()
    for _ in range(K):
        step_streams()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / K
    power = pw.stop()

    def outputs():  # the last block's export: packed tensors, folded norms, shared and searched scales
        return ([t.clone() for o in packs.values() for t in o], [t.clone() for t in n_out.values()],
                [t.clone() for t in s_sh.values()] + [t.clone() for r in res.values() for t in (r.err, r.best_s)])
    snap = outputs()
    tagged = []
    for k in range(K):  # kernel durations: the same steps on one stream, events around each call's main kernel
        tagged += step(ser, k)
    torch.cuda.synchronize()
    if not _same_outputs(snap, outputs()):
        raise RuntimeError("the multi-stream export step differs from the one-stream step")
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
    out = {
        "metric": METRIC, "value": n_search * 20 / (ms_step * 1e-3), "unit": "weight-elem*grid-pt/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_export", "blocks": blocks, "searched_weights": n_search,
                   "exported_weights": n_all, "n_grid": 20, "group_size": G, "score": "weight",
                   "streams": args.streams},
        "weights_exported_per_s": n_all / (ms_step * 1e-3),
        "streams_match_one_stream": True,
        "kernel_ms_per_step": per_step,
        "fold_us_per_call": sums["fold"] / counts["fold"] * 1e3,
        "pack_GBps": pk / (per_step["pack"] * 1e-3) / 1e9,
        "roofline": {"bound": "alu", "achieved": frac * VALU_LANE_OPS_PEAK_T, "peak": VALU_LANE_OPS_PEAK_T,
                     "unit": "TOP/s", "frac": frac, "measured_peak": VALU_LANE_OPS_MEASURED_T,
                     "frac_of_measured_peak": frac * VALU_LANE_OPS_PEAK_T / VALU_LANE_OPS_MEASURED_T,
                     "traffic": None, "kernel": "search_weight_kernel"},
    }
    if power is not None:
        out["power"] = power
    return out


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


def read_floor_per_call(sizes, K):
    """Per-call time (ms, HIP events around each eager launch, K rounds) of the
    read probe over a fresh buffer of each of `sizes` bytes (multiples of 16),
    launched in order on one stream: the floor of a kernel that reads those
    bytes once and does nothing else, timed like the W4A16 calls."""
    import torch
    from post_weight_quantization_awq_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        B.build_probe()
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.awq_probe_read_blocks.argtypes = [ctypes.c_int64]
    lib.awq_probe_read_blocks.restype = ctypes.c_int64
    lib.awq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_probe_read.restype = ctypes.c_int
    bufs = []
    for nb in sizes:
        b = torch.empty(nb, dtype=torch.uint8, device="cuda")
        b.fill_(0x5A)
        bufs.append(b)
    out = torch.zeros(int(max(lib.awq_probe_read_blocks(nb) for nb in sizes)), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    n = len(sizes)
    ev = HipEvents(2 * n * K)
    with torch.cuda.stream(s):
        for nb, b in zip(sizes, bufs):   # warm-up round
            assert lib.awq_probe_read(b.data_ptr(), nb, out.data_ptr(), s.cuda_stream) == 0
        for k in range(K):
            for i, (nb, b) in enumerate(zip(sizes, bufs)):
                ev.record(2 * (k * n + i), s)
                assert lib.awq_probe_read(b.data_ptr(), nb, out.data_ptr(), s.cuda_stream) == 0
                ev.record(2 * (k * n + i) + 1, s)
    s.synchronize()
    ms = [sum(ev.ms(2 * (k * n + i), 2 * (k * n + i) + 1) for k in range(K)) / K for i in range(n)]
    ev.close()
    del bufs
    return ms


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
    # 65 tokens or more run the matrix-core GEMM: quoted against the fp16 MFMA peak;
    # 2..64 tokens the few-token matrix-core path, which reads every packed word
    # once for all tokens and is quoted against HBM like the one-token GEMV
    gemm = M >= 65
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
                      "kernel": ("w4a16_gemv_kernel + w4a16_reduce_kernel (per call)" if M == 1 else
                                 "w4a16_skinny_kernel (+ w4a16_reduce_kernel where the inputs are split; per call)")}),
        "step_TFLOPs": 2.0 * M * sum(d_out * d_in for *_, d_out, d_in in layers) / (ms * 1e-3) / 1e12,
        "fp16_step_TFLOPs": 2.0 * M * sum(d_out * d_in for *_, d_out, d_in in layers) / (ms16 * 1e-3) / 1e12,
    }
    if not gemm:   # the same bytes read by a kernel that does nothing else, timed the same way
        sizes = [(d_out * d_in // 2 + 2 * d_out * (d_in // G) + d_out * (d_in // G) // 2 + 15) // 16 * 16
                 for *_, d_out, d_in in layers]
        fl = read_floor_per_call(sizes, K)
        floor = sum(sizes) / (sum(fl) * 1e-3) / 1e9
        out["read_floor"] = {"per_call_GBps": floor, "us_per_step": 1e3 * sum(fl),
                             "frac_of_floor": sum(fl) / sum(call_ms),   # floor time / W4A16 time
                             "kernel": "stream_read_kernel (probe library): one read of each linear's packed "
                                       "bytes per launch, HIP events around each call"}
    if not args.no_cpu_baseline:
        hl = []
        for qw, sc, qz, x, y, d_out, d_in in layers[:8]:
            hl.append((qw.cpu().numpy().view(np.uint32), sc.cpu().numpy(), qz.cpu().numpy().view(np.uint32),
                       x.cpu().numpy(), d_out, G))
        out["cpu_baseline"] = cpu_baseline_w4a16(hl, M, min(args.cpu_seconds, 20.0))
    return out


PROBE_KINDS = ["v_fma_f32", "v_mul_f32", "v_add_f32", "v_max3_f32", "v_rndne_f32", "v_fmac_f32",
               "v_cvt_f32_f16", "v_max_u32 (DPP row_half_mirror)", "v_fma_f32 + v_rndne_f32",
               "v_fma_f32 + v_mul_f32", "v_fma_f32 + v_max3_f32",
               "search element mix (mul, mul, max3, fma, fma, add, add, fma x4)",
               "v_fma_mix_f32 (fp16 a widened in the multiply)"]


def bench_valu_probe(args):
    """Issue rates (the probe library).  VALU by instruction class: for 1, 2, 3,
    4 and 8 waves per SIMD, wave64 instructions per second, as fp32 lane
    operations per second over the whole chip and as wave instructions per
    clock per SIMD at the published 2.4 GHz.  Matrix cores: 32x32x16 fp16
    products back to back on register operands, zero and random data."""
    import torch
    from post_weight_quantization_awq_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        B.build_probe()
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.awq_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_probe_valu.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4000
    s = torch.cuda.current_stream()
    res = {}
    best = 0.0
    for kind in range(lib.awq_probe_valu_kinds()):
        ipt = lib.awq_probe_valu_insts_per_trip(kind)
        row = {}
        for w in (1, 2, 3, 4, 8):
            blocks = n_cu * w                         # 4 waves per block: w waves per SIMD
            out = torch.empty(blocks * 256, device="cuda")
            for _ in range(2):
                assert lib.awq_probe_valu(kind, blocks, iters, out.data_ptr(), s.cuda_stream) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                assert lib.awq_probe_valu(kind, blocks, iters, out.data_ptr(), s.cuda_stream) == 0
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / args.steps
            wave_insts = blocks * 4 * iters * ipt
            lane_ops = wave_insts * 64 / t / 1e12
            row[f"{w}_waves_per_simd"] = {"lane_ops_T_per_s": lane_ops, "us": t * 1e6,
                                          "wave_insts_per_clk_per_simd_at_2.4GHz": wave_insts / t / (n_cu * 4 * 2.4e9)}
            best = max(best, lane_ops)
        res[PROBE_KINDS[kind]] = row
    # matrix cores: back-to-back 32x32x16 fp16 products on register operands,
    # 2 waves per SIMD, on all-zero and on random operands
    lib.awq_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.awq_probe_mfma.restype = ctypes.c_int
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    mfma = {}
    blocks, m_iters = n_cu * 2, 2000
    out = torch.empty(blocks * 256, device="cuda")
    for name, fill in (("zero operands", lambda n: torch.zeros(n, dtype=torch.float16, device="cuda")),
                       ("random operands N(0,1) fp16", lambda n: torch.randn(n, generator=g, device="cuda").half())):
        Ab, Bb = fill(4 * 64 * 8), fill(2 * 64 * 8)
        for _ in range(2):
            assert lib.awq_probe_mfma(blocks, m_iters, Ab.data_ptr(), Bb.data_ptr(), out.data_ptr(), s.cuda_stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            assert lib.awq_probe_mfma(blocks, m_iters, Ab.data_ptr(), Bb.data_ptr(), out.data_ptr(), s.cuda_stream) == 0
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / args.steps
        tf = blocks * 4 * m_iters * 8 * 2 * 32 * 32 * 16 / t / 1e12
        mfma[name] = {"TFLOP_per_s": tf, "frac_of_2500": tf / MFMA_FP16_PEAK_TFLOPS, "us": t * 1e6}
    return {"metric": "VALU issue rate (probe)", "value": best, "unit": "T fp32 lane-ops/s (best kind and occupancy)",
            "n_gpus": 1, "steps": args.steps, "warmup": 2, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "valu_issue_probe", "compute_units": n_cu, "iters": iters,
                       "chains_per_lane": 8, "threads_per_block": 256},
            "derived_peak_T": VALU_LANE_OPS_PEAK_T, "kinds": res,
            "mfma_f32_32x32x16_f16_2_waves_per_simd": mfma}


def bench_floor_probe(args):
    """Floors of the W4A16 decode step (the probe library).  For the packed
    linears of the 36 Qwen3-8B-shaped blocks, in the step's order: one launch of
    the read probe per linear over as many bytes as its codes, scales and zero
    points (a fresh buffer each, 3.6 GB in all, so nothing is served from a
    cache); the same followed by an empty one-block launch per linear (where a
    split's reduction would go); and empty launches of the read probe's grids.
    Each sequence is captured as a HIP graph and replayed like the W4A16 step;
    each read launch is also timed alone with HIP events around it."""
    import torch
    import workloads as WL
    from post_weight_quantization_awq_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        B.build_probe()
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.awq_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.awq_probe_empty.restype = ctypes.c_int
    lib.awq_probe_read_blocks.argtypes = [ctypes.c_int64]
    lib.awq_probe_read_blocks.restype = ctypes.c_int64
    lib.awq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_probe_read.restype = ctypes.c_int
    wl = WL.WORKLOADS["qwen3_8b_decode_w4a16"]
    G = args.group_size or wl.group_sizes[0]
    dev = torch.device("cuda:0")
    shapes = []
    for g in wl.groups:
        nb = g.d_out * g.d_in // 2 + 2 * g.d_out * (g.d_in // G) + g.d_out * (g.d_in // G) // 2
        shapes.append((f"{g.d_out}x{g.d_in}", (nb + 15) // 16 * 16))
    calls = []
    for b in range(args.blocks):
        for key, nb in shapes:
            buf = torch.empty(nb, dtype=torch.uint8, device=dev)
            buf.fill_(0x5A)
            calls.append((key, nb, buf))
    n_out = max(lib.awq_probe_read_blocks(nb) for _, nb, _ in calls)
    out = torch.zeros(n_out, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    K = args.steps

    def read(nb, buf):
        assert lib.awq_probe_read(buf.data_ptr(), nb, out.data_ptr(), s.cuda_stream) == 0

    def step_read():
        for _, nb, buf in calls:
            read(nb, buf)

    def step_read_empty():
        for _, nb, buf in calls:
            read(nb, buf)
            assert lib.awq_probe_empty(1, 256, s.cuda_stream) == 0

    def step_empty():
        for _, nb, _ in calls:
            assert lib.awq_probe_empty(int(lib.awq_probe_read_blocks(nb)), 256, s.cuda_stream) == 0

    def timed(fn):
        s.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fn()
        s.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    res = {}
    with torch.cuda.stream(s):
        for name, fn in (("read", step_read), ("read_then_empty", step_read_empty), ("empty", step_empty)):
            for _ in range(args.warmup):
                fn()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
            for _ in range(args.warmup):
                g.replay()
            res[name] = {"graph_ms_per_step": timed(g.replay), "eager_ms_per_step": timed(fn)}
    n = len(calls)

    def per_call(launch):
        ev = HipEvents(2 * n * K)
        with torch.cuda.stream(s):
            for k in range(K):
                for i, c in enumerate(calls):
                    ev.record(2 * (k * n + i), s)
                    launch(c)
                    ev.record(2 * (k * n + i) + 1, s)
        s.synchronize()
        ms_ = [sum(ev.ms(2 * (k * n + i), 2 * (k * n + i) + 1) for k in range(K)) / K for i in range(n)]
        ev.close()
        return ms_

    call_ms = per_call(lambda c: read(c[1], c[2]))
    kinds = {}
    for (key, nb, _), t in zip(calls, call_ms):
        kb = kinds.setdefault(key, [0.0, 0, 0])
        kb[0] += t
        kb[1] += nb
        kb[2] += 1
    tot = sum(nb for _, nb, _ in calls)
    # the few-token kernel's load pattern over each linear's codes, no arithmetic
    lib.awq_probe_strip_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_probe_strip_read.restype = ctypes.c_int
    lib.awq_probe_strip_read_blocks.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    lib.awq_probe_strip_read_blocks.restype = ctypes.c_int64
    dims = {f"{g.d_out}x{g.d_in}": (g.d_out, g.d_in) for g in wl.groups}
    strips = {}
    for wpl, spw in ((1, 4), (2, 4), (1, 8)):
        nb_out = max(lib.awq_probe_strip_read_blocks(dims[k][1], dims[k][0] // 8, wpl, spw) for k, _, _ in calls)
        o2 = torch.zeros(int(nb_out), dtype=torch.int32, device=dev)

        def sl(c, wpl=wpl, spw=spw, o2=o2):
            d_out, d_in = dims[c[0]]
            assert lib.awq_probe_strip_read(c[2].data_ptr(), d_in, d_out // 8, wpl, spw, o2.data_ptr(),
                                            s.cuda_stream) == 0
        with torch.cuda.stream(s):
            for c in calls:
                sl(c)
        ms_ = per_call(sl)
        kb = {}
        for c, t in zip(calls, ms_):
            e = kb.setdefault(c[0], [0.0, 0, 0])
            e[0] += t
            e[1] += dims[c[0]][0] * dims[c[0]][1] // 2
            e[2] += 1
        strips[f"{16 * wpl}_words_per_strip_{32 * spw}_rows_per_wave"] = {
            k: {"us": 1e3 * v[0] / v[2], "GBps": v[1] / (v[0] * 1e-3) / 1e9} for k, v in kb.items()}
    ms = res["read"]["graph_ms_per_step"]
    return {"metric": "W4A16 decode step floors (probe)", "value": tot / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "decode_floor_probe", "blocks": args.blocks, "group_size": G,
                       "launches_per_step": n, "bytes_per_step": tot},
            "steps_ms": res,
            "empty_launch_us_in_graph": 1e3 * res["empty"]["graph_ms_per_step"] / n,
            "second_launch_us_in_graph": 1e3 * (res["read_then_empty"]["graph_ms_per_step"] - ms) / n,
            "per_shape_us": {k: 1e3 * v[0] / v[2] for k, v in kinds.items()},
            "per_shape_GBps": {k: v[1] / (v[0] * 1e-3) / 1e9 for k, v in kinds.items()},
            "per_call_GBps": tot / (sum(call_ms) * 1e-3) / 1e9,
            "strip_reads_codes_only": strips}


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
    ap.add_argument("--workload", default="qwen3_8b_sweep",
                    choices=["single_linear_256x512", "q_proj_4096x4096", "qkv_6144x4096_output",
                             "mlp_output_clip", "qwen3_8b_sweep", "qwen3_8b_export", "qwen3_8b_decode_w4a16",
                             "copy_512MiB", "valu_issue_probe", "decode_floor_probe"])
    ap.add_argument("--group-size", type=int, default=None)
    ap.add_argument("--blocks", type=int, default=36, help="blocks of the sweep workload")
    ap.add_argument("--streams", type=int, default=8,
                    help="streams of the sweep's timed steps (--schedule blocks or groups)")
    ap.add_argument("--lookahead", type=int, default=2,
                    help="pipeline schedule: blocks whose statistics may run ahead of the searches")
    ap.add_argument("--search-streams", type=int, default=2,
                    help="pipeline schedule: streams the searches, selections and packs alternate over")
    ap.add_argument("--schedule", default="pipeline", choices=["pipeline", "blocks", "groups"],
                    help="sweep schedule: the statistics on a stream of their own running ahead of the searches "
                         "on two streams (pipeline), blocks round-robin over the streams (blocks), or one "
                         "stream per group kind (groups)")
    ap.add_argument("--out-form", choices=["auto", "direct", "gram"], default="auto",
                    help="output-score form: the library's choice, X times each candidate's dW, or the "
                         "second-moment form dW (X^T X) dW^T")
    ap.add_argument("--duo", action="store_true",
                    help="duo-scaling candidates (x_mean^r / (w_mean^(1-r) + 1e-4)) in the search workloads")
    ap.add_argument("--asym", action="store_true",
                    help="asymmetric INT4 (zero point per group) in the search and pack of the search workloads")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per decode step of the W4A16 workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power", action="store_true",
                    help="sample socket power and shader clock (amd-smi) during the timed steps of the sweep, "
                         "export and output-score workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the CPU oracle baseline")
    ap.add_argument("--cpu-blocks", type=int, default=4,
                    help="most sweep blocks the CPU oracle baseline runs (it stops earlier at --cpu-seconds)")
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
    elif args.workload == "valu_issue_probe":
        out = bench_valu_probe(args)
    elif args.workload == "decode_floor_probe":
        out = bench_floor_probe(args)
    else:
        out = bench_output(args, args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
