"""Benchmark of the CSA2 layer on one MI355X.

The default run measures the Flash-shape prefill layer (1 sequence of 4096
query tokens, m = 4 so 1024 records, indexer 32 x 128, Top-512, 64 heads x
512 latent with 64 rotary dims, window 128, bf16, float32 output) as
``value``.  The same run measures, each in its own object under
``workloads``: that prefill layer with a bf16 output; the decode workloads
(Full decode at 64K context, hierarchical Full/Reindex/Reuse decode at
256K, fp8 decode at 1M, heavily compressed (HCA) decode at 1M, the 1M
decode in the V4.1 cache formats (FP4 main KV, MXFP4 indexer, FP8
window), and a multi-query decode that verifies 5 positions per
sequence); and record construction (16 x 4096 token rows into FP4
records and MXFP4 keys).  ``--workload`` picks another primary workload;
``--only`` skips the others.

A step is one pass of the whole hot path over the workload's batch: for
every layer of its sharing group, indexer scores (Full / Reindex), block
pool (when the Full layer builds one), Top-K and sparse attention -- the
same entry points, in the same order, that csa2_layer enqueues.  HIP
events recorded on the launch stream bracket each call, so each kernel's
average duration over the timed steps is measured live; the dominant
kernel's roofline is reported from it.  Decode workloads are also timed as
one captured HIP graph per step (the same launches replayed without host
gaps).  Inputs are resident in HBM before timing, and decode steps rotate
two cache copies so that the caches are not served from the 256 MB MALL.

One JSON line is printed.  The fp64 CPU oracle is also timed on a bounded
sample of each workload (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clocks after some tens of milliseconds of
    # load: 50 steps (about 30 ms of C2) before the timed ones
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="C2", choices=["C1", "C2", "C3", "C4", "C5", "C6", "C7", "C8", "C9"])
    ap.add_argument("--only", action="store_true", help="measure the primary workload only")
    ap.add_argument("--extra", default="C2b,C3,C4,C5,C6,C7,C8,C9", help="further workloads measured in the same run")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated between steps (0: 2 for decode, 1 for prefill)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extra-cpu-seconds", type=float, default=8.0)
    return ap.parse_args()


# --------------------------------------------------------------- algorithmic work

def entries_per_query(wl, inp):
    """Selected records + window rows each query attends to (the method's
    required reads, independent of the GPU's kernels)."""
    q_pos = inp["layers"][0]["q_pos"]
    n_rec = np.full(wl.B, wl.N) if wl.n_rec is None else np.asarray(wl.n_rec)
    t = q_pos.astype(np.int64)
    vis = np.minimum(n_rec[:, None], (t + 1) // wl.m)
    sel = vis if wl.modes == ("hca",) else np.minimum(wl.K, vis)  # HCA attends to every visible record
    win = np.minimum(wl.W, t + 1)
    return sel, win, vis


def kernel_work(wl, inp, out_bf16=False):
    """Algorithmic bytes and flops per call of each step phase."""
    def row_bytes(n, dt):  # one stored row of n elements, with its scales
        return {"f32": 4 * n, "bf16": 2 * n, "e4m3": n + 4, "fp4": n // 2 + n // 16, "mxfp4": n // 2 + n // 32}[dt]
    kbytes = row_bytes(wl.Di, wl.k_dtype)
    rbytes = row_bytes(wl.D, wl.kv_dtype)
    wbytes = row_bytes(wl.D, wl.swa_dtype)
    qi_bytes = wl.Hi * row_bytes(wl.Di, wl.q_idx_dtype) + wl.Hi * 4
    q_bytes = wl.H * row_bytes(wl.D, wl.q_dtype)
    out_bytes = wl.H * wl.D * (2 if out_bf16 else 4)
    sel, win, vis = entries_per_query(wl, inp)
    rows = wl.B * wl.Tq
    work = {}
    # Full indexer: every visible record's key row once per sequence (decode)
    # or the key tile set once (prefill, keys are L2-resident and counted once
    # per sequence); per query its q_idx/w; flops 2*Hi*Di per visible pair.
    pairs = int(vis.sum())
    key_reads = int(vis.max(axis=1).sum()) if wl.Tq > 1 else pairs
    work["index_full"] = dict(bytes=key_reads * kbytes + rows * qi_bytes,
                              flops=2.0 * wl.Hi * wl.Di * pairs)
    if wl.P:
        cand = min(wl.P * wl.blk, wl.N)
        work["index_pool"] = dict(bytes=rows * (cand * kbytes + qi_bytes),
                                  flops=2.0 * wl.Hi * wl.Di * rows * cand)
    ent = int((sel + win).sum())
    # rows read: per sequence, the distinct records and local rows its queries
    # need (a decode query's own set; a prefill sequence's records and window
    # rows are shared by its tokens and read once)
    t_max = inp["layers"][0]["q_pos"].max(axis=1) + 1
    urec = np.minimum(vis.max(axis=1), sel.sum(axis=1))
    uwin = np.minimum(np.minimum(wl.S, t_max), win.sum(axis=1))
    work["attn"] = dict(bytes=int(urec.sum()) * rbytes + int(uwin.sum()) * wbytes + rows * (q_bytes + out_bytes),
                        flops=4.0 * wl.D * wl.H * ent)
    # Selection steps: their own inputs and outputs (scores are an
    # intermediate of the layer, but they are what these kernels stream).
    work["topk_full"] = dict(bytes=rows * (wl.N * 4 + wl.K * 4), flops=0.0)
    work["attn_dense"] = work["attn"]
    if wl.P:
        work["block_pool"] = dict(bytes=rows * (wl.N * 4 + wl.P * 4), flops=0.0)
        work["topk_pool"] = dict(bytes=rows * (wl.P * wl.blk * 4 + wl.P * 4 + wl.K * 4), flops=0.0)
    return work


# --------------------------------------------------------------- the timed step

class Step:
    """Enqueues the hot path of one workload through the ABI's entry points
    on one stream, optionally recording a HIP event between calls."""

    def __init__(self, grp, torch, stream=None):
        from sparse_long_context_csa2_amd import binding as Bd
        self.Bd, self.torch, self.grp = Bd, torch, grp
        self.stream = stream  # torch stream the calls are enqueued on (None: current)
        wl = grp.wl
        self.calls = []  # (name, fn(copy) -> prepared call)
        self.prepared = None
        dev = grp.device
        rows = wl.B * wl.Tq
        self.scores_full = torch.empty((wl.B, wl.Tq, wl.N), dtype=torch.float32, device=dev)
        self.scores_pool = None
        if wl.P:
            self.scores_pool = torch.empty((wl.B, wl.Tq, wl.P * wl.blk), dtype=torch.float32, device=dev)
        nbp = Bd.lib().csa2_block_pool_workspace_bytes(rows, wl.N, wl.blk) if wl.P else 0
        self.pool_ws = torch.empty(max(nbp, 256), dtype=torch.uint8, device=dev)
        ntk = max(Bd.lib().csa2_topk_workspace_bytes(rows, wl.N, wl.K),
                  Bd.lib().csa2_topk_workspace_bytes(rows, wl.P * wl.blk, wl.K) if wl.P else 0)
        self.topk_ws = torch.empty(max(ntk, 256), dtype=torch.uint8, device=dev)
        na = max(Bd.lib().csa2_sparse_attn_workspace_bytes(wl.B, wl.Tq, wl.H, wl.D, wl.K, wl.W),
                 Bd.lib().csa2_dense_attn_workspace_bytes(wl.B, wl.Tq, wl.H, wl.D, wl.N, wl.W))
        self.attn_ws = torch.empty(max(na, 256), dtype=torch.uint8, device=dev)
        for li, lay in enumerate(grp.layers):
            mode = lay["mode"]
            if mode == "full":
                self.calls.append(("index_full", self._index(lay, None)))
                if lay["build_pool"]:
                    self.calls.append(("block_pool", self._pool(lay)))
                self.calls.append(("topk_full", self._topk(lay, li, pooled=False)))
            elif mode == "reindex":
                self.calls.append(("index_pool", self._index(lay, grp.pool)))
                self.calls.append(("topk_pool", self._topk(lay, li, pooled=True)))
            if mode == "hca":
                self.calls.append(("attn_dense", self._dense(lay)))
            else:
                self.calls.append(("attn", self._attn(lay, li)))

    def _index(self, lay, pool):
        Bd, grp = self.Bd, self.grp

        def f(copy):
            sh = grp.shared[copy]
            out = self.scores_full if pool is None else self.scores_pool
            return Bd.csa2_index_scores(lay["q_idx"], lay["w"], sh["k_idx"], sh["k_scale"], lay["q_pos"], sh["m"],
                                        n_rec=sh["n_rec"], pool=pool, blk=lay["blk"] if pool is not None else 0,
                                        out=out, stream=self.stream, prepare=True, q_scale=lay["q_idx_scale"])
        return f

    def _pool(self, lay):
        def f(copy):
            return self.Bd.csa2_block_pool(self.scores_full, lay["blk"], lay["P"], out=self.grp.pool,
                                           ws=self.pool_ws, stream=self.stream, prepare=True)
        return f

    def _topk(self, lay, li, pooled):
        def f(copy):
            if pooled:
                return self.Bd.csa2_topk(self.scores_pool, lay["K"], pool=self.grp.pool, blk=lay["blk"],
                                         out=self.grp.idx[li], ws=self.topk_ws, stream=self.stream, prepare=True)
            return self.Bd.csa2_topk(self.scores_full, lay["K"], out=self.grp.idx[li], ws=self.topk_ws,
                                     stream=self.stream, prepare=True)
        return f

    def _attn(self, lay, li):
        def f(copy):
            sh = self.grp.shared[copy]
            return self.Bd.csa2_sparse_attn(lay["q"], sh["kv"], sh["kv_scale"], self.grp.idx[li], lay["swa"],
                                            lay["swa_scale"], lay["W"], lay["q_pos"], lay["sink"], lay["rope_dims"],
                                            lay["rope_base"], lay["sm_scale"], out=lay["out"], ws=self.attn_ws,
                                            stream=self.stream, prepare=True)
        return f

    def _dense(self, lay):
        def f(copy):
            sh = self.grp.shared[copy]
            return self.Bd.csa2_dense_attn(lay["q"], sh["kv"], sh["kv_scale"], lay["swa"], lay["swa_scale"],
                                           lay["W"], lay["q_pos"], lay["sink"], lay["rope_dims"], sh["m"],
                                           n_rec=sh["n_rec"], rope_base=lay["rope_base"],
                                           sm_scale=lay["sm_scale"], out=lay["out"], ws=self.attn_ws,
                                           stream=self.stream, prepare=True)
        return f

    def run(self, copy, events=None):
        # every call was prepared once per cache copy (arguments converted
        # up front), so the host keeps ahead of the GPU between launches
        if self.prepared is None:
            self.prepared = [[fn(c) for c in range(len(self.grp.shared))] for _, fn in self.calls]
        for i, calls in enumerate(self.prepared):
            if events is not None:
                events[i].record(self.stream)
            calls[copy]()
        if events is not None:
            events[len(self.calls)].record(self.stream)


# --------------------------------------------------------------- CPU baseline

def cpu_threads():
    """(host cores this process may run on, BLAS threads numpy uses)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        blas = 1
    return cores, blas


def cpu_baseline(inp, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of query rows of
    the same workload (spread over the batch and the sequence)."""
    import oracle as O
    cores, blas = cpu_threads()
    wl = inp["wl"]
    rows = [(b, t) for t in range(wl.Tq) for b in range(wl.B)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(rows))
    sh, lays = inp["shared"], inp["layers"]
    done = 0
    t0 = time.perf_counter()
    for k in order:
        b, ti = rows[k]
        O.group_query(sh, lays, b, ti)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 2), "unit": "query-tokens/s", "cores": min(cores, blas), "kind": "oracle",
            "affinity_cores": cores, "blas_threads": blas,
            "sample": f"{done} of {len(rows)} query rows of the same workload (random order), "
                      f"{len(lays)} layer(s) each, fp64 NumPy, {dt:.1f} s"}


def traffic_for(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    files = rec.get("source", [])
    files = [files] if isinstance(files, str) else files
    h = hashlib.sha256()
    for f in files:
        src = os.path.join(ROOT, "sparse_long_context_csa2_amd", "csrc", f)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if not files or h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


# --------------------------------------------------------------- one workload

# workload variants: (base workload, attention output dtype)
VARIANTS = {"C2b": ("C2", "bf16")}


def measure(key, steps, warmup, copies, cpu_seconds, torch, graph=False):
    """Times `steps` steps of workload `key` and returns its report."""
    from sparse_long_context_csa2_amd import runner as R
    from sparse_long_context_csa2_amd import workloads as WL

    base, odt = VARIANTS.get(key, (key, "f32"))
    wl = WL.CONFIGS[base]
    inp = WL.make_inputs(wl)
    decode = wl.decode_pos is not None
    copies = copies or (2 if decode else 1)
    grp = R.DeviceGroup(inp, device="cuda:0", copies=copies,
                        out_dtype=torch.bfloat16 if odt == "bf16" else torch.float32)
    stream = torch.cuda.Stream()
    step = Step(grp, torch, stream)
    ncalls = len(step.calls)

    for i in range(warmup):
        step.run(i % copies)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step.run(s % copies, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = {}
    for s in range(steps):
        for i, (name, _) in enumerate(step.calls):
            per_call.setdefault(name, []).append(evs[s][i].elapsed_time(evs[s][i + 1]) * 1e-3)
    step_s = [evs[s][0].elapsed_time(evs[s][ncalls]) * 1e-3 for s in range(steps)]
    ms_eager = 1e3 * float(np.mean(step_s))
    tokens = wl.B * wl.Tq

    ms_graph = None
    if graph:
        # one graph per cache copy, each replaying the whole step's launches
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step.run(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for s in range(steps):
                graphs[s % copies].replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / steps
        del graphs
    ms_per_step = ms_graph if ms_graph is not None else ms_eager
    value = tokens / (ms_per_step * 1e-3)

    work = kernel_work(wl, inp, out_bf16=odt == "bf16")
    kern = {}
    for name, ts in per_call.items():
        ntimes = sum(1 for n, _ in step.calls if n == name)
        avg = float(np.mean(ts))
        kern[name] = {"avg_us": round(avg * 1e6, 2), "calls_per_step": ntimes}
        if name in work:
            w = work[name]
            kern[name]["GB_s"] = round(w["bytes"] / avg / 1e9, 1)
            kern[name]["TFLOP_s"] = round(w["flops"] / avg / 1e12, 2)
    # dominant kernel: the largest share of the step
    dom = max(per_call, key=lambda n: float(np.sum(per_call[n])))
    w = work.get(dom)
    avg = float(np.mean(per_call[dom]))
    t_hbm = w["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = w["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        ach, peak, unit, bound = w["flops"] / avg / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = w["bytes"] / avg / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    roof = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic_for(key, dom), "kernel": dom,
            "algorithmic_bytes": w["bytes"], "algorithmic_flops": w["flops"], "avg_us": round(avg * 1e6, 2)}

    # the method's required HBM bytes per step (keys scanned, queries, head
    # weights, gathered and window rows, outputs; no intermediates) against
    # the step time, and the same for the scan and gather calls alone
    scan_gather = ("index_full", "index_pool", "attn", "attn_dense")
    step_bytes = sum(work[n]["bytes"] for n, _ in step.calls if n in scan_gather)
    sg_time = sum(float(np.sum(per_call[n])) for n in per_call if n in scan_gather) / steps
    hbm = {"step_bytes": step_bytes,
           "step_frac": round(step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
           "index_and_gather_frac": round(step_bytes / sg_time / (HBM_PEAK_GBS * 1e9), 4)}

    cpu = cpu_baseline(inp, cpu_seconds) if cpu_seconds > 0 else None
    rep = {
        "workload": wl.name + ("-bf16-out" if odt == "bf16" else ""), "value": round(value, 1),
        "unit": "query-tokens/s", "output_dtype": odt,
        "ms_per_step": round(ms_per_step, 4), "eager_ms_per_step": round(ms_eager, 4),
        "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 4),
        "steps": steps, "warmup": warmup,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3+bf16", "fp4": "fp4+mxfp4+e4m3+bf16"}[wl.kv_dtype],
        "config": {"workload": wl.name + ("-bf16-out" if odt == "bf16" else ""), "B": wl.B, "Tq": wl.Tq, "N": wl.N, "m": wl.m, "Hi": wl.Hi, "Di": wl.Di,
                   "H": wl.H, "D": wl.D, "K": wl.K, "W": wl.W, "blk": wl.blk, "P": wl.P,
                   "layers": list(wl.modes), "cache_copies": copies},
        "roofline": roof, "hbm": hbm, "cpu_baseline": cpu, "kernels": kern, "wall_s": round(wall, 3),
    }
    del step, grp, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rep


# --------------------------------------------------------------- record construction

def compress_work(cw):
    """Algorithmic bytes and flops of one csa2_compress call: the token rows
    c and z read once, gain and W_ik, the records and keys written once;
    flops of the keys (2 D Di per record)."""
    n = cw.B * (cw.T // cw.m)
    ein = 4 if cw.in_dtype == "f32" else 2
    rb = {"f32": 4 * cw.D, "bf16": 2 * cw.D, "e4m3": cw.D + 4, "fp4": cw.D // 2 + cw.D // 16}[cw.kv_dtype]
    kb = {"f32": 4 * cw.Di, "bf16": 2 * cw.Di, "e4m3": cw.Di + 4, "mxfp4": cw.Di // 2 + cw.Di // 32}[cw.k_dtype]
    return dict(bytes=2 * cw.B * cw.T * cw.D * ein + 4 * cw.D + 4 * cw.D * cw.Di + n * (rb + kb),
                flops=2.0 * cw.D * cw.Di * n)


def cpu_baseline_compress(inp, seconds):
    """The oracle's record construction (pooling, RMSNorm, RoPE in fp64, keys
    from the records) on a bounded sample: blocks of 64 records, one
    sequence after another."""
    import oracle as O
    cores, blas = cpu_threads()
    cw = inp["cw"]
    n = cw.T // cw.m
    done = 0
    t0 = time.perf_counter()
    for b in range(cw.B):
        for s0 in range(0, n, 64):
            tok = slice(s0 * cw.m, (s0 + 64) * cw.m)
            x = O.compress_records(O.dequant(inp["c"][b][tok]), O.dequant(inp["z"][b][tok]), cw.m, inp["gain"],
                                   1e-6, int(inp["t0"][b]) + s0 * cw.m, cw.rope_dims, 10000.0)
            O.derive_index_keys(x, inp["w_ik"])
            done += x.shape[0] * cw.m
            if time.perf_counter() - t0 > seconds:
                break
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": min(cores, blas), "kind": "oracle",
            "affinity_cores": cores, "blas_threads": blas,
            "sample": f"{done} of {cw.B * cw.T} token rows (blocks of 64 records, in order), fp64 NumPy, "
                      f"records before quantization and keys from them, {dt:.1f} s"}


def measure_compress(key, steps, warmup, cpu_seconds, torch):
    """Times `steps` csa2_compress calls of workload `key` (HIP events on the
    launch stream) and returns its report."""
    from sparse_long_context_csa2_amd import runner as R
    from sparse_long_context_csa2_amd import workloads as WL

    cw = WL.COMPRESS[key]
    inp = WL.make_compress_inputs(cw)
    dc = R.DeviceCompress(inp, device="cuda:0")
    stream = torch.cuda.Stream()
    for _ in range(warmup):
        dc.run(stream)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for s in range(steps):
            dc.run(stream)
            evs[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ts = [evs[s].elapsed_time(evs[s + 1]) * 1e-3 for s in range(steps)]
    avg = float(np.mean(ts))
    w = compress_work(cw)
    ach = w["bytes"] / avg / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_for(key, "compress"), "kernel": "compress",
            "algorithmic_bytes": w["bytes"], "algorithmic_flops": w["flops"], "avg_us": round(avg * 1e6, 2)}
    cpu = cpu_baseline_compress(inp, cpu_seconds) if cpu_seconds > 0 else None
    rep = {
        "workload": cw.name, "value": round(cw.B * cw.T / avg, 1), "unit": "tokens/s",
        "ms_per_step": round(avg * 1e3, 4), "steps": steps, "warmup": warmup,
        "dtype": f"{cw.in_dtype}->{cw.kv_dtype}+{cw.k_dtype}",
        "config": {"workload": cw.name, "B": cw.B, "T": cw.T, "m": cw.m, "D": cw.D, "Di": cw.Di,
                   "rope_dims": cw.rope_dims, "records": cw.B * (cw.T // cw.m)},
        "roofline": roof, "cpu_baseline": cpu,
        "kernels": {"compress": {"avg_us": round(avg * 1e6, 2), "calls_per_step": 1, "GB_s": round(ach, 1)}},
        "wall_s": round(wall, 3),
    }
    del dc, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rep


# --------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_long_context_csa2_amd import workloads as WL

    if args.workload in WL.COMPRESS:
        prim = measure_compress(args.workload, args.steps, args.warmup, 0 if args.no_cpu else args.cpu_seconds, torch)
    else:
        prim = measure(args.workload, args.steps, args.warmup, args.copies,
                       0 if args.no_cpu else args.cpu_seconds, torch,
                       graph=WL.CONFIGS[args.workload].decode_pos is not None)
    extra = {}
    if not args.only:
        for key in [k for k in args.extra.split(",") if k and k != args.workload]:
            print(f"[bench] {key}", file=sys.stderr, flush=True)
            cpu_s = 0 if args.no_cpu else args.extra_cpu_seconds
            if key in WL.COMPRESS:
                rep = measure_compress(key, args.extra_steps, args.warmup, cpu_s, torch)
            else:
                base = VARIANTS.get(key, (key,))[0]
                rep = measure(key, args.extra_steps, args.warmup, 0, 0 if key in VARIANTS else cpu_s, torch,
                              graph=WL.CONFIGS[base].decode_pos is not None)
            extra[key] = rep

    line = {
        "metric": "CSA2 layer query-tokens/s (prefill & decode) + % of HBM/MFMA peak, 1 GPU",
        "value": prim["value"],
        "unit": prim["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prim["dtype"],
        "data": "synthetic (seeded N(0,1/d) inputs of the workload's shapes)",
        "config": prim["config"],
        "roofline": prim["roofline"],
        "cpu_baseline": prim["cpu_baseline"],
        "kernels": prim["kernels"],
        "hbm": prim.get("hbm"),
        "eager_ms_per_step": prim.get("eager_ms_per_step"),
        "workloads": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
