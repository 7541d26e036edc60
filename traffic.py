"""HBM traffic of the hot path's ABI calls from rocprofv3 counters.

Two counter passes and a summary (from the repository root)::

    rocprofv3 --pmc FETCH_SIZE -f csv -d D1 -o run -- python3 traffic.py run C2
    rocprofv3 --pmc WRITE_SIZE -f csv -d D2 -o run -- python3 traffic.py run C2
    python3 traffic.py summarize C2 D1 D2

``run`` executes the workload's step once (the same calls, in the same
order, as ``bench.py``), then each distinct ABI call of the step on its own
``STEPS`` times, each group preceded by a small bitwise-not kernel that marks where
it starts, and finally an elementwise copy of a known size.  ``summarize``
scales each counter by what it reads for that copy (the copy reads and
writes exactly COPY_BYTES), splits the dispatches at the markers, and writes
``profiles/traffic_<call>_<workload>.json`` (bytes per call, tagged with the
SHA-256 of the kernel source it was measured on) and a short Markdown
summary beside it.  ``bench.py`` reports a figure only while its source is
unchanged.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
STEPS = 4
COPY_BYTES = 256 << 20
MARK = "bitwise_not"   # kernel-name fragment of the group markers
COPY = "MulFunctor"    # kernel-name fragment of the reference copy

# source files of each ABI call's kernels
_ATTN = ["attn.hip", "attn_kernel.h", "attn_dec.hip"]
SOURCE = {"attn": _ATTN, "attn_dense": _ATTN, "index_full": ["indexer.hip"], "index_pool": ["indexer.hip"],
          "topk_full": ["topk.hip"], "topk_pool": ["topk.hip"], "block_pool": ["topk.hip"],
          "compress": ["compress.hip"]}


def source_sha256(files) -> str:
    """SHA-256 over the listed kernel sources (csrc/), concatenated in order."""
    h = hashlib.sha256()
    for f in ([files] if isinstance(files, str) else files):
        h.update(open(os.path.join(ROOT, "sparse_long_context_csa2_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _run(workload: str) -> None:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch

    import bench
    from sparse_long_context_csa2_amd import runner as R
    from sparse_long_context_csa2_amd import workloads as WL

    if workload in WL.COMPRESS:  # record construction: one call per step
        dc = R.DeviceCompress(WL.make_compress_inputs(WL.COMPRESS[workload]), device="cuda:0")
        dc.run()
        torch.cuda.synchronize()
        mark = torch.zeros(64, dtype=torch.int32, device="cuda:0")
        torch.bitwise_not(mark, out=mark)
        for s in range(STEPS):
            dc.run()
        torch.bitwise_not(mark, out=mark)  # closes the group
        torch.cuda.synchronize()
        _copy(torch)
        print(json.dumps({"workload": workload, "steps": STEPS, "calls": ["compress"], "copy_bytes": COPY_BYTES}))
        return
    wl = WL.CONFIGS[workload]
    copies = 2 if wl.decode_pos is not None else 1  # as bench.py: decode rotates two cache copies
    grp = R.DeviceGroup(WL.make_inputs(wl), device="cuda:0", copies=copies)
    step = bench.Step(grp, torch)
    step.run(0)
    torch.cuda.synchronize()
    names = []
    mark = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    for i, (name, _) in enumerate(step.calls):
        if name in names:
            continue
        names.append(name)
        torch.bitwise_not(mark, out=mark)  # marks the start of this call's group
        for s in range(STEPS):
            step.prepared[i][s % copies]()
        torch.cuda.synchronize()
    torch.bitwise_not(mark, out=mark)  # closes the last group
    torch.cuda.synchronize()
    _copy(torch)
    print(json.dumps({"workload": workload, "steps": STEPS, "calls": names, "copy_bytes": COPY_BYTES}))


def _copy(torch) -> None:
    """The reference copy: reads and writes COPY_BYTES."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _calls_of(workload: str):
    """Distinct ABI call names of a workload's step, in order (as bench.Step
    enqueues them)."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from sparse_long_context_csa2_amd import workloads as WL

    if workload in WL.COMPRESS:
        return ["compress"]
    names = []
    for mode in WL.CONFIGS[workload].modes:
        m = mode.split("+")[0]
        seq = {"full": ["index_full"] + (["block_pool"] if mode.endswith("+pool") else []) + ["topk_full"],
               "reindex": ["index_pool", "topk_pool"], "reuse": [], "hca": []}[m] + \
            (["attn_dense"] if m == "hca" else ["attn"])
        names += [n for n in seq if n not in names]
    return names


def _algorithmic(workload: str):
    """Algorithmic bytes per call (bench.py's accounting)."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    from sparse_long_context_csa2_amd import workloads as WL

    if workload in WL.COMPRESS:
        return {"compress": bench.compress_work(WL.COMPRESS[workload])["bytes"]}
    wl = WL.CONFIGS[workload]
    return {k: v["bytes"] for k, v in bench.kernel_work(wl, WL.make_inputs(wl)).items()}


def _rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(files[0])))


def _per_kernel(rows, counter: str):
    """(kernel name, KiB) per dispatch in dispatch order."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        out[did] = (r["Kernel_Name"], out.get(did, (None, 0.0))[1] + float(r["Counter_Value"]))
    return [out[k] for k in sorted(out)]


def _groups(disp, ncalls):
    """Dispatches between consecutive markers (the step run before the
    first marker and the reference copy after the last are dropped)."""
    copy_at = max(i for i, (name, _) in enumerate(disp) if COPY in name)
    # the last ncalls + 1 markers before the copy (set-up fills come earlier)
    marks = [i for i, (name, _) in enumerate(disp) if MARK in name and i < copy_at][-(ncalls + 1):]
    if len(marks) != ncalls + 1:
        raise SystemExit(f"expected {ncalls + 1} markers, found {len(marks)}")
    return [disp[a + 1:b] for a, b in zip(marks[:-1], marks[1:])]


def _summarize(workload: str, fetch_dir: str, write_dir: str, calls) -> None:
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = _per_kernel(_rows(d), counter)
        copy = [v for name, v in disp if COPY in name]
        if not copy:
            raise SystemExit(f"{counter}: the reference copy's dispatch is missing")
        scale = (COPY_BYTES / 1024.0) / copy[-1]  # true KiB per counted KiB
        res[counter] = (_groups(disp, len(calls)), scale, copy[-1])
    out_dir = os.path.join(ROOT, "profiles")
    lines = [f"# HBM traffic per call: {workload}", "",
             "Commands (from the repository root):", "",
             f"    rocprofv3 --pmc FETCH_SIZE -f csv -d D1 -o run -- python3 traffic.py run {workload}",
             f"    rocprofv3 --pmc WRITE_SIZE -f csv -d D2 -o run -- python3 traffic.py run {workload}",
             f"    python3 traffic.py summarize {workload} D1 D2", "",
             "Scale: counted KiB of an elementwise copy that reads and writes "
             f"{COPY_BYTES >> 20} MiB: FETCH_SIZE {res['FETCH_SIZE'][2]:.0f} KiB (factor {res['FETCH_SIZE'][1]:.4f}), "
             f"WRITE_SIZE {res['WRITE_SIZE'][2]:.0f} KiB (factor {res['WRITE_SIZE'][1]:.4f}).", "",
             f"Each call ran {STEPS} times on its own; figures are per call.", "",
             "| call | kernels | fetch MB/call | write MB/call | HBM bytes/call | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|"]
    algo = _algorithmic(workload)
    for gi, call in enumerate(calls):
        tot, kern = {}, set()
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            groups, scale, _ = res[counter]
            tot[counter] = sum(v for _, v in groups[gi]) * scale * 1024.0 / STEPS
            kern |= {name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("csa2::", "")
                     for name, _ in groups[gi]}
        per = tot["FETCH_SIZE"] + tot["WRITE_SIZE"]
        src = SOURCE[call]
        rec = {"workload": workload, "call": call, "source": src,
               "source_sha256": source_sha256(src),
               "kernels": sorted(kern),
               "fetch_bytes_per_launch": round(tot["FETCH_SIZE"]),
               "write_bytes_per_launch": round(tot["WRITE_SIZE"]),
               "bytes_per_launch": round(per),
               "fetch_scale": res["FETCH_SIZE"][1], "write_scale": res["WRITE_SIZE"][1]}
        a = algo.get(call)
        rec["algorithmic_bytes"] = a
        json.dump(rec, open(os.path.join(out_dir, f"traffic_{call}_{workload}.json"), "w"), indent=1)
        lines.append(f"| {call} | {', '.join(sorted(kern))} | {tot['FETCH_SIZE'] / 1e6:.2f} | "
                     f"{tot['WRITE_SIZE'] / 1e6:.2f} | {per:.4g} | {a if a else '-'} | "
                     f"{per / a:.2f} |" if a else f"| {call} | {', '.join(sorted(kern))} | "
                     f"{tot['FETCH_SIZE'] / 1e6:.2f} | {tot['WRITE_SIZE'] / 1e6:.2f} | {per:.4g} | - | - |")
    open(os.path.join(out_dir, f"traffic_{workload}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "run":
        _run(sys.argv[2])
    elif len(sys.argv) >= 5 and sys.argv[1] == "summarize":
        _summarize(sys.argv[2], sys.argv[3], sys.argv[4], _calls_of(sys.argv[2]))
    else:
        raise SystemExit(__doc__)
