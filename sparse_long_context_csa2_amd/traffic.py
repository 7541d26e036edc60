"""HBM traffic of the hot path's kernels from rocprofv3 counters.

Two steps (run each ``run`` under its own counter pass)::

    rocprofv3 --pmc FETCH_SIZE -f csv -d D1 -o run -- python3 -m sparse_long_context_csa2_amd.traffic run C2
    rocprofv3 --pmc WRITE_SIZE -f csv -d D2 -o run -- python3 -m sparse_long_context_csa2_amd.traffic run C2
    python3 -m sparse_long_context_csa2_amd.traffic summarize C2 D1 D2

``run`` executes the workload's step (the same calls, in the same order, as
``bench.py``) a fixed number of times and then an elementwise copy of a
known size.  ``summarize`` scales each counter by what it reads for that
copy (the copy reads and writes exactly COPY_BYTES), attributes the
dispatches of each ABI call of the step to that call, and writes
``profiles/traffic_<call>_<workload>.json`` (bytes per call, tagged with the
SHA-256 of the kernel source it was measured on) and a short Markdown
summary beside it.  ``bench.py`` reports the figure only while the source
is unchanged.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STEPS = 4
COPY_BYTES = 256 << 20

# kernel-name fragments of each ABI call, and the source file they come from
CALLS = {
    "attn": (("attn_mfma_kernel", "attn_combine_kernel", "attn_generic_kernel"), "attn.hip"),
    "index_full": (("idx_",), "indexer.hip"),
    "topk_full": (("topk_",), "topk.hip"),
}


def _run(workload: str) -> None:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch

    import bench
    from sparse_long_context_csa2_amd import runner as R
    from sparse_long_context_csa2_amd import workloads as WL

    wl = WL.CONFIGS[workload]
    copies = 2 if wl.decode_pos is not None else 1  # as bench.py: decode rotates two cache copies
    grp = R.DeviceGroup(WL.make_inputs(wl), device="cuda:0", copies=copies)
    step = bench.Step(grp, torch)
    for i in range(STEPS):
        step.run(i % copies)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)  # the reference: reads and writes COPY_BYTES
    torch.cuda.synchronize()
    print(json.dumps({"workload": workload, "steps": STEPS,
                      "calls": [name for name, _ in step.calls], "copy_bytes": COPY_BYTES}))


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


def _summarize(workload: str, fetch_dir: str, write_dir: str) -> None:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from sparse_long_context_csa2_amd import workloads as WL

    wl = WL.CONFIGS[workload]
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = _per_kernel(_rows(d), counter)
        copy = [v for name, v in disp if "MulFunctor" in name]
        if not copy:
            raise SystemExit(f"{counter}: the reference copy's dispatch is missing")
        scale = (COPY_BYTES / 1024.0) / copy[-1]  # true KiB per counted KiB
        res[counter] = (disp, scale, copy[-1])
    modes = [m.split("+")[0] for m in wl.modes]
    out_dir = os.path.join(ROOT, "profiles")
    lines = [f"# HBM traffic per call: {workload}", "",
             "Commands (from the repository root):", "",
             f"    rocprofv3 --pmc FETCH_SIZE -f csv -d D1 -o run -- python3 -m sparse_long_context_csa2_amd.traffic run {workload}",
             f"    rocprofv3 --pmc WRITE_SIZE -f csv -d D2 -o run -- python3 -m sparse_long_context_csa2_amd.traffic run {workload}",
             f"    python3 -m sparse_long_context_csa2_amd.traffic summarize {workload} D1 D2", "",
             "Scale: counted KiB of an elementwise copy that reads and writes "
             f"{COPY_BYTES >> 20} MiB: FETCH_SIZE {res['FETCH_SIZE'][2]:.0f} KiB (factor {res['FETCH_SIZE'][1]:.4f}), "
             f"WRITE_SIZE {res['WRITE_SIZE'][2]:.0f} KiB (factor {res['WRITE_SIZE'][1]:.4f}).", "",
             "| call | kernels | calls | fetch MB/call | write MB/call | HBM bytes/call |", "|---|---|---|---|---|---|"]
    for call, (frags, src) in CALLS.items():
        # a call's kernels must be unique to it within the step
        if call == "index_full" and "reindex" in modes:
            continue
        if call == "topk_full" and (wl.P or "reindex" in modes):
            continue
        tot = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            disp, scale, _ = res[counter]
            tot[counter] = sum(v for name, v in disp if any(f in name for f in frags)) * scale * 1024.0
        ncalls = STEPS * sum(1 for m in modes if call == "attn" or m == "full")
        if ncalls == 0 or tot["FETCH_SIZE"] == 0:
            continue
        per = (tot["FETCH_SIZE"] + tot["WRITE_SIZE"]) / ncalls
        src_path = os.path.join(ROOT, "sparse_long_context_csa2_amd", "csrc", src)
        rec = {"workload": workload, "call": call, "source": src,
               "source_sha256": hashlib.sha256(open(src_path, "rb").read()).hexdigest(),
               "fetch_bytes_per_launch": round(tot["FETCH_SIZE"] / ncalls),
               "write_bytes_per_launch": round(tot["WRITE_SIZE"] / ncalls),
               "bytes_per_launch": round(per),
               "fetch_scale": res["FETCH_SIZE"][1], "write_scale": res["WRITE_SIZE"][1]}
        json.dump(rec, open(os.path.join(out_dir, f"traffic_{call}_{workload}.json"), "w"), indent=1)
        lines.append(f"| {call} | {', '.join(frags)} | {ncalls} | {tot['FETCH_SIZE'] / ncalls / 1e6:.2f} | "
                     f"{tot['WRITE_SIZE'] / ncalls / 1e6:.2f} | {per:.4g} |")
    open(os.path.join(out_dir, f"traffic_{workload}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "run":
        _run(sys.argv[2])
    elif len(sys.argv) >= 5 and sys.argv[1] == "summarize":
        _summarize(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        raise SystemExit(__doc__)
