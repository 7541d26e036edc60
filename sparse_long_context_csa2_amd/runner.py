"""Device-side driver of a CSA2 sharing group through the C ABI.

``DeviceGroup`` uploads a workload's storage arrays (see
:mod:`.workloads`) to the GPU once, owns the per-layer index, pool, output
and workspace buffers, and enqueues the layers with ``csa2_layer`` in
order: a Full layer (optionally building the block pool), Reindex layers
searching that pool, Reuse layers reading the last index set, and HCA
layers attending to every visible record.  ``DeviceCompress`` does the
same for record construction (csa2_compress).
"""

from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as _b


def to_device(arr, device="cuda", fmt: Optional[str] = None) -> Optional[torch.Tensor]:
    """numpy storage array -> device tensor (uint16 bf16 bits become a
    bfloat16 view, uint8 e4m3 codes stay uint8).  ``fmt`` "fp4" or "mxfp4"
    tags packed four-bit codes as torch.float4_e2m1fn_x2, "e8m0" tags MX
    block scales as torch.float8_e8m0fnu (views of the same bytes)."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    t = torch.from_numpy(a).to(device)
    if fmt in ("fp4", "mxfp4"):
        return t.view(torch.float4_e2m1fn_x2)
    if fmt == "e8m0":
        return t.view(torch.float8_e8m0fnu)
    return t


def _scale_fmt(fmt: Optional[str]) -> Optional[str]:
    return "e8m0" if fmt == "mxfp4" else None


class DeviceGroup:
    def __init__(self, inputs: Dict, device: str = "cuda", copies: int = 1, out_dtype=torch.float32):
        wl = inputs["wl"]
        self.wl = wl
        self.device = device
        sh = inputs["shared"]
        kf, vf = sh.get("k_format"), sh.get("kv_format")
        self.shared = [dict(m=sh["m"], n_rec=to_device(sh["n_rec"], device),
                            k_idx=to_device(sh["k_idx"], device, kf),
                            k_scale=to_device(sh["k_scale"], device, _scale_fmt(kf)),
                            kv=to_device(sh["kv"], device, vf), kv_scale=to_device(sh["kv_scale"], device))]
        # extra copies of the shared store let a benchmark rotate caches
        for _ in range(copies - 1):
            self.shared.append({k: (v.clone() if isinstance(v, torch.Tensor) else v)
                                for k, v in self.shared[0].items()})
        self.layers: List[Dict] = []
        B, Tq = wl.B, wl.Tq
        for lay in inputs["layers"]:
            d = {k: lay[k] for k in ("mode", "build_pool", "K", "W", "blk", "P", "rope_dims", "rope_base",
                                     "sm_scale")}
            for k in ("w", "q", "swa", "swa_scale", "sink", "q_pos"):
                d[k] = to_device(lay[k], device)
            qf = lay.get("q_idx_format")
            d["q_idx"] = to_device(lay["q_idx"], device, qf)
            d["q_idx_scale"] = to_device(lay.get("q_idx_scale"), device, _scale_fmt(qf))
            d["out"] = torch.empty((B, Tq, wl.H, wl.D), dtype=out_dtype, device=device)
            self.layers.append(d)
        # index sets: Full/Reindex write their own; Reuse reads the last one
        self.idx: List[torch.Tensor] = []
        cur = None
        for d in self.layers:
            if d["mode"] in ("full", "reindex"):
                cur = torch.full((B, Tq, d["K"]), -1, dtype=torch.int32, device=device)
            self.idx.append(cur if d["mode"] != "hca" else None)
        self.pool = None
        if any(d["build_pool"] for d in self.layers):
            self.pool = torch.full((B, Tq, wl.P), -1, dtype=torch.int32, device=device)
        self.descs = []
        ws_need = 0
        for copy in range(copies):
            row = []
            for li, d in enumerate(self.layers):
                pool = self.pool if (d["build_pool"] or d["mode"] == "reindex") else None
                desc = _b.make_layer_desc(d["mode"], self.shared[copy], d, self.idx[li], pool, d["out"])
                ws_need = max(ws_need, _b.csa2_workspace_bytes(desc))
                row.append(desc)
            self.descs.append(row)
        self.ws = torch.empty(max(ws_need, 256), dtype=torch.uint8, device=device)
        for row in self.descs:
            for desc in row:
                desc.ws = self.ws.data_ptr()
                desc.ws_bytes = self.ws.numel()

    def run(self, copy: int = 0, stream=None) -> None:
        """The whole group through one csa2_group call."""
        _b.csa2_group(self.descs[copy], stream)

    def capture(self, copy: int = 0) -> "torch.cuda.CUDAGraph":
        """The group's launches captured as one HIP graph (replay() reruns
        the whole group on the same buffers)."""
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            self.run(copy, s)
        return g

    def outputs(self) -> List[np.ndarray]:
        return [d["out"].float().cpu().numpy() for d in self.layers]

    def index_sets(self) -> List[Optional[np.ndarray]]:
        return [None if i is None else i.cpu().numpy() for i in self.idx]


class DeviceCompress:
    """One record-construction workload on a device: token rows, gain and
    W_ik uploaded once, record and key caches (with their scales) allocated
    in the workload's formats."""

    _NP = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "fp4": np.uint8, "mxfp4": np.uint8}

    def __init__(self, inputs: Dict, device: str = "cuda"):
        cw = inputs["cw"]
        self.cw = cw
        B, n, D, Di = cw.B, cw.T // cw.m, cw.D, cw.Di
        self.n_out = n
        self.c = to_device(inputs["c"], device)
        self.z = to_device(inputs["z"], device)
        self.t0 = to_device(inputs["t0"], device)
        self.gain = to_device(inputs["gain"], device)
        self.w = to_device(inputs["w_ik"], device)
        kv_w = D // 2 + D // 16 if cw.kv_dtype == "fp4" else D
        k_w = Di // 2 if cw.k_dtype == "mxfp4" else Di
        self.kv = to_device(np.zeros((B, n, kv_w), self._NP[cw.kv_dtype]), device,
                            "fp4" if cw.kv_dtype == "fp4" else None)
        self.k = to_device(np.zeros((B, n, k_w), self._NP[cw.k_dtype]), device,
                           "mxfp4" if cw.k_dtype == "mxfp4" else None)
        self.kv_scale = torch.zeros((B, n), dtype=torch.float32, device=device) if cw.kv_dtype == "e4m3" else None
        self.k_scale = None
        if cw.k_dtype == "e4m3":
            self.k_scale = torch.zeros((B, n), dtype=torch.float32, device=device)
        elif cw.k_dtype == "mxfp4":
            self.k_scale = torch.zeros((B, n, Di // 32), dtype=torch.uint8, device=device).view(torch.float8_e8m0fnu)

    def run(self, stream=None) -> None:
        cw = self.cw
        _b.csa2_compress(self.c, self.z, self.t0, self.gain, self.w, cw.m, self.kv, self.k,
                        kv_scale=self.kv_scale, k_scale=self.k_scale, rope_dims=cw.rope_dims, stream=stream)

    def fetch(self):
        """(records, record scales, keys, key scales) as numpy storage arrays."""
        cw = self.cw

        def raw(t, fmt):
            if t is None:
                return None
            if fmt == "f32":
                return t.cpu().numpy()
            return t.view(torch.uint8).cpu().numpy().view(self._NP[fmt])

        ks = None if self.k_scale is None else (
            self.k_scale.view(torch.uint8).cpu().numpy() if cw.k_dtype == "mxfp4" else self.k_scale.cpu().numpy())
        return (raw(self.kv, cw.kv_dtype), None if self.kv_scale is None else self.kv_scale.cpu().numpy(),
                raw(self.k, cw.k_dtype), ks)
