"""Workload registry and seeded synthetic input generators.

This module prepares inputs only: it draws random numbers, rounds them to
the storage formats (bf16 bit patterns, e4m3 codes with a per-row scale) and
lays them out.  It holds none of the layer's arithmetic, imports neither the
HIP binding nor the CPU oracle, and serves both of them.

Shapes and distributions follow the pages' workloads: Top-512, window 128,
64 heads x 512 latent with 64 rotary dims, 32 indexer heads, compression
m = 4 and contexts up to 1,048,576 tokens ("DeepSeek V4 Inside: One Token
Through Every Block", Flash-0731 config and "What does HCA change?"), and
the hierarchy of "DeepSeek V4.1-Flash. Every layer, connected." (toy:
128 positions, blocks of 4, 8 blocks, Top-8).

Random streams: ``SeedSequence(seed)`` spawns one child per tensor in a fixed
order (shared ``k_idx``, shared ``kv``, then for each layer ``q_idx``,
``w``, ``q``, ``swa``, ``sink``); a tensor with a batch axis spawns one
grandchild per sequence, so any sequence can be drawn on its own and the
chunks can be drawn in parallel with identical results.
"""

from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Storage-format encoders (input preparation only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even), as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values already in [-448, 448] -> OCP e4m3fn codes, rounding to
    nearest even and saturating at +-448 (never NaN)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), np.float32(448.0))
    u = a.view(np.uint32)
    # normal range: keep 3 mantissa bits, round half to even
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = (u + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
    exp = (r >> np.uint32(23)).astype(np.int32) - 127 + 7
    man = ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    code_n = (exp << 3) | man
    # subnormal range: multiples of 2^-9
    code_s = np.rint(a * np.float32(512.0)).astype(np.int32)  # exact scaling, RNE
    code = np.where(a < np.float32(2.0 ** -6), code_s, code_n)
    code = np.minimum(code, 0x7E)  # 448 is the largest finite code
    return (code | (neg.astype(np.int32) << 7)).astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3 quantization of a cache: scale = max|x| / 448 in float32,
    code = RNE(x / scale), saturating; an all-zero row has scale 0, codes 0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    v = (x / safe[..., None]).astype(np.float32)
    v = np.where((scale > 0)[..., None], v, np.float32(0.0))
    return e4m3_encode(v), scale


def _e4m3_decode_f32(codes: np.ndarray) -> np.ndarray:
    """Value of e4m3fn codes as float32 (the quantizers need the stored
    scale's value)."""
    c = np.asarray(codes, dtype=np.int32)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float32)
    v = np.where(e == 0, m / np.float32(8.0) * np.float32(2.0 ** -6),
                 (np.float32(1.0) + m / np.float32(8.0)) * np.exp2((e - 7).astype(np.float32)))
    return np.where(c & 0x80, -v, v).astype(np.float32)


# midpoints between neighbouring E2M1 magnitudes (0, 0.5, 1, 1.5, 2, 3, 4,
# 6), and whether an exact tie there rounds up: it does when the lower code
# is odd (mantissa bit set), so that ties go to the even code
_E2M1_MIDS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> four-bit E2M1 codes (one per element, 0..15): the
    nearest of the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the code
    with an even mantissa bit, saturating at 6; bit 3 is the sign."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.uint8)
    for mid, up in _E2M1_MIDS:
        code += (a >= np.float32(mid)) if up else (a > np.float32(mid))
    return code | (np.signbit(v).astype(np.uint8) << 3)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """One E2M1 code per element -> two per byte (element 2j in the low
    nibble of byte j)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _by_rows(fn, x: np.ndarray, rows: int = 8192):
    """Applies fn to chunks of rows of x (bounded temporaries)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1, x.shape[-1])
    if flat.shape[0] <= rows:
        return fn(x)
    parts = [fn(flat[i:i + rows]) for i in range(0, flat.shape[0], rows)]
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[k] for p in parts]).reshape(x.shape[:-1] + (parts[0][k].shape[-1],))
                     for k in range(len(parts[0])))
    return np.concatenate(parts).reshape(x.shape[:-1] + (parts[0].shape[-1],))


def quantize_rows_fp4(x: np.ndarray) -> np.ndarray:
    """FP4 main-KV rows: every 16 channels share one E4M3 scale, the largest
    magnitude of the group / 6 rounded to nearest even (an all-zero group has
    scale 0 and codes 0); codes = E2M1(x / scale).  Row layout: the D/2 code
    bytes, then the D/16 scale bytes (288 bytes for 512 channels)."""
    return _by_rows(_fp4_rows, x)


def _fp4_rows(x: np.ndarray) -> np.ndarray:
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // 16, 16))
    amax = np.abs(g).max(axis=-1)
    sc_code = e4m3_encode(amax / np.float32(6.0))
    sc = _e4m3_decode_f32(sc_code)
    safe = np.where(sc > 0, sc, np.float32(1.0))
    v = np.where((sc > 0)[..., None], g / safe[..., None], np.float32(0.0))
    codes = e2m1_encode(v).reshape(x.shape)
    return np.concatenate([pack_fp4(codes), sc_code], axis=-1)


def quantize_mxfp4(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """OCP MXFP4: blocks of 32 elements share an E8M0 scale 2^e with e =
    floor(log2(max |x|)) - 2 (2 is E2M1's largest exponent), clamped to
    [-127, 127]; elements = E2M1(x / 2^e), saturating.  Returns (packed
    codes [..., n/2], scale bytes e + 127 [..., n/32])."""
    return _by_rows(_mxfp4_rows, x)


def _mxfp4_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    n = x.shape[-1]
    blk = x.reshape(x.shape[:-1] + (n // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, np.float32(1e-38)))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    v = blk / np.exp2(e.astype(np.float32))[..., None]
    codes = e2m1_encode(v).reshape(x.shape)
    return pack_fp4(codes), (e + 127).astype(np.uint8)


# --------------------------------------------------------------------------
# Workload description
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    """One synthetic CSA2 workload (a sharing group of one or more layers)."""

    name: str
    seed: int
    B: int
    Tq: int
    N: int
    m: int
    Hi: int
    Di: int
    H: int
    D: int
    rope_dims: int
    W: int
    K: int
    blk: int = 0
    P: int = 0
    rope_base: float = 10000.0
    # decode: all queries at position `decode_pos`; prefill: q_pos = 0..Tq-1
    decode_pos: Optional[int] = None
    # storage dtypes: "f32" | "bf16" | "e4m3"; "fp4" (main KV rows: E2M1 + an
    # E4M3 scale per 16 channels); "mxfp4" (indexer queries and keys)
    q_idx_dtype: str = "bf16"
    k_dtype: str = "bf16"
    q_dtype: str = "bf16"
    kv_dtype: str = "bf16"
    swa_dtype: str = "bf16"
    # ring size of the local cache; 0 means Tq (prefill) or W (decode)
    swa_slots: int = 0
    # layer modes of the sharing group; "full+pool" builds the block pool
    modes: Tuple[str, ...] = ("full",)
    # distributions
    qk_idx_std: Optional[float] = None  # default 1/sqrt(Di)
    q_std: Optional[float] = None  # default 1/sqrt(D)
    kv_std: Optional[float] = None  # default 1/sqrt(D)
    w_dist: str = "softmax"  # "softmax" of N(0,1) over heads, or "uniform"
    # per-sequence visible record count; None means N for every sequence
    n_rec: Optional[Tuple[int, ...]] = None
    description: str = ""

    @property
    def S(self) -> int:
        if self.swa_slots:
            return self.swa_slots
        return self.W if self.decode_pos is not None else self.Tq

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS: Dict[str, Workload] = {
    "C1": Workload(
        name="C1-toy-fp32", seed=0, B=1, Tq=128, N=128, m=1, Hi=4, Di=16,
        H=2, D=16, rope_dims=4, W=8, K=8, blk=4, P=8,
        q_idx_dtype="f32", k_dtype="f32", q_dtype="f32", kv_dtype="f32", swa_dtype="f32",
        modes=("full+pool",), qk_idx_std=0.25, q_std=0.25, kv_std=1.0, w_dist="uniform",
        description="toy: T=128, m=1, 4x16 indexer, blocks of 4, keep 8, Top-8, "
                    "2 heads x 16 latent (4 rotary), SWA 8, fp32"),
    "C2": Workload(
        name="C2-prefill-bf16", seed=1, B=1, Tq=4096, N=1024, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512,
        description="Flash-shape prefill: T=4096, m=4 (N=1024), indexer 32x128, "
                    "Top-512, 64x512 latent (64 rotary), SWA 128, bf16"),
    "C3": Workload(
        name="C3-decode-full-bf16", seed=2, B=64, Tq=1, N=16384, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512, decode_pos=65536,
        description="decode, Full mode: B=64, context 65,536 (N=16,384), bf16"),
    "C4": Workload(
        name="C4-hier-decode-bf16", seed=3, B=16, Tq=1, N=65536, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512, blk=64, P=64, decode_pos=262144,
        modes=("full+pool", "reindex", "reindex", "reuse", "reuse"),
        description="hierarchical decode: B=16, context 262,144 (N=65,536); Full "
                    "pools 64 blocks of 64, then 2 Reindex and 2 Reuse layers, bf16"),
    "C5": Workload(
        name="C5-long-decode-e4m3", seed=4, B=8, Tq=1, N=262144, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512, decode_pos=1048576,
        k_dtype="e4m3", kv_dtype="e4m3", swa_dtype="e4m3",
        description="long-context decode: B=8, context 1,048,576 (N=262,144); "
                    "keys, latent and window in e4m3 with an fp32 scale per row"),
    "C6": Workload(
        name="C6-hca-decode-bf16", seed=5, B=8, Tq=1, N=8192, m=128, Hi=32, Di=128, H=64, D=512,
        rope_dims=64, W=128, K=0, decode_pos=1048576, modes=("hca",),
        description="heavily compressed attention decode: B=8, context 1,048,576 at m'=128 "
                    "(N=8,192 records, all visible), no indexer, SWA 128 plus sink, bf16"),
    "C7": Workload(
        name="C7-long-decode-fp4", seed=6, B=8, Tq=1, N=262144, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512, decode_pos=1048576,
        q_idx_dtype="mxfp4", k_dtype="mxfp4", kv_dtype="fp4", swa_dtype="e4m3",
        description="long-context decode in the V4.1 cache formats: B=8, context 1,048,576 "
                    "(N=262,144); main KV FP4 (E2M1 + E4M3 scale per 16 channels, 288 B rows), "
                    "indexer queries and keys MXFP4, window FP8"),
    "C8": Workload(
        name="C8-verify-decode-bf16", seed=7, B=16, Tq=5, N=16384, m=4, Hi=32, Di=128,
        H=64, D=512, rope_dims=64, W=128, K=512, decode_pos=65536,
        description="multi-query decode, Full mode: B=16 sequences at context 65,536 (N=16,384), "
                    "5 query positions each (a verification pass over drafted tokens), bf16"),
}

_NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "fp4": np.uint8, "mxfp4": np.uint8}

# --------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------

_POOL: Optional[_cf.ThreadPoolExecutor] = None


def _pool() -> _cf.ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = _cf.ThreadPoolExecutor(max_workers=n)
    return _POOL


def _normal_f32(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _store(x: np.ndarray, dtype: str):
    """float32 draw -> (storage array, scale array or None)."""
    if dtype == "f32":
        return x, None
    if dtype == "bf16":
        return f32_to_bf16_bits(x), None
    if dtype == "e4m3":
        return quantize_rows_e4m3(x)
    if dtype == "fp4":
        return quantize_rows_fp4(x), None
    if dtype == "mxfp4":
        return quantize_mxfp4(x)
    raise ValueError(dtype)


def stored_shape(row_shape, dtype: str):
    """(storage shape, scale shape or None) of a [..., n] float tensor."""
    *lead, n = row_shape
    if dtype == "fp4":
        return tuple(lead) + (n // 2 + n // 16,), None
    if dtype == "mxfp4":
        return tuple(lead) + (n // 2,), tuple(lead) + (n // 32,)
    if dtype == "e4m3":
        return tuple(row_shape), tuple(lead)
    return tuple(row_shape), None


def _batched_normal(ss: np.random.SeedSequence, B: int, row_shape, std: float, dtype: str,
                    only: Optional[List[int]] = None):
    """Draw a [B, *row_shape] tensor one sequence at a time (one grandchild
    stream per sequence) and store it.  ``only`` restricts the draw to some
    sequences (the others stay zero) for memory-bounded samples."""
    kids = ss.spawn(B)
    shp, sshp = stored_shape(row_shape, dtype)
    out = np.zeros((B,) + shp, dtype=_NP_STORAGE[dtype])
    scale = None
    if sshp is not None:
        scale = np.zeros((B,) + sshp, dtype=np.float32 if dtype == "e4m3" else np.uint8)
    idx = range(B) if only is None else only

    def one(b):
        arr, sc = _store(_normal_f32(kids[b], row_shape, std), dtype)
        out[b] = arr
        if scale is not None:
            scale[b] = sc

    list(_pool().map(one, idx))
    return out, scale


def make_inputs(wl: Workload, only: Optional[List[int]] = None, q_gain: float = 1.0) -> Dict:
    """Seeded inputs of a workload in storage form.

    Returns ``{"shared": {...}, "layers": [{...}, ...], "wl": wl}`` with
    numpy arrays: float32, uint16 (bf16 bits) or uint8 (e4m3 codes plus a
    float32 scale per row).  ``q_gain`` multiplies the main queries before
    rounding (a "sharp logits" stress variant).  ``only`` draws the given
    sequences only.
    """
    B, Tq, N = wl.B, wl.Tq, wl.N
    qk_std = wl.qk_idx_std if wl.qk_idx_std is not None else 1.0 / math.sqrt(wl.Di)
    q_std = (wl.q_std if wl.q_std is not None else 1.0 / math.sqrt(wl.D)) * q_gain
    kv_std = wl.kv_std if wl.kv_std is not None else 1.0 / math.sqrt(wl.D)
    n_layers = len(wl.modes)
    kids = np.random.SeedSequence(wl.seed).spawn(2 + 5 * n_layers)

    k_idx, k_scale = _batched_normal(kids[0], B, (N, wl.Di), qk_std, wl.k_dtype, only)
    kv, kv_scale = _batched_normal(kids[1], B, (N, wl.D), kv_std, wl.kv_dtype, only)
    n_rec = None if wl.n_rec is None else np.asarray(wl.n_rec, dtype=np.int32)
    shared = dict(N=N, m=wl.m, n_rec=n_rec, k_idx=k_idx, k_scale=k_scale,
                  kv=kv, kv_scale=kv_scale, k_format=wl.k_dtype, kv_format=wl.kv_dtype)

    if wl.decode_pos is not None:
        q_pos = np.full((B, Tq), wl.decode_pos, dtype=np.int64)
        if Tq > 1:
            q_pos = q_pos + np.arange(Tq, dtype=np.int64)[None, :] - (Tq - 1)
    else:
        q_pos = np.broadcast_to(np.arange(Tq, dtype=np.int64), (B, Tq)).copy()

    layers = []
    for li, mode_s in enumerate(wl.modes):
        base = 2 + 5 * li
        mode = mode_s.split("+")[0]
        q_idx, q_idx_scale = _batched_normal(kids[base + 0], B, (Tq, wl.Hi, wl.Di), qk_std,
                                             wl.q_idx_dtype, only)
        wk = kids[base + 1].spawn(B)
        w = np.zeros((B, Tq, wl.Hi), dtype=np.float32)
        for b in (range(B) if only is None else only):
            g = np.random.Generator(np.random.PCG64(wk[b]))
            if wl.w_dist == "uniform":
                w[b] = g.random(size=(Tq, wl.Hi), dtype=np.float32)
            else:
                z = g.standard_normal(size=(Tq, wl.Hi))
                z = np.exp(z - z.max(axis=-1, keepdims=True))
                w[b] = (z / z.sum(axis=-1, keepdims=True)).astype(np.float32)
        q, _ = _batched_normal(kids[base + 2], B, (Tq, wl.H, wl.D), q_std, wl.q_dtype, only)
        swa, swa_scale = _batched_normal(kids[base + 3], B, (wl.S, wl.D), kv_std,
                                         wl.swa_dtype, only)
        g = np.random.Generator(np.random.PCG64(kids[base + 4]))
        sink = g.standard_normal(size=wl.H).astype(np.float32)
        layers.append(dict(
            mode=mode, build_pool=mode_s.endswith("+pool"), q_pos=q_pos, q_idx=q_idx, w=w,
            q_idx_scale=q_idx_scale, q_idx_format=wl.q_idx_dtype, swa_format=wl.swa_dtype,
            q=q, swa=swa, swa_scale=swa_scale, sink=sink, K=wl.K, W=wl.W, blk=wl.blk,
            P=wl.P, rope_dims=wl.rope_dims, rope_base=wl.rope_base, sm_scale=0.0))
    return {"shared": shared, "layers": layers, "wl": wl}


def dtype_code(dtype: str) -> int:
    """Storage dtype name -> the library's dtype code (0 f32, 1 bf16, 2 e4m3,
    3 fp4 main-KV rows, 4 mxfp4)."""
    return {"f32": 0, "bf16": 1, "e4m3": 2, "fp4": 3, "mxfp4": 4}[dtype]


def storage_dtype_name(arr: np.ndarray) -> str:
    return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16",
            np.dtype(np.uint8): "e4m3"}[np.asarray(arr).dtype]


# --------------------------------------------------------------------------
# Record construction workloads (csa2_compress)
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class CompressWorkload:
    """Token rows of B sequences turned into records and indexer keys."""

    name: str
    seed: int
    B: int
    T: int
    m: int
    D: int
    Di: int
    rope_dims: int
    in_dtype: str = "bf16"
    kv_dtype: str = "fp4"
    k_dtype: str = "mxfp4"
    description: str = ""


COMPRESS: Dict[str, CompressWorkload] = {
    "C9": CompressWorkload(
        name="C9-compress-prefill-fp4", seed=8, B=16, T=4096, m=4, D=512, Di=128, rope_dims=64,
        description="record construction for 16 sequences x 4096 tokens at m=4 (16,384 records): "
                    "channel-wise softmax pooling, RMSNorm, RoPE, FP4 records and MXFP4 indexer keys"),
}


def make_compress_inputs(cw: CompressWorkload) -> Dict:
    """Token rows c (candidate latents) and z (gate logits) ~ N(0, 1), gain ~
    U(0.5, 1.5), W_ik ~ N(0, 1/D); sequences start at position 0."""
    kids = np.random.SeedSequence(cw.seed).spawn(4)
    c, _ = _batched_normal(kids[0], cw.B, (cw.T, cw.D), 1.0, cw.in_dtype)
    z, _ = _batched_normal(kids[1], cw.B, (cw.T, cw.D), 1.0, cw.in_dtype)
    g = np.random.Generator(np.random.PCG64(kids[2]))
    gain = g.uniform(0.5, 1.5, size=cw.D).astype(np.float32)
    w = (np.random.Generator(np.random.PCG64(kids[3])).standard_normal((cw.D, cw.Di)) /
         math.sqrt(cw.D)).astype(np.float32)
    return dict(c=c, z=z, gain=gain, w_ik=w, t0=np.zeros(cw.B, dtype=np.int64), cw=cw)
