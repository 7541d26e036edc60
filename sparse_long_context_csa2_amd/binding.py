"""ctypes binding of libcsa2.so (argument marshalling only).

Each function mirrors one C entry point of ``include/csa2.h`` and takes
torch tensors that already live on the GPU; it passes their data pointers,
sizes and dtype codes through and enqueues on the current torch stream.
Every step of the computation runs in the HIP kernels of the library.  A
missing library raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

CSA2_OK, CSA2_EINVAL, CSA2_EUNSUPPORTED, CSA2_EWORKSPACE, CSA2_EHIP = 0, -1, -2, -3, -4
F32, BF16, E4M3, FP4, MXFP4 = 0, 1, 2, 3, 4
FULL, REINDEX, REUSE, HCA = 0, 1, 2, 3
MODES = {"full": FULL, "reindex": REINDEX, "reuse": REUSE, "hca": HCA}
MAX_K = 2048

_c_int, _c_size, _vp, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class LayerDesc(ctypes.Structure):
    """Mirror of ``csa2_layer_desc``."""

    _fields_ = [
        ("mode", _c_int), ("B", _c_int), ("Tq", _c_int),
        ("N", _c_int), ("m", _c_int), ("n_rec", _vp),
        ("k_idx", _vp), ("k_scale", _vp), ("k_dtype", _c_int),
        ("kv", _vp), ("kv_scale", _vp), ("kv_dtype", _c_int),
        ("Hi", _c_int), ("Di", _c_int), ("q_idx", _vp), ("q_idx_dtype", _c_int), ("q_idx_scale", _vp), ("w", _vp),
        ("H", _c_int), ("D", _c_int), ("q", _vp), ("q_dtype", _c_int),
        ("swa", _vp), ("swa_scale", _vp), ("swa_dtype", _c_int), ("S", _c_int), ("W", _c_int),
        ("sink", _vp), ("sm_scale", _c_float), ("rope_dims", _c_int), ("rope_base", _c_float),
        ("q_pos", _vp),
        ("K", _c_int), ("idx_inout", _vp), ("blk", _c_int), ("P", _c_int), ("pool_inout", _vp),
        ("out", _vp), ("ws", _vp), ("ws_bytes", _c_size), ("out_dtype", _c_int),
    ]


class CSA2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"csa2 error {code}: {msg}")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """Opens libcsa2.so (built in-tree by ``build.py``); raises if absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python sparse_long_context_csa2_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        i, s, v, f = _c_int, _c_size, _vp, _c_float
        L.csa2_index_scores.argtypes = [i, i, i, i, i, i, v, i, v, v, v, v, i, v, v, v, i, i, v, v, s, v]
        L.csa2_block_pool.argtypes = [i, i, i, i, v, v, v, s, v]
        L.csa2_block_pool_workspace_bytes.argtypes = [i, i, i]
        L.csa2_block_pool_workspace_bytes.restype = s
        L.csa2_topk.argtypes = [i, i, i, v, v, i, i, v, v, s, v]
        L.csa2_topk_workspace_bytes.argtypes = [i, i, i]
        L.csa2_topk_workspace_bytes.restype = s
        L.csa2_sparse_attn.argtypes = [i, i, i, i, i, i, v, i, v, v, i, v, v, v, i, i, i, v, v, f, i, f, v, i,
                                       v, s, v]
        L.csa2_sparse_attn_noalloc.argtypes = [i, i, i, i, i, i, v, i, v, v, i, v, v, v, i, i, i, v, v, f, i, f,
                                               v, i, v]
        L.csa2_sparse_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.csa2_dense_attn.argtypes = [i, i, i, i, i, i, v, v, i, v, v, i, v, v, i, i, i, v, v, f, i, f, v, i, v, s,
                                      v]
        L.csa2_dense_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.csa2_dense_attn_workspace_bytes.restype = s
        L.csa2_sparse_attn_workspace_bytes.restype = s
        L.csa2_layer.argtypes = [ctypes.POINTER(LayerDesc), v]
        L.csa2_group.argtypes = [ctypes.POINTER(LayerDesc), i, v]
        L.csa2_compress.argtypes = [i, i, i, i, i, v, v, i, v, v, f, i, f, v, i, i, v, v, i, v, v, i, v]
        L.csa2_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.csa2_workspace_bytes.restype = s
        L.csa2_status_str.argtypes = [i]
        L.csa2_status_str.restype = ctypes.c_char_p
        L.csa2_version.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def _check(code: int) -> None:
    if code != CSA2_OK:
        raise CSA2Error(code, lib().csa2_status_str(code).decode())


class Prepared:
    """One entry-point call with its arguments converted to ctypes values
    once; calling it enqueues the same work again (same tensors, same
    stream) with almost no host cost per launch."""

    def __init__(self, cfunc, args, result=None, keep=()):
        self._f = cfunc
        self._args = tuple(t(a) if a is not None else None for t, a in zip(cfunc.argtypes, args))
        self.result = result
        self._keep = keep  # buffers the call uses that no caller holds (an allocated workspace)

    def __call__(self):
        code = self._f(*self._args)
        if code != CSA2_OK:
            _check(code)
        return self.result


def _call(cfunc, args, result, prepare: bool, keep=()):
    if prepare:
        return Prepared(cfunc, args, result, keep)
    _check(cfunc(*args))
    return result


def dtype_code(t: Optional[torch.Tensor], scale: Optional[torch.Tensor] = None) -> int:
    """Library dtype code of a storage tensor.  Packed four-bit tensors
    (torch.float4_e2m1fn_x2) are MXFP4 when an E8M0 scale tensor comes with
    them and FP4 main-KV rows (inline E4M3 group scales) otherwise."""
    if t is None:
        return F32
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return E4M3
    if t.dtype == torch.float4_e2m1fn_x2:
        return MXFP4 if scale is not None else FP4
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _elems(t: torch.Tensor) -> int:
    """Elements along the last axis (a packed four-bit byte holds two)."""
    return 2 * t.shape[-1] if t.dtype == torch.float4_e2m1fn_x2 else t.shape[-1]


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _torch_stream(stream, device):
    """The torch stream a call is enqueued on (a raw handle is wrapped)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _empty(shape, dtype, device, stream) -> torch.Tensor:
    """A temporary or output buffer allocated on the stream the kernels run
    on, so that torch's caching allocator orders its reuse after them."""
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(shape, dtype=dtype, device=device)


def _ws(nbytes: int, device, ws: Optional[torch.Tensor], stream=None) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return _empty(nbytes, torch.uint8, device, stream)


def csa2_index_scores(q_idx, w, k_idx, k_scale, q_pos, m: int, n_rec=None, pool=None, blk: int = 0,
                      out=None, stream=None, prepare: bool = False, q_scale=None) -> torch.Tensor:
    """Scores [B][Tq][N] (or [B][Tq][P*blk] with a pool); see csa2.h.
    ``q_scale``: the E8M0 block scales of MXFP4 queries.  With ``prepare``
    the call is returned as a ``Prepared`` instead of being enqueued
    (likewise for the other entry points)."""
    B, Tq, Hi = q_idx.shape[:3]
    Di = _elems(q_idx)
    N = k_idx.shape[1]
    P = 0 if pool is None else pool.shape[-1]
    ncols = N if pool is None else P * blk
    if out is None:
        out = _empty((B, Tq, ncols), torch.float32, q_idx.device, stream)
    return _call(lib().csa2_index_scores,
                 (B, Tq, N, Hi, Di, m, _p(q_idx), dtype_code(q_idx, q_scale), _p(q_scale), _p(w), _p(k_idx),
                  _p(k_scale), dtype_code(k_idx, k_scale), _p(q_pos), _p(n_rec), _p(pool), P,
                  blk if pool is not None else 0, _p(out), None, 0, _stream(stream)), out, prepare)


def csa2_block_pool(scores, blk: int, P: int, out=None, ws=None, stream=None, prepare: bool = False) -> torch.Tensor:
    """Block ids [rows][P] ordered by (block max desc, id asc), -1 padded."""
    N = scores.shape[-1]
    rows = scores.numel() // N
    if out is None:
        out = _empty(scores.shape[:-1] + (P,), torch.int32, scores.device, stream)
    nb = lib().csa2_block_pool_workspace_bytes(rows, N, blk)
    ws = _ws(nb, scores.device, ws, stream)
    return _call(lib().csa2_block_pool, (rows, N, blk, P, _p(scores), _p(out), _p(ws), nb, _stream(stream)), out,
                 prepare, (ws,))


def csa2_topk(scores, K: int, pool=None, blk: int = 0, out=None, ws=None, stream=None,
              prepare: bool = False) -> torch.Tensor:
    """Record ids [rows][K] of the K best scores (set, column order), -1 padded."""
    ncols = scores.shape[-1]
    rows = scores.numel() // ncols
    P = 0 if pool is None else pool.shape[-1]
    if out is None:
        out = _empty(scores.shape[:-1] + (K,), torch.int32, scores.device, stream)
    nb = lib().csa2_topk_workspace_bytes(rows, ncols, K)
    ws = _ws(nb, scores.device, ws, stream)
    return _call(lib().csa2_topk, (rows, ncols, K, _p(scores), _p(pool), P, blk if pool is not None else 0, _p(out),
                                   _p(ws), nb, _stream(stream)), out, prepare, (ws,))


def _out_code(out: torch.Tensor) -> int:
    """Output dtype code: float32 or bfloat16 tensors."""
    if out.dtype == torch.float32:
        return F32
    if out.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"attention output must be float32 or bfloat16, got {out.dtype}")


def csa2_sparse_attn(q, kv, kv_scale, idx, swa, swa_scale, W: int, q_pos, sink, rope_dims: int,
                     rope_base: float = 10000.0, sm_scale: float = 0.0, out=None, ws=None,
                     stream=None, prepare: bool = False, out_dtype=torch.float32) -> torch.Tensor:
    """Attention output [B][Tq][H][D] (float32, or bfloat16 rounded to
    nearest even: the dtype of ``out`` or ``out_dtype``); see csa2.h."""
    B, Tq, H, D = q.shape
    N = kv.shape[1]
    S = swa.shape[1]
    K = 0 if idx is None else idx.shape[-1]
    if out is None:
        out = _empty((B, Tq, H, D), out_dtype, q.device, stream)
    nb = lib().csa2_sparse_attn_workspace_bytes(B, Tq, H, D, K, W)
    ws = _ws(nb, q.device, ws, stream)
    return _call(lib().csa2_sparse_attn,
                 (B, Tq, H, D, N, K, _p(q), dtype_code(q), _p(kv), _p(kv_scale), dtype_code(kv, kv_scale), _p(idx),
                  _p(swa), _p(swa_scale), dtype_code(swa, swa_scale), S, W, _p(q_pos), _p(sink), float(sm_scale),
                  rope_dims, float(rope_base), _p(out), _out_code(out), _p(ws), nb, _stream(stream)), out, prepare,
                 (ws,))


def csa2_dense_attn(q, kv, kv_scale, swa, swa_scale, W: int, q_pos, sink, rope_dims: int, m: int, n_rec=None,
                    rope_base: float = 10000.0, sm_scale: float = 0.0, out=None, ws=None, stream=None,
                    prepare: bool = False, out_dtype=torch.float32) -> torch.Tensor:
    """HCA attention output [B][Tq][H][D] (float32 or bfloat16) over every
    visible record of kv at compression m; see csa2.h."""
    B, Tq, H, D = q.shape
    N = kv.shape[1]
    S = swa.shape[1]
    if out is None:
        out = _empty((B, Tq, H, D), out_dtype, q.device, stream)
    nb = lib().csa2_dense_attn_workspace_bytes(B, Tq, H, D, N, W)
    ws = _ws(nb, q.device, ws, stream)
    return _call(lib().csa2_dense_attn,
                 (B, Tq, H, D, N, m, _p(n_rec), _p(q), dtype_code(q), _p(kv), _p(kv_scale), dtype_code(kv, kv_scale),
                  _p(swa), _p(swa_scale), dtype_code(swa, swa_scale), S, W, _p(q_pos), _p(sink), float(sm_scale),
                  rope_dims, float(rope_base), _p(out), _out_code(out), _p(ws), nb, _stream(stream)), out, prepare,
                 (ws,))


def make_layer_desc(mode: str, shared: dict, layer: dict, idx_inout, pool_inout, out, ws=None) -> LayerDesc:
    """Fills a csa2_layer_desc from device tensors.

    ``shared``: k_idx, k_scale, kv, kv_scale, n_rec (tensors or None), m.
    ``layer``: q_idx, w, q, swa, swa_scale, sink, q_pos (tensors) and K, W,
    blk, P, rope_dims, rope_base, sm_scale.
    """
    d = LayerDesc()
    q = layer["q"]
    B, Tq, H, D = q.shape
    d.mode = MODES[mode] if isinstance(mode, str) else int(mode)
    d.B, d.Tq = B, Tq
    kv = shared["kv"]
    d.N, d.m = kv.shape[1], int(shared["m"])
    d.n_rec = _p(shared.get("n_rec"))
    k_idx = shared["k_idx"]
    d.k_idx, d.k_scale, d.k_dtype = _p(k_idx), _p(shared.get("k_scale")), dtype_code(k_idx, shared.get("k_scale"))
    d.kv, d.kv_scale, d.kv_dtype = _p(kv), _p(shared.get("kv_scale")), dtype_code(kv, shared.get("kv_scale"))
    q_idx = layer.get("q_idx")
    if q_idx is not None:
        qs = layer.get("q_idx_scale")
        d.Hi, d.Di = q_idx.shape[2], _elems(q_idx)
        d.q_idx, d.q_idx_dtype, d.q_idx_scale, d.w = _p(q_idx), dtype_code(q_idx, qs), _p(qs), _p(layer["w"])
    d.H, d.D, d.q, d.q_dtype = H, D, _p(q), dtype_code(q)
    swa = layer["swa"]
    d.swa, d.swa_scale, d.swa_dtype, d.S, d.W = _p(swa), _p(layer.get("swa_scale")), \
        dtype_code(swa, layer.get("swa_scale")), swa.shape[1], int(layer["W"])
    d.sink, d.sm_scale = _p(layer["sink"]), float(layer.get("sm_scale", 0.0))
    d.rope_dims, d.rope_base = int(layer["rope_dims"]), float(layer["rope_base"])
    d.q_pos = _p(layer["q_pos"])
    d.K, d.idx_inout = int(layer["K"]), _p(idx_inout)
    d.blk, d.P = int(layer.get("blk", 0) or 0), int(layer.get("P", 0) or 0)
    d.pool_inout = _p(pool_inout)
    d.out = _p(out)
    d.out_dtype = F32 if out is None else _out_code(out)
    d.ws = _p(ws)
    d.ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    return d


def csa2_workspace_bytes(desc: LayerDesc) -> int:
    return int(lib().csa2_workspace_bytes(ctypes.byref(desc)))


def csa2_layer(desc: LayerDesc, stream=None) -> None:
    """Enqueues one layer (see csa2.h); outputs land in the desc's buffers."""
    _check(lib().csa2_layer(ctypes.byref(desc), _stream(stream)))


def csa2_compress(c, z, t0, gain, w_ik, m: int, kv, k_idx, kv_scale=None, k_scale=None, rope_dims: int = 64,
                  rope_base: float = 10000.0, eps: float = 1e-6, stream=None, prepare: bool = False):
    """Records [B][N_out][..] and indexer keys from token rows c, z
    [B][T][D]; see csa2.h.  The cache tensors' dtypes (with their scale
    tensors) select the storage formats."""
    B, T, D = c.shape
    Di = _elems(k_idx)
    N_out = kv.shape[1]
    return _call(lib().csa2_compress,
                 (B, T, D, m, Di, _p(c), _p(z), dtype_code(c), _p(t0), _p(gain), float(eps), rope_dims,
                  float(rope_base), _p(w_ik), dtype_code(w_ik), N_out, _p(kv), _p(kv_scale),
                  dtype_code(kv, kv_scale), _p(k_idx), _p(k_scale), dtype_code(k_idx, k_scale), _stream(stream)),
                 (kv, k_idx), prepare)


def csa2_group(descs, stream=None) -> None:
    """Enqueues a sharing group (a sequence of layer descriptors) in one
    call; see csa2.h."""
    arr = (LayerDesc * len(descs))(*descs)
    _check(lib().csa2_group(arr, len(descs), _stream(stream)))


def version() -> str:
    return lib().csa2_version().decode()
