"""Host-side checks of the C ABI: the library loads, exports every function
that include/csa2.h declares, and rejects bad arguments with the documented
status codes before anything is launched (no GPU is touched: every call
below fails validation, and the *_workspace_bytes helpers are pure host
code)."""

import ctypes
import os
import re

import pytest

from sparse_long_context_csa2_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from sparse_long_context_csa2_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"csa2_index_scores", "csa2_block_pool", "csa2_topk", "csa2_sparse_attn", "csa2_layer"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, 7):
        assert L.csa2_status_str(code)
    assert B.version().startswith("csa2")


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_index_scores_validation(L):
    f = L.csa2_index_scores
    ok = dict(B=1, Tq=1, N=8, Hi=4, Di=16, m=1)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["B"], a["Tq"], a["N"], a["Hi"], a["Di"], a["m"], kw.get("q", FAKE), kw.get("qdt", 0),
                 kw.get("qs", None), kw.get("w", FAKE), kw.get("k", FAKE), kw.get("ks", None), kw.get("kdt", 0),
                 kw.get("pos", FAKE), None, kw.get("pool", None), kw.get("P", 0), kw.get("blk", 0),
                 kw.get("out", FAKE), None, 0, None)

    assert call(B=0) == B.CSA2_EINVAL
    assert call(m=0) == B.CSA2_EINVAL
    assert call(q=None) == B.CSA2_EINVAL
    assert call(out=None) == B.CSA2_EINVAL
    assert call(kdt=9) == B.CSA2_EINVAL
    assert call(kdt=2) == B.CSA2_EINVAL              # e4m3 without scale
    assert call(ks=FAKE) == B.CSA2_EINVAL            # scale for f32 keys
    assert call(qdt=2, qs=FAKE) == B.CSA2_EUNSUPPORTED  # e4m3 queries
    assert call(qdt=4) == B.CSA2_EINVAL              # mxfp4 queries without their scales
    assert call(qdt=4, qs=FAKE, kdt=1) == B.CSA2_EUNSUPPORTED  # mxfp4 queries need mxfp4 keys
    assert call(kdt=4) == B.CSA2_EINVAL              # mxfp4 keys without their scales
    assert call(kdt=4, ks=FAKE) == B.CSA2_EUNSUPPORTED  # mxfp4 needs the 32 x 128 kernel
    assert call(kdt=3) == B.CSA2_EUNSUPPORTED        # fp4 main-KV rows are no key format
    assert call(kdt=3, ks=FAKE) == B.CSA2_EINVAL     # fp4 rows carry their scales inline
    assert call(Hi=65) == B.CSA2_EUNSUPPORTED
    assert call(pool=FAKE, P=0, blk=4) == B.CSA2_EINVAL
    assert call(P=2, blk=4) == B.CSA2_EINVAL         # P/blk without a pool
    msg = L.csa2_status_str(B.CSA2_EINVAL).decode()
    assert "index_scores" in msg


def test_topk_and_pool_validation(L):
    assert L.csa2_topk(0, 8, 2, FAKE, None, 0, 0, FAKE, None, 0, None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 0, FAKE, None, 0, 0, FAKE, None, 0, None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 2049, FAKE, None, 0, 0, FAKE, None, 0, None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 2, None, None, 0, 0, FAKE, None, 0, None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 2, FAKE, FAKE, 3, 4, FAKE, None, 0, None) == B.CSA2_EINVAL  # 3*4 != 8
    assert L.csa2_block_pool(1, 64, 0, 4, FAKE, FAKE, FAKE, 1 << 20, None) == B.CSA2_EINVAL
    assert L.csa2_block_pool(1, 64, 4, 2049, FAKE, FAKE, FAKE, 1 << 20, None) == B.CSA2_EINVAL
    need = L.csa2_block_pool_workspace_bytes(3, 64, 4)
    assert need >= 3 * 16 * 4
    assert L.csa2_block_pool(3, 64, 4, 2, FAKE, FAKE, FAKE, need - 1, None) == B.CSA2_EWORKSPACE
    assert L.csa2_block_pool(3, 64, 4, 2, FAKE, FAKE, None, need, None) == B.CSA2_EWORKSPACE


def _attn(L, **kw):
    a = dict(B=1, Tq=1, H=64, D=512, N=100, K=16, q=FAKE, qdt=1, kv=FAKE, kvs=None, kvdt=1, idx=FAKE,
             swa=FAKE, swas=None, swadt=1, S=128, W=128, pos=FAKE, sink=FAKE, sm=0.0, r=64, base=10000.0,
             out=FAKE, ws=None, wsb=0)
    a.update(kw)
    return L.csa2_sparse_attn(a["B"], a["Tq"], a["H"], a["D"], a["N"], a["K"], a["q"], a["qdt"], a["kv"],
                              a["kvs"], a["kvdt"], a["idx"], a["swa"], a["swas"], a["swadt"], a["S"], a["W"],
                              a["pos"], a["sink"], a["sm"], a["r"], a["base"], a["out"], a.get("odt", 0), a["ws"],
                              a["wsb"], None)


def test_sparse_attn_validation(L):
    assert _attn(L, W=129) == B.CSA2_EINVAL           # window larger than ring
    assert _attn(L, K=2049) == B.CSA2_EINVAL
    assert _attn(L, r=63) == B.CSA2_EINVAL             # odd rotary dims
    assert _attn(L, r=1024) == B.CSA2_EINVAL
    assert _attn(L, base=0.0) == B.CSA2_EINVAL
    assert _attn(L, sm=-1.0) == B.CSA2_EINVAL
    assert _attn(L, sink=None) == B.CSA2_EINVAL
    assert _attn(L, kvdt=2) == B.CSA2_EINVAL           # e4m3 without scale
    assert _attn(L, kvs=FAKE) == B.CSA2_EINVAL         # scale for bf16
    assert _attn(L, qdt=2) == B.CSA2_EUNSUPPORTED
    assert _attn(L, kvdt=3) == B.CSA2_EUNSUPPORTED    # fp4 records need e4m3 window rows
    assert _attn(L, kvdt=3, kvs=FAKE, swadt=2, swas=FAKE) == B.CSA2_EINVAL  # fp4 scales are inline
    assert _attn(L, kvdt=4, kvs=FAKE) == B.CSA2_EUNSUPPORTED  # mxfp4 is no attention row format
    assert _attn(L, kvdt=3, swadt=2, swas=FAKE, H=2, D=16, qdt=0) == B.CSA2_EUNSUPPORTED  # 64 x 512 only
    assert _attn(L, H=3, D=2048, qdt=0, kvdt=0, swadt=0) == B.CSA2_EUNSUPPORTED
    assert _attn(L, odt=2) == B.CSA2_EUNSUPPORTED      # outputs are f32 or bf16
    assert _attn(L, odt=9) == B.CSA2_EINVAL
    assert _attn_noalloc(L, odt=3) == B.CSA2_EUNSUPPORTED
    # decode-shaped calls need split partials: an empty workspace is refused
    need = L.csa2_sparse_attn_workspace_bytes(1, 1, 64, 512, 512, 128)
    assert need > 0
    assert _attn(L, K=512, ws=None, wsb=0) == B.CSA2_EWORKSPACE
    assert _attn(L, K=512, ws=FAKE, wsb=need - 1) == B.CSA2_EWORKSPACE


def test_layer_validation_and_workspace(L):
    d = B.LayerDesc()
    d.mode, d.B, d.Tq, d.N, d.m = 0, 2, 1, 1000, 4
    d.k_idx, d.k_dtype, d.kv, d.kv_dtype = FAKE, 1, FAKE, 1
    d.Hi, d.Di, d.q_idx, d.q_idx_dtype, d.w = 32, 128, FAKE, 1, FAKE
    d.H, d.D, d.q, d.q_dtype = 64, 512, FAKE, 1
    d.swa, d.swa_dtype, d.S, d.W = FAKE, 1, 128, 128
    d.sink, d.rope_dims, d.rope_base, d.q_pos = FAKE, 64, 10000.0, FAKE
    d.K, d.idx_inout, d.out = 512, FAKE, FAKE
    need = L.csa2_workspace_bytes(ctypes.byref(d))
    assert need >= 2 * 1000 * 4
    d.ws, d.ws_bytes = FAKE, need - 1
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EWORKSPACE
    d.mode = 7
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EINVAL
    assert L.csa2_workspace_bytes(ctypes.byref(d)) == 0
    d.mode = 2
    d.idx_inout = None
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EINVAL
    d.idx_inout = FAKE
    d.K = 0
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EINVAL
    # pooled Reindex scores P*blk columns instead of N
    d.K, d.mode, d.pool_inout, d.P, d.blk = 512, 1, FAKE, 64, 64
    assert L.csa2_workspace_bytes(ctypes.byref(d)) >= 2 * 64 * 64 * 4
    assert L.csa2_layer(None, None) == B.CSA2_EINVAL


def test_misaligned_pointers_are_refused(L):
    """Every tensor pointer must be 16-byte aligned and every workspace
    256-byte aligned; a misaligned one is refused before any launch."""
    f = L.csa2_index_scores
    assert f(1, 1, 8, 4, 16, 1, FAKE + 8, 0, None, FAKE, FAKE, None, 0, FAKE, None, None, 0, 0, FAKE, None, 0,
             None) == B.CSA2_EINVAL
    assert "16-byte" in L.csa2_status_str(B.CSA2_EINVAL).decode()
    assert f(1, 1, 8, 4, 16, 1, FAKE, 0, None, FAKE, FAKE, None, 0, FAKE + 4, None, None, 0, 0, FAKE, None, 0,
             None) == B.CSA2_EINVAL
    assert f(1, 1, 8, 4, 16, 1, FAKE, 0, None, FAKE, FAKE, None, 0, FAKE, None, None, 0, 0, FAKE + 2, None, 0,
             None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 2, FAKE, None, 0, 0, FAKE + 4, FAKE, 1 << 20, None) == B.CSA2_EINVAL
    assert L.csa2_topk(1, 8, 2, FAKE, None, 0, 0, FAKE, FAKE + 16, 1 << 20, None) == B.CSA2_EINVAL
    assert "256-byte" in L.csa2_status_str(B.CSA2_EINVAL).decode()
    assert L.csa2_block_pool(3, 64, 4, 2, FAKE + 8, FAKE, FAKE, 1 << 20, None) == B.CSA2_EINVAL
    assert _attn(L, out=FAKE + 8) == B.CSA2_EINVAL
    assert _attn(L, kv=FAKE + 2) == B.CSA2_EINVAL
    assert _attn(L, K=512, ws=FAKE + 128, wsb=1 << 30) == B.CSA2_EINVAL
    d = B.LayerDesc()
    d.mode, d.B, d.Tq, d.N, d.m = 0, 2, 1, 1000, 4
    d.k_idx, d.k_dtype, d.kv, d.kv_dtype = FAKE, 1, FAKE, 1
    d.Hi, d.Di, d.q_idx, d.q_idx_dtype, d.w = 32, 128, FAKE, 1, FAKE
    d.H, d.D, d.q, d.q_dtype = 64, 512, FAKE, 1
    d.swa, d.swa_dtype, d.S, d.W = FAKE, 1, 128, 128
    d.sink, d.rope_dims, d.rope_base, d.q_pos = FAKE, 64, 10000.0, FAKE
    d.K, d.idx_inout, d.out = 512, FAKE, FAKE
    d.ws, d.ws_bytes = FAKE + 64, 1 << 30
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EINVAL
    d.ws, d.q = FAKE, FAKE + 8
    assert L.csa2_layer(ctypes.byref(d), None) == B.CSA2_EINVAL


def _attn_noalloc(L, **kw):
    a = dict(B=1, Tq=1, H=64, D=512, N=100, K=16, q=FAKE, qdt=1, kv=FAKE, kvs=None, kvdt=1, idx=FAKE,
             swa=FAKE, swas=None, swadt=1, S=128, W=128, pos=FAKE, sink=FAKE, sm=0.0, r=64, base=10000.0,
             out=FAKE)
    a.update(kw)
    return L.csa2_sparse_attn_noalloc(a["B"], a["Tq"], a["H"], a["D"], a["N"], a["K"], a["q"], a["qdt"], a["kv"],
                                      a["kvs"], a["kvdt"], a["idx"], a["swa"], a["swas"], a["swadt"], a["S"],
                                      a["W"], a["pos"], a["sink"], a["sm"], a["r"], a["base"], a["out"],
                                      a.get("odt", 0), None)


def test_sparse_attn_noalloc_validation(L):
    """The allocation-free entry point validates like csa2_sparse_attn.  A
    shape whose workspace call splits its queries into more partials than
    the 6 MiB static scratch holds (16 queries x 640 entries in four splits:
    8 MiB) is not refused: the splits taken only for parallelism give way,
    so it passes validation and fails here only at the launch (no device on
    this host).  Sparse decode shapes split into at most 64 partials."""
    assert _attn_noalloc(L, W=129) == B.CSA2_EINVAL
    assert _attn_noalloc(L, out=FAKE + 8) == B.CSA2_EINVAL
    assert _attn_noalloc(L, kvdt=2) == B.CSA2_EINVAL
    need = L.csa2_sparse_attn_workspace_bytes(16, 1, 64, 512, 512, 128)
    assert need > 6 << 20
    assert _attn_noalloc(L, B=16, K=512) == B.CSA2_EHIP
    # at most 64 partials of 64 heads x 512 channels (fp32), plus (max, sum)
    for Q in range(1, 65):
        assert L.csa2_sparse_attn_workspace_bytes(Q, 1, 64, 512, 2048, 256) <= 64 * (128 << 10) + (32 << 10)
    assert L.csa2_sparse_attn_workspace_bytes(64, 1, 64, 512, 512, 128) == 0


def test_dense_attn_validation(L):
    """csa2_dense_attn (HCA): the attention checks plus m >= 1; its
    workspace grows with the record count, since a long dense list is
    split across compute units."""
    def call(**kw):
        a = dict(B=1, Tq=1, H=64, D=512, N=8192, m=128, nrec=None, q=FAKE, qdt=1, kv=FAKE, kvs=None, kvdt=1,
                 swa=FAKE, swas=None, swadt=1, S=128, W=128, pos=FAKE, sink=FAKE, out=FAKE, ws=None, wsb=0)
        a.update(kw)
        return L.csa2_dense_attn(a["B"], a["Tq"], a["H"], a["D"], a["N"], a["m"], a["nrec"], a["q"], a["qdt"],
                                 a["kv"], a["kvs"], a["kvdt"], a["swa"], a["swas"], a["swadt"], a["S"], a["W"],
                                 a["pos"], a["sink"], 0.0, 64, 10000.0, a["out"], a.get("odt", 0), a["ws"],
                                 a["wsb"], None)
    assert call(m=0) == B.CSA2_EINVAL
    assert call(W=129) == B.CSA2_EINVAL
    assert call(nrec=FAKE + 4) == B.CSA2_EINVAL
    assert call(kvdt=2) == B.CSA2_EINVAL
    need = L.csa2_dense_attn_workspace_bytes(8, 1, 64, 512, 8192, 128)
    assert need >= 8 * 8 * 64 * 512 * 4  # 8 queries x 8 splits of fp32 partials
    assert call(B=8) == B.CSA2_EWORKSPACE
    assert L.csa2_dense_attn_workspace_bytes(8, 1, 64, 512, 10, 8) == 0  # one tile: no split
    assert call(H=3, D=2048, qdt=0, kvdt=0, swadt=0) == B.CSA2_EUNSUPPORTED


def test_group_validates_every_layer_first(L):
    """csa2_group refuses an empty group and, when any layer is invalid,
    returns that layer's error before enqueuing any layer."""
    d = B.LayerDesc()
    d.mode, d.B, d.Tq, d.N, d.m = 2, 1, 1, 100, 4
    d.kv, d.kv_dtype, d.H, d.D, d.q, d.q_dtype = FAKE, 1, 64, 512, FAKE, 1
    d.swa, d.swa_dtype, d.S, d.W = FAKE, 1, 128, 128
    d.sink, d.rope_dims, d.rope_base, d.q_pos = FAKE, 64, 10000.0, FAKE
    d.K, d.idx_inout, d.out = 16, FAKE, FAKE
    d.ws, d.ws_bytes = FAKE, 1 << 30
    bad = B.LayerDesc()
    ctypes.pointer(bad)[0] = d
    bad.mode = 9
    arr = (B.LayerDesc * 2)(d, bad)
    assert L.csa2_group(arr, 2, None) == B.CSA2_EINVAL
    assert "unknown mode" in L.csa2_status_str(B.CSA2_EINVAL).decode()
    d.ws_bytes = 16
    arr = (B.LayerDesc * 2)(d, d)
    assert L.csa2_group(arr, 2, None) == B.CSA2_EWORKSPACE
    assert L.csa2_group(arr, 0, None) == B.CSA2_EINVAL
    assert L.csa2_group(None, 1, None) == B.CSA2_EINVAL


def test_compress_validation(L):
    """csa2_compress: sizes, formats and scale arrays are checked on the
    host before any launch."""
    def call(**kw):
        a = dict(B=1, T=8, D=512, m=4, Di=128, c=FAKE, z=FAKE, idt=1, t0=FAKE, gain=FAKE, eps=1e-6, r=64,
                 base=10000.0, w=FAKE, wdt=1, N=16, kv=FAKE, kvs=None, kvdt=1, k=FAKE, ks=None, kdt=1)
        a.update(kw)
        return L.csa2_compress(a["B"], a["T"], a["D"], a["m"], a["Di"], a["c"], a["z"], a["idt"], a["t0"],
                               a["gain"], a["eps"], a["r"], a["base"], a["w"], a["wdt"], a["N"], a["kv"], a["kvs"],
                               a["kvdt"], a["k"], a["ks"], a["kdt"], None)
    assert call(T=10) == B.CSA2_EINVAL                 # T not a multiple of m
    assert call(m=0) == B.CSA2_EINVAL
    assert call(c=None) == B.CSA2_EINVAL
    assert call(z=FAKE + 8) == B.CSA2_EINVAL           # misaligned
    assert call(D=96) == B.CSA2_EUNSUPPORTED
    assert call(Di=100) == B.CSA2_EUNSUPPORTED
    assert call(idt=2) == B.CSA2_EUNSUPPORTED          # e4m3 token rows
    assert call(kvdt=2) == B.CSA2_EINVAL               # e4m3 records without their scales
    assert call(kvdt=3, kvs=FAKE) == B.CSA2_EINVAL     # fp4 records carry their scales inline
    assert call(kvdt=4, kvs=FAKE) == B.CSA2_EUNSUPPORTED
    assert call(kdt=4) == B.CSA2_EINVAL                # mxfp4 keys without their scales
    assert call(kdt=3) == B.CSA2_EUNSUPPORTED          # fp4 rows are no key format
    assert call(kdt=4, ks=FAKE, Di=192) == B.CSA2_EUNSUPPORTED  # mxfp4 keys: Di = 128 or 256
    assert call(r=63) == B.CSA2_EINVAL
    assert call(eps=-1.0) == B.CSA2_EINVAL
