"""The allocation-free attention entry point (csa2_sparse_attn_noalloc),
called through the C ABI, against csa2_sparse_attn with a caller
workspace on the same inputs: two calls in a row, the second with a
smaller input, so the second call runs over the scratch the first left
behind.  Both must agree to the attention bound (they run the same
kernels, so they agree exactly), and the first is also checked against
the fp64 oracle."""

import ctypes

import numpy as np
import pytest
import torch

from sparse_long_context_csa2_amd import binding as Bd
from sparse_long_context_csa2_amd import runner as R
from sparse_long_context_csa2_amd import workloads as WL
from tests import parity as PR

pytestmark = pytest.mark.gpu


def _inputs(B, K, W, kdt, seed, Tq=1):
    N = 4096
    wl = WL.Workload(name="noalloc", seed=seed, B=B, Tq=Tq, N=N, m=4, Hi=32, Di=128, H=64, D=512, rope_dims=64,
                     W=W, K=K, decode_pos=5 * N, k_dtype=kdt, kv_dtype=kdt, swa_dtype=kdt, swa_slots=W + Tq + 3)
    inp = WL.make_inputs(wl)
    rng = np.random.default_rng(seed)
    idx = np.stack([[rng.permutation(N)[:K] for _ in range(Tq)] for _ in range(B)]).astype(np.int32)
    idx[0, 0, 3] = -1
    return wl, inp, idx


def _noalloc(L, q, kv, kv_scale, idx, swa, swa_scale, W, q_pos, sink, out):
    B, Tq, H, D = q.shape
    p = lambda t: None if t is None else t.data_ptr()
    return L.csa2_sparse_attn_noalloc(B, Tq, H, D, kv.shape[1], idx.shape[-1], p(q), Bd.dtype_code(q), p(kv),
                                      p(kv_scale), Bd.dtype_code(kv), p(idx), p(swa), p(swa_scale),
                                      Bd.dtype_code(swa), swa.shape[1], W, p(q_pos), p(sink), 0.0, 64, 10000.0,
                                      p(out), Bd.F32 if out.dtype == torch.float32 else Bd.BF16,
                                      torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("kdt", ["bf16", "e4m3"])
def test_noalloc_matches_workspace_entry_point(kdt):
    L = Bd.lib()
    for call, (B, K, W) in enumerate([(4, 512, 128), (2, 200, 64)]):
        print(f"[case] noalloc {kdt} call {call}: B={B} K={K} W={W}", flush=True)
        wl, inp, idx = _inputs(B, K, W, kdt, 40 + call)
        sh, lay = inp["shared"], inp["layers"][0]
        need = L.csa2_sparse_attn_workspace_bytes(B, 1, 64, 512, K, W)
        assert 0 < need <= 6 << 20  # both calls use the scratch
        d = {k: R.to_device(v) for k, v in (("q", lay["q"]), ("kv", sh["kv"]), ("kvs", sh["kv_scale"]),
                                            ("idx", idx), ("swa", lay["swa"]), ("swas", lay["swa_scale"]),
                                            ("pos", lay["q_pos"]), ("sink", lay["sink"]))}
        ref = Bd.csa2_sparse_attn(d["q"], d["kv"], d["kvs"], d["idx"], d["swa"], d["swas"], W, d["pos"],
                                  d["sink"], 64)
        out = torch.full_like(ref, float("nan"))
        rc = _noalloc(L, d["q"], d["kv"], d["kvs"], d["idx"], d["swa"], d["swas"], W, d["pos"], d["sink"], out)
        assert rc == 0, L.csa2_status_str(rc).decode()
        torch.cuda.synchronize()
        g, r = out.cpu().numpy(), ref.cpu().numpy()
        assert np.isfinite(g).all()
        for b in range(B):
            rows = PR.entry_rows(sh, lay, b, 0, idx[b, 0])
            PR.check_attn(g[b, 0], r[b, 0], PR.attn_tol(kdt, rows), f"call {call} b={b} vs csa2_sparse_attn")
        if call == 0:
            for b in (0, B - 1):
                PR.check_attn_query(g[b, 0], sh, lay, b, 0, idx[b, 0], kdt, f"call {call} b={b} vs oracle")
        print(f"max |noalloc - workspace| = {np.abs(g - r).max():.3g}", flush=True)


def test_noalloc_fewer_splits_when_scratch_is_short():
    """28 queries of one sequence: with a workspace the call splits every
    query's entries two ways (7.3 MB of partials); without one the splits
    taken only for parallelism give way to the 6 MiB scratch (here: none),
    and the result agrees with the workspace call to the attention bound."""
    L = Bd.lib()
    B, Tq, K, W = 1, 28, 512, 128
    print(f"[case] noalloc fewer splits: B={B} Tq={Tq} K={K} W={W}", flush=True)
    wl, inp, idx = _inputs(B, K, W, "bf16", 50, Tq=Tq)
    sh, lay = inp["shared"], inp["layers"][0]
    assert L.csa2_sparse_attn_workspace_bytes(B, Tq, 64, 512, K, W) > 6 << 20
    d = {k: R.to_device(v) for k, v in (("q", lay["q"]), ("kv", sh["kv"]), ("kvs", sh["kv_scale"]),
                                        ("idx", idx), ("swa", lay["swa"]), ("swas", lay["swa_scale"]),
                                        ("pos", lay["q_pos"]), ("sink", lay["sink"]))}
    ref = Bd.csa2_sparse_attn(d["q"], d["kv"], d["kvs"], d["idx"], d["swa"], d["swas"], W, d["pos"], d["sink"], 64)
    out = torch.full_like(ref, float("nan"))
    rc = _noalloc(L, d["q"], d["kv"], d["kvs"], d["idx"], d["swa"], d["swas"], W, d["pos"], d["sink"], out)
    assert rc == 0, L.csa2_status_str(rc).decode()
    torch.cuda.synchronize()
    g, r = out.cpu().numpy(), ref.cpu().numpy()
    assert np.isfinite(g).all()
    for ti in (0, 1, Tq // 2, Tq - 1):
        rows = PR.entry_rows(sh, lay, 0, ti, idx[0, ti])
        PR.check_attn(g[0, ti], r[0, ti], PR.attn_tol("bf16", rows), f"t={ti} vs csa2_sparse_attn")
        PR.check_attn_query(g[0, ti], sh, lay, 0, ti, idx[0, ti], "bf16", f"t={ti} vs oracle")
