"""The five workloads at full size, in the launch configuration the
benchmark times (one csa2_layer call per layer through DeviceGroup).  The
oracle checks sampled query rows one by one; every row is checked for the
properties that hold at any size (index counts, ranges, uniqueness,
finiteness)."""

import numpy as np
import pytest
import torch

import oracle as O
from sparse_long_context_csa2_amd import runner as R
from sparse_long_context_csa2_amd import workloads as WL
from tests import parity as PR

pytestmark = pytest.mark.gpu

SAMPLES = {
    "C1": [(0, t) for t in range(128)],
    "C2": [(0, t) for t in (0, 2, 3, 4, 100, 1000, 2046, 2047, 2050, 3333, 4095)],
    "C3": [(0, 0), (17, 0), (63, 0)],
    "C4": [(0, 0), (9, 0), (15, 0)],
    "C5": [(0, 0), (7, 0)],
}


def _row_properties(inp, idx, K, modes):
    """Every row: min(K, |visible|) unique valid ids, ascending, then -1."""
    wl = inp["wl"]
    q_pos = inp["layers"][0]["q_pos"]
    for b in range(wl.B):
        for ti in range(wl.Tq):
            t = int(q_pos[b, ti])
            nvis = min(wl.N, (t + 1) // wl.m)
            row = idx[b, ti]
            nv = int((row >= 0).sum())
            assert nv == min(K, nvis), (b, ti, nv)
            v = row[:nv]
            assert np.all(v >= 0) and np.all(v < nvis)
            assert np.all(np.diff(v) > 0)
            assert np.all(row[nv:] == -1)


@pytest.mark.parametrize("cfg", ["C1", "C2", "C3", "C4", "C5"])
def test_config_full_size(cfg):
    print(f"[case] full-size {cfg}", flush=True)
    wl = WL.CONFIGS[cfg]
    inp = WL.make_inputs(wl)
    grp = R.DeviceGroup(inp)
    grp.run()
    torch.cuda.synchronize()
    outs = grp.outputs()
    idxs = grp.index_sets()
    pool = None if grp.pool is None else grp.pool.cpu().numpy()
    for o in outs:
        assert np.isfinite(o).all()
    _row_properties(inp, idxs[0], wl.K, wl.modes)
    sh, lays = inp["shared"], inp["layers"]
    tol = PR.ATTN_TOL[wl.kv_dtype]
    worst = 0.0
    nd = 0
    for (b, ti) in SAMPLES[cfg]:
        prev = None
        for li, lay in enumerate(lays):
            where = f"{cfg} layer {li} ({lay['mode']}) b={b} t={ti}"
            ids = idxs[li][b, ti]
            if lay["mode"] == "full":
                r = O.layer_query(sh, lay, b, ti, O.FULL, build_pool=lay["build_pool"])
                nd += PR.check_topk(ids, r["cand"], r["scores"], lay["K"], where)
                if lay["build_pool"]:
                    gp = pool[b, ti]
                    valid = gp[gp >= 0]
                    blocks = r["cand"] // lay["blk"]
                    bids = np.unique(blocks)
                    beta = np.array([r["scores"][blocks == x].max() for x in bids])
                    PR.check_topk(np.concatenate([np.sort(valid), gp[len(valid):]]), bids, beta, lay["P"],
                                  where + " pool")
            elif lay["mode"] == "reindex":
                gp = pool[b, ti]
                r = O.layer_query(sh, lay, b, ti, O.REINDEX, pool_in=gp[gp >= 0])
                nd += PR.check_topk(ids, r["cand"], r["scores"], lay["K"], where)
            else:
                assert np.array_equal(ids, prev), where
            ref = PR.oracle_attention(sh, lay, b, ti, ids)
            worst = max(worst, PR.check_attn(outs[li][b, ti], ref, tol, where))
            prev = ids
    print(f"{cfg}: max attention error {worst:.3g}, boundary set differences {nd}")
