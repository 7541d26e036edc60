"""Comparison rules between the HIP library and the fp64 oracle.

* Indexer scores: -inf exactly where the oracle has -inf; elsewhere
  |gpu - oracle| <= 1e-4 * max(|oracle|, 1e-3 * max_s |oracle[row, s]|)
  (relative 1e-4; the floor keeps a score that fp32 rounds across zero from
  failing the relative test).
* Top-K sets: equal sizes; every id valid, unique and a candidate; ids in
  the symmetric difference must have oracle scores within 1e-4 (relative)
  of the oracle's K-th score.
* Attention: evaluated on the GPU's own admissible index set.  The
  contract's max-abs bounds (2e-3 for f32/bf16 rows, 5e-2 for e4m3 rows)
  are stated for unit-scale inputs.  An output is a weighted mean of the
  rows it attends to, so every error term (rounding of the probabilities,
  fp32 accumulation) scales with the rows: for rows of RMS sigma below 1
  the bound used is bound * sigma.  Quantized rows are held to the bf16
  bound as well, because the oracle decodes the very codes the kernel
  reads: the fp8 allowance covers quantization against unquantized data,
  which is not a difference here.
"""

import math

import numpy as np

import oracle as O

SCORE_RTOL = 1e-4
SET_BAND = 1e-4
# contract bounds for unit-scale rows; the one applied to every dtype here
ATTN_TOL = {"f32": 2e-3, "bf16": 2e-3, "e4m3": 2e-3, "fp4": 2e-3}
ATTN_TOL_CONTRACT = {"f32": 2e-3, "bf16": 2e-3, "e4m3": 5e-2, "fp4": 5e-2}


def check_scores(gpu_row, ora_row, where=""):
    g = np.asarray(gpu_row, dtype=np.float64)
    o = np.asarray(ora_row, dtype=np.float64)
    gi, oi = np.isneginf(g), np.isneginf(o)
    assert np.array_equal(gi, oi), f"{where}: -inf pattern differs at {np.nonzero(gi != oi)[0][:10]}"
    fin = ~oi
    if not fin.any():
        return 0.0
    floor = 1e-3 * np.abs(o[fin]).max()
    tol = SCORE_RTOL * np.maximum(np.abs(o[fin]), floor)
    err = np.abs(g[fin] - o[fin])
    bad = err > tol
    assert not bad.any(), f"{where}: {bad.sum()} scores off, worst rel {(err / np.maximum(np.abs(o[fin]), floor)).max():.3g}"
    return float((err / np.maximum(np.abs(o[fin]), floor)).max())


def check_topk(gpu_ids, cand, ora_scores, K, where=""):
    """gpu_ids: the GPU's row (ids then -1); cand/ora_scores: the oracle's
    candidates and fp64 scores."""
    gpu_ids = np.asarray(gpu_ids)
    valid = gpu_ids[gpu_ids >= 0]
    n_exp = min(K, len(cand))
    assert len(valid) == n_exp, f"{where}: {len(valid)} ids, expected {n_exp}"
    assert np.all(gpu_ids[len(valid):] == -1), f"{where}: -1 padding not at the tail"
    assert len(np.unique(valid)) == len(valid), f"{where}: duplicate ids"
    score_of = dict(zip((int(c) for c in cand), ora_scores))
    assert all(int(v) in score_of for v in valid), f"{where}: id outside the candidates"
    ref = O.top_k(ora_scores, cand, K)
    if n_exp == 0:
        return 0
    kth = score_of[int(ref[-1])]
    diff = set(int(v) for v in valid) ^ set(int(r) for r in ref)
    band = SET_BAND * max(abs(kth), 1e-30)
    for d in diff:
        assert abs(score_of[d] - kth) <= band, f"{where}: id {d} score {score_of[d]} vs K-th {kth}"
    return len(diff)


def oracle_attention(shared, layer, b, ti, ids):
    """Oracle steps 7-10 (window, logits, sink softmax, inverse RoPE) on a
    given index set."""
    r = O.layer_query(shared, layer, b, ti, O.REUSE, prev_sel=np.asarray(ids, dtype=np.int64))
    return r["out"]


def entry_rows(shared, layer, b, ti, ids):
    """The dequantized rows one query attends to (its valid selected records
    and its window rows), for the scale of the attention bound."""
    ids = np.asarray(ids, dtype=np.int64)
    ids = ids[(ids >= 0) & (ids < shared["N"])]
    glob = O.dequant(shared["kv"][b][ids], None if shared.get("kv_scale") is None else shared["kv_scale"][b][ids],
                     shared.get("kv_format"))
    t = int(layer["q_pos"][b, ti])
    S = layer["swa"].shape[1]
    slots = O.window_positions(t, int(layer["W"])) % S
    loc = O.dequant(layer["swa"][b][slots], None if layer.get("swa_scale") is None else layer["swa_scale"][b][slots],
                    layer.get("swa_format"))
    return np.concatenate([glob, loc], 0)


def attn_tol(kv_dtype, rows):
    """Max-abs bound for one query's output (see the module docstring)."""
    rows = np.asarray(rows, dtype=np.float64)
    sigma = math.sqrt(float(np.mean(rows * rows))) if rows.size else 1.0
    return ATTN_TOL[kv_dtype] * min(1.0, sigma)


def check_attn(gpu_out, ora_out, tol, where=""):
    err = np.abs(np.asarray(gpu_out, dtype=np.float64) - ora_out).max()
    assert err <= tol, f"{where}: attention max-abs error {err:.3g} > {tol:.3g}"
    return float(err)


def check_attn_query(gpu_out, shared, layer, b, ti, ids, kv_dtype, where="", out_bf16=False):
    """Oracle attention on the GPU's index set, held to attn_tol (plus, for
    a bf16 output, the rounding of the exact value to bf16: half a unit in
    the last place of the slightly larger magnitude); returns (error, bound)."""
    ref = oracle_attention(shared, layer, b, ti, ids)
    tol = attn_tol(kv_dtype, entry_rows(shared, layer, b, ti, ids))
    if not out_bf16:
        return check_attn(gpu_out, ref, tol, where), tol
    err = np.abs(np.asarray(gpu_out, dtype=np.float64) - ref)
    bound = tol + bf16_half_ulp(np.abs(ref) + tol) * (1 + 1e-6)
    assert np.all(err <= bound), f"{where}: bf16 output off by {(err - bound).max():.3g} beyond its bound"
    return float(err.max()), tol


# ------------------------------------------------------------------ record construction

def e4m3_half_step(v):
    """Half the spacing of e4m3 values around |v| (subnormal spacing 2^-9)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def bf16_half_ulp(v):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 8)


def e2m1_half_step(v):
    a = np.abs(v)
    return 0.5 * np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))


def check_rounding(got, exact, scale, half_step, where, sat=None):
    """Every stored value is a nearest rounding of the exact one (within
    half a step of the format at that magnitude, plus float32 noise);
    values beyond the format's range saturate."""
    g = np.asarray(got, np.float64)
    x = np.asarray(exact, np.float64)
    v = x / scale
    tol = half_step(v) * scale * (1 + 1e-3) + 1e-6 * np.abs(x) + 1e-30
    if sat is not None:
        over = np.abs(v) > sat
        tol = np.where(over, np.abs(x) - sat * scale + tol, tol)
    bad = np.abs(g - x) > tol
    assert not bad.any(), f"{where}: {bad.sum()} values off, worst {np.abs(g - x)[bad].max():.3g}"


def check_compressed(kv_rows, kv_scale, k_rows, k_scale, x, w, kvf, kf, where=""):
    """Stored records and keys of n records against the oracle's exact
    records x [n][D] (before quantization) and W_ik w [D][Di].

    float32 records match element by element; quantized ones (scales
    included) are nearest roundings of x.  The keys are held to the exact
    keys x @ W_ik, moved by at most what the record rounding (eb, bounded
    from the oracle's values alone) and float32 accumulation allow, plus
    their own format's rounding."""
    n, D = x.shape
    Di = w.shape[1]
    w64 = np.asarray(w, np.float64)
    # eb: how far a correct storage of x may lie from x
    if kvf == "f32":
        got = np.asarray(kv_rows, np.float64)
        eb = np.full_like(x, 2e-5 * np.abs(x).max())
        assert np.all(np.abs(got - x) <= eb), f"{where} f32 records"
    elif kvf == "bf16":
        eb = bf16_half_ulp(x) * (1 + 1e-3) + 1e-6 * np.abs(x)
        check_rounding(O.dequant(kv_rows), x, 1.0, bf16_half_ulp, f"{where} bf16 records")
    elif kvf == "e4m3":
        so = np.abs(x).max(1) / 448
        assert np.allclose(kv_scale, so, rtol=1e-5), f"{where} e4m3 record scales"
        eb = e4m3_half_step(x / so[:, None]) * so[:, None] * (1 + 1e-3) + 1e-6 * np.abs(x)
        check_rounding(O.dequant(kv_rows, kv_scale), x, so[:, None], e4m3_half_step, f"{where} e4m3 records")
    else:
        go = np.repeat(np.abs(x.reshape(n, D // 16, 16)).max(-1) / 6, 16, -1)  # exact group scales
        hs = e4m3_half_step(go) * (1 + 1e-3) + 1e-7 * go
        gs = np.repeat(O.decode_e4m3(kv_rows[:, D // 2:]), 16, -1)   # the stored ones
        assert np.all(np.abs(gs - go) <= hs), f"{where} fp4 group scales"
        # any scale within [go - hs, go + hs] may have been chosen: the largest steps
        # and the earliest saturation bound the element error
        eb = e2m1_half_step(x / (go - hs)) * (go + hs) * (1 + 1e-3) + np.maximum(0, np.abs(x) - 6 * (go - hs))
        err = np.abs(O.dequant(kv_rows, None, "fp4") - x)
        assert np.all(err <= eb + 1e-6 * np.abs(x)), f"{where} fp4 records: worst {(err - eb).max():.3g} over"
    kexact = x @ w64
    kb = eb @ np.abs(w64) + 1e-5 * (np.abs(x) @ np.abs(w64))
    if kf == "f32":
        assert np.all(np.abs(k_rows - kexact) <= kb), f"{where} f32 keys"
    elif kf == "bf16":
        err = np.abs(O.dequant(k_rows) - kexact)
        assert np.all(err <= kb + bf16_half_ulp(kexact + np.sign(kexact) * kb) * (1 + 1e-3)), f"{where} bf16 keys"
    elif kf == "e4m3":
        so = np.abs(kexact).max(1) / 448
        sk = kb.max(1) / 448
        assert np.all(np.abs(k_scale - so) <= sk + 1e-5 * so), f"{where} e4m3 key scales"
        smax = (so + sk + 1e-5 * so)[:, None]
        err = np.abs(O.dequant(k_rows, k_scale) - kexact)
        assert np.all(err <= kb + e4m3_half_step((np.abs(kexact) + kb) / smax) * smax * (1 + 1e-3)), \
            f"{where} e4m3 keys"
    else:
        sc = O.decode_e8m0(k_scale)
        amax = np.abs(kexact.reshape(n, Di // 32, 32)).max(-1)
        amb = kb.reshape(n, Di // 32, 32).max(-1)
        lo = 2.0 ** (np.floor(np.log2(np.maximum(amax - amb, 1e-30))) - 2)
        hi = 2.0 ** (np.floor(np.log2(amax + amb)) - 2)
        assert np.all((sc >= lo) & (sc <= hi)), f"{where} mxfp4 block scales"
        s32 = np.repeat(sc, 32, -1)
        err = np.abs(O.dequant_mxfp4(k_rows, k_scale) - kexact)
        bound = kb + e2m1_half_step((np.abs(kexact) + kb) / s32) * s32 * (1 + 1e-3) + \
            np.maximum(0, np.abs(kexact) + kb - 6 * s32)
        assert np.all(err <= bound), f"{where} mxfp4 keys"
