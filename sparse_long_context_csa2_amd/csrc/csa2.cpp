// C ABI of the CSA2 layer: argument validation, workspace carving, kernel
// dispatch and the Full / Reindex / Reuse composition.  Host code only: it
// validates everything before enqueuing anything and never allocates,
// frees or synchronises.
#include "../../include/csa2.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_detail;
thread_local int g_detail_code = 0;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    g_detail_code = code;
    return code;
}

int hip_fail(int err, const char* what) {
    return fail(CSA2_EHIP, "%s: HIP error %d", what, err);
}

bool dtype_ok(int dt) { return dt >= CSA2_F32 && dt <= CSA2_MXFP4; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Tensor pointers must be 16-byte aligned (the kernels use 16-byte vector
// loads and stores and copy rows straight into LDS); workspaces 256-byte
// aligned (they are carved into 256-byte aligned parts).
bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

int check_align(const char* who, std::initializer_list<const void*> ptrs, const void* ws) {
    int i = 0;
    for (const void* p : ptrs) {
        if (p && misaligned(p, 16))
            return fail(CSA2_EINVAL, "%s: pointer argument %d (%p) is not 16-byte aligned", who, i, p);
        ++i;
    }
    if (ws && misaligned(ws, 256)) return fail(CSA2_EINVAL, "%s: workspace %p is not 256-byte aligned", who, ws);
    return CSA2_OK;
}

// e4m3 needs its per-row scales and MXFP4 its E8M0 block scales; FP4 rows
// carry their scales inline, and f32/bf16 have none.
int check_scale(const char* name, int dt, const void* scale) {
    if (!dtype_ok(dt)) return fail(CSA2_EINVAL, "%s: unknown dtype %d", name, dt);
    const bool needs = dt == CSA2_E4M3 || dt == CSA2_MXFP4;
    if (needs && !scale) return fail(CSA2_EINVAL, "%s: dtype %d needs its scale array", name, dt);
    if (!needs && scale) return fail(CSA2_EINVAL, "%s: scale array given for dtype %d, which has none", name, dt);
    return CSA2_OK;
}

// ---------------------------------------------------------------- indexer

int validate_index(const csa2::IndexArgs& a) {
    if (a.B < 1 || a.Tq < 1 || a.N < 1 || a.Hi < 1 || a.Di < 1 || a.m < 1)
        return fail(CSA2_EINVAL, "index_scores: sizes must be >= 1 (B=%d Tq=%d N=%d Hi=%d Di=%d m=%d)", a.B,
                    a.Tq, a.N, a.Hi, a.Di, a.m);
    if (!a.q_idx || !a.w || !a.k_idx || !a.q_pos || !a.scores)
        return fail(CSA2_EINVAL, "index_scores: null required pointer");
    if (a.q_dtype != CSA2_F32 && a.q_dtype != CSA2_BF16 && a.q_dtype != CSA2_MXFP4)
        return fail(dtype_ok(a.q_dtype) ? CSA2_EUNSUPPORTED : CSA2_EINVAL,
                    "index_scores: queries must be f32, bf16 or mxfp4");
    int e = check_align("index_scores",
                        {a.q_idx, a.q_scale, a.w, a.k_idx, a.k_scale, a.q_pos, a.n_rec, a.pool, a.scores}, nullptr);
    if (e) return e;
    e = check_scale("index_scores queries", a.q_dtype, a.q_scale);
    if (e) return e;
    e = check_scale("index_scores keys", a.k_dtype, a.k_scale);
    if (e) return e;
    if (a.k_dtype == CSA2_FP4)
        return fail(CSA2_EUNSUPPORTED, "index_scores: FP4 main-KV rows are not an indexer key format (use mxfp4)");
    if (a.q_dtype == CSA2_MXFP4 && a.k_dtype != CSA2_MXFP4)
        return fail(CSA2_EUNSUPPORTED, "index_scores: mxfp4 queries need mxfp4 keys");
    if ((a.q_dtype == CSA2_MXFP4 || a.k_dtype == CSA2_MXFP4) && !csa2::index_scores_mfma_ok(a))
        return fail(CSA2_EUNSUPPORTED, "index_scores: mxfp4 needs Hi=32, Di=128 (got Hi=%d Di=%d)", a.Hi, a.Di);
    if (a.pool) {
        if (a.P < 1 || a.blk < 1) return fail(CSA2_EINVAL, "index_scores: pool needs P >= 1 and blk >= 1");
        if (static_cast<long long>(a.P) * a.blk > (1LL << 30))
            return fail(CSA2_EINVAL, "index_scores: P*blk too large");
    } else if (a.P || a.blk) {
        return fail(CSA2_EINVAL, "index_scores: P/blk given without a pool");
    }
    if (!csa2::index_scores_mfma_ok(a)) {
        if (a.Hi > 64 || a.Di > 256 || a.Hi * a.Di > 8192)
            return fail(CSA2_EUNSUPPORTED, "index_scores: no kernel for Hi=%d Di=%d with these dtypes", a.Hi,
                        a.Di);
    }
    return CSA2_OK;
}

// ---------------------------------------------------------------- attention

int validate_attn(const csa2::AttnArgs& a) {
    if (a.B < 1 || a.Tq < 1 || a.H < 1 || a.D < 1 || a.N < 1 || a.K < 0 || a.S < 1 || a.W < 1)
        return fail(CSA2_EINVAL, "sparse_attn: bad sizes (B=%d Tq=%d H=%d D=%d N=%d K=%d S=%d W=%d)", a.B, a.Tq,
                    a.H, a.D, a.N, a.K, a.S, a.W);
    if (a.W > a.S) return fail(CSA2_EINVAL, "sparse_attn: window W=%d larger than ring S=%d", a.W, a.S);
    if (a.K > CSA2_MAX_K) return fail(CSA2_EINVAL, "sparse_attn: K=%d above %d", a.K, CSA2_MAX_K);
    if (!a.q || !a.kv || !a.swa || !a.q_pos || !a.sink || !a.out || (a.K > 0 && !a.idx))
        return fail(CSA2_EINVAL, "sparse_attn: null required pointer");
    if (a.q_dtype != CSA2_F32 && a.q_dtype != CSA2_BF16)
        return fail(dtype_ok(a.q_dtype) ? CSA2_EUNSUPPORTED : CSA2_EINVAL,
                    "sparse_attn: queries must be f32 or bf16");
    if (a.out_dtype != CSA2_F32 && a.out_dtype != CSA2_BF16)
        return fail(dtype_ok(a.out_dtype) ? CSA2_EUNSUPPORTED : CSA2_EINVAL,
                    "sparse_attn: the output must be f32 or bf16 (out_dtype=%d)", a.out_dtype);
    int e = check_align("sparse_attn",
                        {a.q, a.kv, a.kv_scale, a.idx, a.swa, a.swa_scale, a.q_pos, a.sink, a.out}, a.ws);
    if (e) return e;
    e = check_scale("sparse_attn kv", a.kv_dtype, a.kv_scale);
    if (e) return e;
    e = check_scale("sparse_attn swa", a.swa_dtype, a.swa_scale);
    if (e) return e;
    if (a.kv_dtype == CSA2_MXFP4 || a.swa_dtype == CSA2_MXFP4 || a.swa_dtype == CSA2_FP4)
        return fail(CSA2_EUNSUPPORTED, "sparse_attn: mxfp4 rows, and fp4 window rows, are not attention formats");
    if (a.kv_dtype == CSA2_FP4 && (a.swa_dtype != CSA2_E4M3 || !csa2::sparse_attn_mfma_ok(a)))
        return fail(CSA2_EUNSUPPORTED, "sparse_attn: fp4 records need e4m3 window rows and H=64, D=512");
    if (a.rope_dims < 0 || a.rope_dims > a.D || (a.rope_dims & 1))
        return fail(CSA2_EINVAL, "sparse_attn: rope_dims=%d must be even and <= D", a.rope_dims);
    if (!(a.rope_base > 0.f)) return fail(CSA2_EINVAL, "sparse_attn: rope_base must be > 0");
    if (!(a.sm_scale >= 0.f) || isinf(a.sm_scale)) return fail(CSA2_EINVAL, "sparse_attn: bad sm_scale");
    if (!csa2::sparse_attn_mfma_ok(a)) {
        const long long klist = a.dense_m ? a.N : a.K;  // longest list of records
        if (a.D > 1024 || 2LL * a.D + klist + a.W > 16384)
            return fail(CSA2_EUNSUPPORTED, "sparse_attn: no kernel for H=%d D=%d K=%lld W=%d with these dtypes",
                        a.H, a.D, klist, a.W);
    }
    return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_index_scores(int B, int Tq, int N, int Hi, int Di, int m, const void* q_idx, int q_dtype,
                      const void* q_scale, const float* w, const void* k_idx, const void* k_scale, int k_dtype,
                      const int64_t* q_pos, const int32_t* n_rec, const int32_t* pool, int P, int blk,
                      float* scores, void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    csa2::IndexArgs a;
    a.B = B; a.Tq = Tq; a.N = N; a.Hi = Hi; a.Di = Di; a.m = m;
    a.q_idx = q_idx; a.q_dtype = q_dtype; a.q_scale = q_scale; a.w = w; a.k_idx = k_idx; a.k_scale = k_scale;
    a.k_dtype = k_dtype; a.q_pos = q_pos; a.n_rec = n_rec; a.pool = pool; a.P = P; a.blk = blk;
    a.scores = scores;
    a.ncols = pool ? P * blk : N;
    int e = validate_index(a);
    if (e) return e;
    e = csa2::launch_index_scores(a, stream);
    return e ? hip_fail(e, "index_scores launch") : CSA2_OK;
}

size_t csa2_block_pool_workspace_bytes(int rows, int N, int blk) {
    if (rows < 1 || N < 1 || blk < 1) return 0;
    return csa2::block_pool_ws_bytes(rows, N, blk);
}

int csa2_block_pool(int rows, int N, int blk, int P, const float* scores, int32_t* pool, void* ws,
                    size_t ws_bytes, void* stream) {
    if (rows < 1 || N < 1 || blk < 1 || P < 1)
        return fail(CSA2_EINVAL, "block_pool: sizes must be >= 1 (rows=%d N=%d blk=%d P=%d)", rows, N, blk, P);
    if (P > CSA2_MAX_K) return fail(CSA2_EINVAL, "block_pool: P=%d above %d", P, CSA2_MAX_K);
    if (!scores || !pool) return fail(CSA2_EINVAL, "block_pool: null required pointer");
    if (int e = check_align("block_pool", {scores, pool}, ws)) return e;
    const size_t need = csa2::block_pool_ws_bytes(rows, N, blk);
    if (ws_bytes < need || (need && !ws))
        return fail(CSA2_EWORKSPACE, "block_pool: workspace %zu bytes, need %zu", ws_bytes, need);
    const int e = csa2::launch_block_pool(rows, N, blk, P, scores, pool, ws, ws_bytes, stream);
    return e ? hip_fail(e, "block_pool launch") : CSA2_OK;
}

size_t csa2_topk_workspace_bytes(int rows, int ncols, int K) {
    if (rows < 1 || ncols < 1 || K < 1) return 0;
    return csa2::topk_ws_bytes(rows, ncols, K);
}

int csa2_topk(int rows, int ncols, int K, const float* scores, const int32_t* pool, int P, int blk, int32_t* idx,
              void* ws, size_t ws_bytes, void* stream) {
    if (rows < 1 || ncols < 1 || K < 1)
        return fail(CSA2_EINVAL, "topk: sizes must be >= 1 (rows=%d ncols=%d K=%d)", rows, ncols, K);
    if (K > CSA2_MAX_K) return fail(CSA2_EINVAL, "topk: K=%d above %d", K, CSA2_MAX_K);
    if (ncols > csa2::kTopkMaxCols)
        return fail(CSA2_EUNSUPPORTED, "topk: ncols=%d above %d", ncols, csa2::kTopkMaxCols);
    if (!scores || !idx) return fail(CSA2_EINVAL, "topk: null required pointer");
    if (int e = check_align("topk", {scores, pool, idx}, ws)) return e;
    if (pool) {
        if (P < 1 || blk < 1 || static_cast<long long>(P) * blk != ncols)
            return fail(CSA2_EINVAL, "topk: pool mapping needs P*blk == ncols (P=%d blk=%d ncols=%d)", P, blk,
                        ncols);
    } else if (P || blk) {
        return fail(CSA2_EINVAL, "topk: P/blk given without a pool");
    }
    const size_t need = csa2::topk_ws_bytes(rows, ncols, K);
    if (ws_bytes < need || (need && !ws))
        return fail(CSA2_EWORKSPACE, "topk: workspace %zu bytes, need %zu", ws_bytes, need);
    csa2::TopkArgs a;
    a.rows = rows; a.ncols = ncols; a.K = K; a.scores = scores; a.pool = pool; a.P = P; a.blk = blk;
    a.idx = idx; a.sort_by_key = false; a.ws = ws; a.ws_bytes = ws_bytes;
    const int e = csa2::launch_topk(a, stream);
    return e ? hip_fail(e, "topk launch") : CSA2_OK;
}

size_t csa2_sparse_attn_workspace_bytes(int B, int Tq, int H, int D, int K, int W) {
    if (B < 1 || Tq < 1 || H < 1 || D < 1 || K < 0 || W < 1) return 0;
    return csa2::sparse_attn_ws_bytes(B, Tq, H, D, K, W);
}

static void fill_attn(csa2::AttnArgs& a, int B, int Tq, int H, int D, int N, int K, const void* q, int q_dtype,
                      const void* kv, const float* kv_scale, int kv_dtype, const int32_t* idx, const void* swa,
                      const float* swa_scale, int swa_dtype, int S, int W, const int64_t* q_pos,
                      const float* sink, float sm_scale, int rope_dims, float rope_base, void* out,
                      int out_dtype, void* ws, size_t ws_bytes) {
    a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.N = N; a.K = K;
    a.q = q; a.q_dtype = q_dtype; a.kv = kv; a.kv_scale = kv_scale; a.kv_dtype = kv_dtype; a.idx = idx;
    a.swa = swa; a.swa_scale = swa_scale; a.swa_dtype = swa_dtype; a.S = S; a.W = W; a.q_pos = q_pos;
    a.sink = sink; a.sm_scale = sm_scale; a.rope_dims = rope_dims; a.rope_base = rope_base; a.out = out;
    a.out_dtype = out_dtype; a.ws = ws; a.ws_bytes = ws_bytes;
}

int csa2_sparse_attn(int B, int Tq, int H, int D, int N, int K, const void* q, int q_dtype, const void* kv,
                     const float* kv_scale, int kv_dtype, const int32_t* idx, const void* swa,
                     const float* swa_scale, int swa_dtype, int S, int W, const int64_t* q_pos, const float* sink,
                     float sm_scale, int rope_dims, float rope_base, void* out, int out_dtype, void* ws,
                     size_t ws_bytes, void* stream) {
    csa2::AttnArgs a;
    fill_attn(a, B, Tq, H, D, N, K, q, q_dtype, kv, kv_scale, kv_dtype, idx, swa, swa_scale, swa_dtype, S, W,
              q_pos, sink, sm_scale, rope_dims, rope_base, out, out_dtype, ws, ws_bytes);
    int e = validate_attn(a);
    if (e) return e;
    const size_t need = csa2::sparse_attn_ws_bytes(B, Tq, H, D, K, W);
    if (ws_bytes < need || (need && !ws))
        return fail(CSA2_EWORKSPACE, "sparse_attn: workspace %zu bytes, need %zu", ws_bytes, need);
    e = csa2::launch_sparse_attn(a, stream);
    return e ? hip_fail(e, "sparse_attn launch") : CSA2_OK;
}

int csa2_sparse_attn_noalloc(int B, int Tq, int H, int D, int N, int K, const void* q, int q_dtype,
                             const void* kv, const float* kv_scale, int kv_dtype, const int32_t* idx,
                             const void* swa, const float* swa_scale, int swa_dtype, int S, int W,
                             const int64_t* q_pos, const float* sink, float sm_scale, int rope_dims,
                             float rope_base, void* out, int out_dtype, void* stream) {
    csa2::AttnArgs a;
    fill_attn(a, B, Tq, H, D, N, K, q, q_dtype, kv, kv_scale, kv_dtype, idx, swa, swa_scale, swa_dtype, S, W,
              q_pos, sink, sm_scale, rope_dims, rope_base, out, out_dtype, nullptr, 0);
    int e = validate_attn(a);
    if (e) return e;
    // splits taken only for parallelism give way to the static scratch size
    const size_t have = csa2::sparse_attn_scratch_bytes();
    a.part_cap = have;
    const size_t need = csa2::sparse_attn_ws_bytes(B, Tq, H, D, K, W, have);
    if (need > have)
        return fail(CSA2_EWORKSPACE,
                    "sparse_attn_noalloc: this shape needs %zu bytes of scratch, above the static %zu "
                    "(use csa2_sparse_attn with a workspace)", need, have);
    if (need) {
        int herr = 0;
        a.ws = csa2::sparse_attn_scratch(herr);
        if (!a.ws) return hip_fail(herr, "sparse_attn_noalloc: scratch address");
        a.ws_bytes = have;
    }
    e = csa2::launch_sparse_attn(a, stream);
    return e ? hip_fail(e, "sparse_attn_noalloc launch") : CSA2_OK;
}

size_t csa2_dense_attn_workspace_bytes(int B, int Tq, int H, int D, int N, int W) {
    if (B < 1 || Tq < 1 || H < 1 || D < 1 || N < 1 || W < 1) return 0;
    return csa2::dense_attn_ws_bytes(B, Tq, H, D, N, W);
}

int csa2_dense_attn(int B, int Tq, int H, int D, int N, int m, const int32_t* n_rec, const void* q, int q_dtype,
                    const void* kv, const float* kv_scale, int kv_dtype, const void* swa, const float* swa_scale,
                    int swa_dtype, int S, int W, const int64_t* q_pos, const float* sink, float sm_scale,
                    int rope_dims, float rope_base, void* out, int out_dtype, void* ws, size_t ws_bytes,
                    void* stream) {
    if (m < 1) return fail(CSA2_EINVAL, "dense_attn: compression ratio m=%d must be >= 1", m);
    if (int e = check_align("dense_attn", {n_rec}, nullptr)) return e;
    csa2::AttnArgs a;
    fill_attn(a, B, Tq, H, D, N, 0, q, q_dtype, kv, kv_scale, kv_dtype, nullptr, swa, swa_scale, swa_dtype, S, W,
              q_pos, sink, sm_scale, rope_dims, rope_base, out, out_dtype, ws, ws_bytes);
    a.dense_m = m;
    a.n_rec = n_rec;
    int e = validate_attn(a);
    if (e) return e;
    const size_t need = csa2::dense_attn_ws_bytes(B, Tq, H, D, N, W);
    if (ws_bytes < need || (need && !ws))
        return fail(CSA2_EWORKSPACE, "dense_attn: workspace %zu bytes, need %zu", ws_bytes, need);
    e = csa2::launch_sparse_attn(a, stream);
    return e ? hip_fail(e, "dense_attn launch") : CSA2_OK;
}

// ---------------------------------------------------------------- layer

struct LayerPlan {
    int rows, ncols;
    size_t off_scores, off_pool, off_topk, off_attn, total;
};

static int plan_layer(const csa2_layer_desc* d, LayerPlan& pl) {
    if (!d) return fail(CSA2_EINVAL, "layer: null descriptor");
    if (d->mode != CSA2_FULL && d->mode != CSA2_REINDEX && d->mode != CSA2_REUSE && d->mode != CSA2_HCA)
        return fail(CSA2_EINVAL, "layer: unknown mode %d", d->mode);
    if (d->B < 1 || d->Tq < 1 || d->N < 1 || d->m < 1)
        return fail(CSA2_EINVAL, "layer: sizes must be >= 1 (B=%d Tq=%d N=%d m=%d)", d->B, d->Tq, d->N, d->m);
    pl.rows = d->B * d->Tq;
    pl.ncols = d->N;
    if (d->mode == CSA2_HCA) {  // no selection: attention over every visible record
        if (int e = check_align("layer", {d->n_rec}, d->ws)) return e;
        pl.off_scores = pl.off_pool = pl.off_topk = pl.off_attn = 0;
        pl.total = align256(csa2::dense_attn_ws_bytes(d->B, d->Tq, d->H, d->D, d->N, d->W));
        return CSA2_OK;
    }
    if (d->K < 1 || d->K > CSA2_MAX_K) return fail(CSA2_EINVAL, "layer: K=%d outside 1..%d", d->K, CSA2_MAX_K);
    if (!d->idx_inout) return fail(CSA2_EINVAL, "layer: idx_inout is required");
    if (int e = check_align("layer", {d->idx_inout, d->pool_inout}, d->ws)) return e;
    const bool scores_needed = d->mode != CSA2_REUSE;
    if (d->mode == CSA2_FULL && d->pool_inout) {
        if (d->blk < 1 || d->P < 1 || d->P > CSA2_MAX_K)
            return fail(CSA2_EINVAL, "layer: pool needs blk >= 1 and 1 <= P <= %d", CSA2_MAX_K);
    }
    if (d->mode == CSA2_REINDEX && d->pool_inout) {
        if (d->blk < 1 || d->P < 1 || static_cast<long long>(d->P) * d->blk > (1LL << 30))
            return fail(CSA2_EINVAL, "layer: pool needs blk >= 1 and P >= 1");
        pl.ncols = d->P * d->blk;
    }
    if (scores_needed && pl.ncols > csa2::kTopkMaxCols)
        return fail(CSA2_EUNSUPPORTED, "layer: %d columns to select from, above %d", pl.ncols, csa2::kTopkMaxCols);
    size_t off = 0;
    pl.off_scores = off;
    if (scores_needed) off += align256(static_cast<size_t>(pl.rows) * pl.ncols * sizeof(float));
    pl.off_pool = off;
    if (d->mode == CSA2_FULL && d->pool_inout) off += align256(csa2::block_pool_ws_bytes(pl.rows, d->N, d->blk));
    pl.off_topk = off;
    if (scores_needed) off += align256(csa2::topk_ws_bytes(pl.rows, pl.ncols, d->K));
    pl.off_attn = off;
    off += align256(csa2::sparse_attn_ws_bytes(d->B, d->Tq, d->H, d->D, d->K, d->W));
    pl.total = off;
    return CSA2_OK;
}

size_t csa2_workspace_bytes(const csa2_layer_desc* desc) {
    LayerPlan pl;
    if (plan_layer(desc, pl)) return 0;
    return pl.total;
}

int csa2_layer(const csa2_layer_desc* d, void* stream) {
    LayerPlan pl;
    int e = plan_layer(d, pl);
    if (e) return e;
    if (d->mode == CSA2_HCA)
        return csa2_dense_attn(d->B, d->Tq, d->H, d->D, d->N, d->m, d->n_rec, d->q, d->q_dtype, d->kv, d->kv_scale,
                               d->kv_dtype, d->swa, d->swa_scale, d->swa_dtype, d->S, d->W, d->q_pos, d->sink,
                               d->sm_scale, d->rope_dims, d->rope_base, d->out, d->out_dtype, d->ws, d->ws_bytes,
                               stream);
    csa2::IndexArgs ia;
    const bool scoring = d->mode != CSA2_REUSE;
    const bool pooled = d->mode == CSA2_REINDEX && d->pool_inout;
    float* scores = reinterpret_cast<float*>(static_cast<uint8_t*>(d->ws) + pl.off_scores);
    if (scoring) {
        ia.B = d->B; ia.Tq = d->Tq; ia.N = d->N; ia.Hi = d->Hi; ia.Di = d->Di; ia.m = d->m;
        ia.q_idx = d->q_idx; ia.q_dtype = d->q_idx_dtype; ia.q_scale = d->q_idx_scale; ia.w = d->w;
        ia.k_idx = d->k_idx;
        ia.k_scale = d->k_scale; ia.k_dtype = d->k_dtype; ia.q_pos = d->q_pos; ia.n_rec = d->n_rec;
        ia.pool = pooled ? d->pool_inout : nullptr;
        ia.P = pooled ? d->P : 0;
        ia.blk = pooled ? d->blk : 0;
        ia.scores = scores;
        ia.ncols = pl.ncols;
        e = validate_index(ia);
        if (e) return e;
    }
    csa2::AttnArgs aa;
    fill_attn(aa, d->B, d->Tq, d->H, d->D, d->N, d->K, d->q, d->q_dtype, d->kv, d->kv_scale, d->kv_dtype,
              d->idx_inout, d->swa, d->swa_scale, d->swa_dtype, d->S, d->W, d->q_pos, d->sink, d->sm_scale,
              d->rope_dims, d->rope_base, d->out, d->out_dtype, static_cast<uint8_t*>(d->ws) + pl.off_attn,
              d->ws_bytes > pl.off_attn ? d->ws_bytes - pl.off_attn : 0);
    e = validate_attn(aa);
    if (e) return e;
    if (pl.total && (!d->ws || d->ws_bytes < pl.total))
        return fail(CSA2_EWORKSPACE, "layer: workspace %zu bytes, need %zu", d->ws_bytes, pl.total);

    if (scoring) {
        e = csa2::launch_index_scores(ia, stream);
        if (e) return hip_fail(e, "layer: index_scores launch");
        if (d->mode == CSA2_FULL && d->pool_inout) {
            e = csa2::launch_block_pool(pl.rows, d->N, d->blk, d->P, scores, d->pool_inout,
                                        static_cast<uint8_t*>(d->ws) + pl.off_pool,
                                        csa2::block_pool_ws_bytes(pl.rows, d->N, d->blk), stream);
            if (e) return hip_fail(e, "layer: block_pool launch");
        }
        csa2::TopkArgs ta;
        ta.rows = pl.rows; ta.ncols = pl.ncols; ta.K = d->K; ta.scores = scores;
        ta.pool = pooled ? d->pool_inout : nullptr;
        ta.P = pooled ? d->P : 0;
        ta.blk = pooled ? d->blk : 0;
        ta.idx = d->idx_inout; ta.sort_by_key = false;
        ta.ws = static_cast<uint8_t*>(d->ws) + pl.off_topk;
        ta.ws_bytes = csa2::topk_ws_bytes(pl.rows, pl.ncols, d->K);
        e = csa2::launch_topk(ta, stream);
        if (e) return hip_fail(e, "layer: topk launch");
    }
    e = csa2::launch_sparse_attn(aa, stream);
    return e ? hip_fail(e, "layer: sparse_attn launch") : CSA2_OK;
}

int csa2_compress(int B, int T, int D, int m, int Di, const void* c, const void* z, int in_dtype, const int64_t* t0,
                  const float* gain, float eps, int rope_dims, float rope_base, const void* w_ik, int w_dtype,
                  int N_out, void* kv, float* kv_scale, int kv_dtype, void* k_idx, void* k_scale, int k_dtype,
                  void* stream) {
    if (B < 1 || T < 1 || m < 1 || N_out < 1 || T % m)
        return fail(CSA2_EINVAL, "compress: need B, T, m, N_out >= 1 and T a multiple of m (B=%d T=%d m=%d N_out=%d)",
                    B, T, m, N_out);
    if (!c || !z || !t0 || !gain || !w_ik || !kv || !k_idx)
        return fail(CSA2_EINVAL, "compress: null required pointer");
    if (int e = check_align("compress", {c, z, t0, gain, w_ik, kv, kv_scale, k_idx, k_scale}, nullptr)) return e;
    if ((in_dtype != CSA2_F32 && in_dtype != CSA2_BF16) || (w_dtype != CSA2_F32 && w_dtype != CSA2_BF16))
        return fail(dtype_ok(in_dtype) && dtype_ok(w_dtype) ? CSA2_EUNSUPPORTED : CSA2_EINVAL,
                    "compress: token rows and W_ik must be f32 or bf16");
    if (kv_dtype == CSA2_MXFP4 || k_dtype == CSA2_FP4)
        return fail(CSA2_EUNSUPPORTED, "compress: records are f32/bf16/e4m3/fp4, keys f32/bf16/e4m3/mxfp4");
    if (int e = check_scale("compress records", kv_dtype, kv_scale)) return e;
    if (int e = check_scale("compress keys", k_dtype, k_scale)) return e;
    if (D != 128 && D != 256 && D != 512 && D != 1024)
        return fail(CSA2_EUNSUPPORTED, "compress: D=%d not in {128, 256, 512, 1024}", D);
    if (Di < 64 || Di > 256 || Di % 64)
        return fail(CSA2_EUNSUPPORTED, "compress: Di=%d must be 64, 128, 192 or 256", Di);
    if (k_dtype == CSA2_MXFP4 && Di % 128)  // whole MX blocks and byte pairs per lane
        return fail(CSA2_EUNSUPPORTED, "compress: mxfp4 keys need Di = 128 or 256 (got %d)", Di);
    if (rope_dims < 0 || rope_dims > D || (rope_dims & 1))
        return fail(CSA2_EINVAL, "compress: rope_dims=%d must be even and <= D", rope_dims);
    if (!(rope_base > 0.f)) return fail(CSA2_EINVAL, "compress: rope_base must be > 0");
    if (!(eps >= 0.f) || isinf(eps)) return fail(CSA2_EINVAL, "compress: bad eps");
    csa2::CompressArgs a;
    a.B = B; a.T = T; a.D = D; a.m = m; a.Di = Di; a.N_out = N_out;
    a.c = c; a.z = z; a.in_dtype = in_dtype; a.t0 = t0; a.gain = gain; a.eps = eps;
    a.rope_dims = rope_dims; a.rope_base = rope_base; a.w_ik = w_ik; a.w_dtype = w_dtype;
    a.kv = kv; a.kv_scale = kv_scale; a.kv_dtype = kv_dtype; a.k_idx = k_idx; a.k_scale = k_scale; a.k_dtype = k_dtype;
    const int e = csa2::launch_compress(a, stream);
    return e ? hip_fail(e, "compress launch") : CSA2_OK;
}

int csa2_group(const csa2_layer_desc* layers, int n_layers, void* stream) {
    if (!layers || n_layers < 1) return fail(CSA2_EINVAL, "group: need at least one layer descriptor");
    // every layer is validated before anything is enqueued
    for (int i = 0; i < n_layers; ++i) {
        LayerPlan pl;
        int e = plan_layer(&layers[i], pl);
        if (e) return e;
        if (pl.total && (!layers[i].ws || layers[i].ws_bytes < pl.total))
            return fail(CSA2_EWORKSPACE, "group: layer %d workspace %zu bytes, need %zu", i, layers[i].ws_bytes,
                        pl.total);
    }
    for (int i = 0; i < n_layers; ++i) {
        const int e = csa2_layer(&layers[i], stream);
        if (e) return e;
    }
    return CSA2_OK;
}

const char* csa2_status_str(int status) {
    if (status != CSA2_OK && status == g_detail_code && !g_detail.empty()) return g_detail.c_str();
    switch (status) {
        case CSA2_OK: return "ok";
        case CSA2_EINVAL: return "invalid argument";
        case CSA2_EUNSUPPORTED: return "unsupported shape or dtype combination";
        case CSA2_EWORKSPACE: return "workspace missing or too small";
        case CSA2_EHIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

const char* csa2_version(void) { return "csa2-gfx950 0.1"; }

}  // extern "C"
