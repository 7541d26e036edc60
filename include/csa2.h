/*
 * csa2.h -- C ABI of the MI355X (gfx950) CSA2 sparse-attention layer.
 *
 * One CSA2 layer separates three operations: creating memory, selecting
 * positions and attending to those positions ("DeepSeek-V4.1-Flash
 * explained", section 2 "CSA2: share memory without copying the answer").
 * This library covers writing that memory (csa2_compress), selection and
 * attention:
 *
 *   csa2_compress      records and indexer keys from token rows
 *   csa2_index_scores  lightning-indexer scores with causal visibility
 *   csa2_block_pool    hierarchical block-max candidate pool
 *   csa2_topk          Top-K record addresses (lower record id wins ties)
 *   csa2_sparse_attn   shared-latent MQA over selected records + SWA window,
 *                      per-head sink, inverse RoPE on the output
 *   csa2_layer         one layer in Full, Reindex or Reuse mode
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to a dense row-major array with
 *   the shape given in brackets; pointers must be 16-byte aligned and
 *   workspaces 256-byte aligned (a misaligned one is refused with
 *   CSA2_EINVAL before anything is enqueued).
 * - Storage dtypes (csa2_dtype): CSA2_F32 = IEEE float32, CSA2_BF16 =
 *   bfloat16 (uint16 bit patterns), CSA2_E4M3 = OCP fp8 e4m3fn codes with
 *   one float32 scale per row (value = decode(code) * scale[row]).  Scales
 *   are finite and >= 0, as max|x|/448 is; the indexer may apply a key
 *   row's scale after the ReLU.
 *   CSA2_FP4 = the FP4 main-KV row ("DeepSeek-V4.1-Flash explained",
 *   section 7: each group of 16 channels holds 16 four-bit E2M1 values and
 *   one E4M3 scale, 72 bits, so a 512-channel row takes 288 bytes): a row
 *   of D channels is D/2 code bytes (channel 2j in the low nibble of byte
 *   j) followed by D/16 E4M3 scale bytes; value = E2M1(code) * scale of its
 *   group; no separate scale array.  Attention rows only, with E4M3 window
 *   rows (the local cache stays FP8).
 *   CSA2_MXFP4 = OCP MXFP4 (the indexer's query and key format, same
 *   section): packed E2M1 codes [..][n/2] in the tensor and one E8M0 scale
 *   byte (2^(b-127)) per 32 elements [..][n/32] in its scale argument.
 *   Indexer queries and keys only.
 * - Positions are 0-based absolute token positions (int64).  Record s of
 *   a cache compressed at ratio m covers tokens m*s .. m*s+m-1 and is
 *   visible to a query at t only if m*s+m-1 <= t and s < n_rec ("DeepSeek V4
 *   Inside: One Token Through Every Block", section "How does CSA compress 8
 *   tokens into 4 KV entries?": an entry is visible only if all its tokens
 *   are at or before the query).
 * - The caller owns every buffer.  The library never allocates, frees or
 *   synchronises, keeps no pointer after returning and has no global state
 *   (except the static scratch of csa2_sparse_attn_noalloc); calls on
 *   different streams are independent.  `stream` is a
 *   hipStream_t passed as void* (NULL = the default stream).  Work is only
 *   enqueued: results are ready after the caller synchronises the stream.
 * - `ws`/`ws_bytes` is a caller-provided device workspace of at least the
 *   size the matching *_workspace_bytes function returns (it may be NULL
 *   when that size is 0).  Its contents on entry do not matter.
 * - Errors: every argument is validated on the host before anything is
 *   enqueued; on an error nothing is launched and the return value is
 *   negative.  csa2_status_str() gives a message (thread-local detail of
 *   the last error when one was recorded on this thread).
 * - Device code never dereferences an index outside [0, N): such entries
 *   (including the -1 padding) are skipped.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_OK 0
#define CSA2_EINVAL (-1)       /* null required pointer, bad size, bad combination */
#define CSA2_EUNSUPPORTED (-2) /* valid request with no kernel instance */
#define CSA2_EWORKSPACE (-3)   /* workspace missing or too small */
#define CSA2_EHIP (-4)         /* a HIP launch failed */

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1, CSA2_E4M3 = 2, CSA2_FP4 = 3, CSA2_MXFP4 = 4 } csa2_dtype;
typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2, CSA2_HCA = 3 } csa2_mode;

/* Largest K accepted by csa2_topk and csa2_layer. */
#define CSA2_MAX_K 2048

/* ------------------------------------------------------------------------
 * csa2_index_scores -- lightning-indexer scores.
 *
 *   I[b,t,s] = sum_h w[b,t,h] * max(0, q_idx[b,t,h,:] . k[b,s,:])
 *
 * Rectified query-key products combined over weighted indexer heads
 * ("DeepSeek V4.1-Flash. Every layer, connected.", caption "The global and
 * index paths"; "DeepSeek V4 Inside", Fig. 10).  Invisible records score
 * -INFINITY (the selection is causal).  Arithmetic: products of the stored
 * values accumulated in float32; e4m3 keys are applied as code*scale.
 *
 * Inputs
 *   B, Tq      sequences and query tokens per sequence (>= 1)
 *   N          records per sequence in k_idx (>= 1)
 *   Hi, Di     indexer heads and head dim (1..64, 1..256)
 *   m          compression ratio (>= 1): tokens per record
 *   q_idx      [B][Tq][Hi][Di]  q_dtype in {F32, BF16, MXFP4}
 *   q_scale    MXFP4 queries: [B][Tq][Hi][Di/32] E8M0 bytes; else NULL
 *   w          [B][Tq][Hi] float32 head weights
 *   k_idx      [B][N][Di]       k_dtype in {F32, BF16, E4M3, MXFP4}
 *   k_scale    E4M3: [B][N] float32; MXFP4: [B][N][Di/32] E8M0 bytes;
 *              NULL otherwise.  MXFP4 needs Hi = 32, Di = 128, and MXFP4
 *              queries need MXFP4 keys.
 *   q_pos      [B][Tq] int64 absolute query positions
 *   n_rec      [B] int32 valid record counts (<= N), or NULL for N
 *   pool, P, blk
 *              NULL/0/0 scores every record column s in [0, N).
 *              Otherwise [B][Tq][P] int32 block ids (-1 = empty slot) and
 *              the output has P*blk columns: column c is record
 *              pool[b,t,c/blk]*blk + c%blk ("DeepSeek-V4.1-Flash explained",
 *              section 3: later indexers search only the candidate pool).
 * Output
 *   scores     [B][Tq][ncols] float32, ncols = N or P*blk
 * Workspace: none (ws may be NULL).
 * ------------------------------------------------------------------------ */
int csa2_index_scores(int B, int Tq, int N, int Hi, int Di, int m,
                      const void* q_idx, int q_dtype, const void* q_scale, const float* w,
                      const void* k_idx, const void* k_scale, int k_dtype,
                      const int64_t* q_pos, const int32_t* n_rec,
                      const int32_t* pool, int P, int blk,
                      float* scores, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa2_block_pool -- hierarchical candidate pool.
 *
 * Records are grouped into blocks of `blk` consecutive ids; a block scores
 * the maximum of its members' scores; the P best blocks are kept ("DeepSeek
 * V4.1-Flash. Every layer, connected.", hierarchy caption; "Create DeepSeek
 * from scratch", lesson 07 "Hierarchical indexing").  Blocks whose members
 * are all -INFINITY (not visible) are never kept.
 *
 * Inputs
 *   rows       number of score rows (B*Tq)
 *   N          columns per row; blocks cover [b*blk, min((b+1)*blk, N))
 *   blk, P     block size (>= 1) and blocks kept (1..CSA2_MAX_K)
 *   scores     [rows][N] float32 (as written by csa2_index_scores)
 * Output
 *   pool       [rows][P] int32 block ids ordered by (block score desc,
 *              block id asc); -1 pads when fewer blocks qualify.
 * Workspace: csa2_block_pool_workspace_bytes(rows, N, blk).
 * ------------------------------------------------------------------------ */
int csa2_block_pool(int rows, int N, int blk, int P, const float* scores,
                    int32_t* pool, void* ws, size_t ws_bytes, void* stream);
size_t csa2_block_pool_workspace_bytes(int rows, int N, int blk);

/* ------------------------------------------------------------------------
 * csa2_topk -- Top-K record addresses.
 *
 * Returns the ADDRESSES of the K best records, never their scores ("Create
 * DeepSeek from scratch", lesson 06 worked example: keep the positions,
 * then retrieve the rows).  Order of preference: score descending, then
 * record id ascending.  -INFINITY and NaN scores are never selected.
 *
 * Inputs
 *   rows, ncols, K  (K in 1..CSA2_MAX_K; ncols up to 2^24, else
 *              CSA2_EUNSUPPORTED)
 *   scores     [rows][ncols] float32
 *   pool, P, blk
 *              NULL/0/0: column c is record c.  Otherwise [rows][P] int32
 *              block ids and ncols == P*blk: column c is record
 *              pool[row][c/blk]*blk + c%blk (ties then compare these ids).
 * Output
 *   idx        [rows][K] int32: the min(K, #selectable) chosen record ids
 *              in ascending COLUMN order (a set; deterministic), then -1.
 * Workspace: csa2_topk_workspace_bytes(rows, ncols, K).
 * ------------------------------------------------------------------------ */
int csa2_topk(int rows, int ncols, int K, const float* scores,
              const int32_t* pool, int P, int blk, int32_t* idx,
              void* ws, size_t ws_bytes, void* stream);
size_t csa2_topk_workspace_bytes(int rows, int ncols, int K);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn -- shared-latent attention over selected records plus
 * the local sliding window, with a per-head sink and inverse output RoPE.
 *
 * For query (b,t) at position p = q_pos[b,t] and head h, the entries are
 * the selected global records kv[b, idx[b,t,k]] (k < K, idx in [0,N)) and
 * the window rows swa[b, (p-W+1 .. p) mod S] (positions >= 0 only); every
 * entry serves as both key and value ("DeepSeek V4 Inside", Fig. 11: the
 * compressed entry is both K and V; window and record share one softmax):
 *
 *   z_j   = sm_scale * q[b,t,h,:] . x_j
 *   ctx_h = sum_j exp(z_j) x_j / (sum_j exp(z_j) + exp(sink[h]))
 *
 * (the sink enters the denominator only, "DeepSeek V4 Inside", eq. (27)),
 * then the last `rope_dims` channels of ctx_h are rotated by position -p
 * in adjacent pairs (D-r+2j, D-r+2j+1) with angle p*rope_base^(-2j/r)
 * ("DeepSeek V4.1-Flash. Every layer, connected.", caption "The query and
 * output paths"; "DeepSeek V4 Inside", Fig. 12).  Queries and caches are
 * post-RoPE.
 *
 * Inputs
 *   B, Tq, H, D, N, K  sizes (K in 0..CSA2_MAX_K; K = 0 means window only)
 *   q          [B][Tq][H][D]  q_dtype in {F32, BF16}
 *   kv         [B][N][D]      kv_dtype in {F32, BF16, E4M3, FP4}; kv_scale
 *                             [B][N] for E4M3, NULL otherwise (FP4 rows are
 *                             [B][N][D/2 + D/16] bytes with inline scales and
 *                             need E4M3 window rows, H = 64, D = 512)
 *   idx        [B][Tq][K] int32 record ids (-1 or out of range = empty)
 *   swa        [B][S][D]      ring of local rows: position p lives in slot
 *                             p mod S; swa_dtype like kv; swa_scale [B][S]
 *   S, W       ring slots and window length (1 <= W <= S)
 *   q_pos      [B][Tq] int64
 *   sink       [H] float32 sink logits (not multiplied by sm_scale)
 *   sm_scale   logit scale; 0 means 1/sqrt(D)
 *   rope_dims  even, 0..D; rope_base > 0
 * Output
 *   out        [B][Tq][H][D] in out_dtype: CSA2_F32, or CSA2_BF16 (the
 *              float32 result rounded to nearest even; half the bytes of
 *              the largest write of a prefill step)
 * Workspace: csa2_sparse_attn_workspace_bytes(B, Tq, H, D, K, W).
 * ------------------------------------------------------------------------ */
int csa2_sparse_attn(int B, int Tq, int H, int D, int N, int K,
                     const void* q, int q_dtype,
                     const void* kv, const float* kv_scale, int kv_dtype,
                     const int32_t* idx,
                     const void* swa, const float* swa_scale, int swa_dtype,
                     int S, int W, const int64_t* q_pos, const float* sink,
                     float sm_scale, int rope_dims, float rope_base,
                     void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream);
size_t csa2_sparse_attn_workspace_bytes(int B, int Tq, int H, int D, int K, int W);

/* ------------------------------------------------------------------------
 * csa2_dense_attn -- heavily compressed attention (HCA): the same shared-
 * latent MQA, window, sink and inverse output RoPE as csa2_sparse_attn,
 * with no indexer and no selection: every visible compressed record is an
 * entry ("DeepSeek V4 Inside: One Token Through Every Block", section
 * "What does HCA change?": dense attention over the n/m' compressed
 * entries plus the window; 8192 + 128 entries per query at 1,048,576
 * tokens and m' = 128).
 *
 * For query (b,t) at position p = q_pos[b,t] the entries are the records
 * s = 0 .. v-1 with v = min(n_rec[b], floor((p+1)/m)) (record s covers
 * tokens m*s .. m*s+m-1 and is visible once all of them are <= p), then the
 * window rows as in csa2_sparse_attn.
 *
 * Inputs: as csa2_sparse_attn, without idx/K, plus
 *   m          compression ratio of the records (>= 1)
 *   n_rec      [B] int32 records written per sequence (<= N), or NULL for N
 *   N          records per sequence in kv; N + W <= 73728 for the 64x512
 *              kernels
 * Output
 *   out        [B][Tq][H][D] in out_dtype (CSA2_F32 or CSA2_BF16)
 * Workspace: csa2_dense_attn_workspace_bytes(B, Tq, H, D, N, W).
 * ------------------------------------------------------------------------ */
int csa2_dense_attn(int B, int Tq, int H, int D, int N, int m, const int32_t* n_rec,
                    const void* q, int q_dtype,
                    const void* kv, const float* kv_scale, int kv_dtype,
                    const void* swa, const float* swa_scale, int swa_dtype,
                    int S, int W, const int64_t* q_pos, const float* sink,
                    float sm_scale, int rope_dims, float rope_base,
                    void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream);
size_t csa2_dense_attn_workspace_bytes(int B, int Tq, int H, int D, int N, int W);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn_noalloc -- csa2_sparse_attn without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as csa2_sparse_attn.
 *
 * It allocates nothing: when a shape needs scratch (the split partials of
 * decode shapes with fewer than 32 queries), it uses a 6 MiB array that
 * the library holds in each GPU's memory for the life of the process.
 * Where the workspace call would split a shape's queries into more
 * partials than that (up to 8 MiB: at most 64 partials of 128 KiB, e.g.
 * 8 queries in 8 splits or 16 in 4), it takes fewer splits (those only add
 * parallelism): same result to the attention bound, not bit for bit.  CSA2_EWORKSPACE remains for a shape
 * whose entry lists alone would need more.  All calls on one GPU share
 * that array, so calls that overlap on one GPU (other streams, other
 * threads) race; calls on different GPUs do not.  The first call on a
 * device looks the array up (no allocation).
 * ------------------------------------------------------------------------ */
int csa2_sparse_attn_noalloc(int B, int Tq, int H, int D, int N, int K,
                             const void* q, int q_dtype,
                             const void* kv, const float* kv_scale, int kv_dtype,
                             const int32_t* idx,
                             const void* swa, const float* swa_scale, int swa_dtype,
                             int S, int W, const int64_t* q_pos, const float* sink,
                             float sm_scale, int rope_dims, float rope_base,
                             void* out, int out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * csa2_layer -- one CSA2 layer in one of the three sharing modes
 * ("DeepSeek-V4.1-Flash explained", section 2, mode table; "Create DeepSeek
 * from scratch", lesson "How CSA2 compresses, shares, and selects attention
 * memory"):
 *
 *   FULL     scores every visible record, optionally builds the block pool
 *            (pool_inout != NULL), takes a fresh Top-K over all visible
 *            records, attends.  Writes idx_inout (and pool_inout).
 *   REINDEX  scores the records of the pool in pool_inout when it is not
 *            NULL (else every visible record) with this layer's own indexer
 *            queries over the shared keys, takes a fresh Top-K, attends.
 *            Writes idx_inout.
 *   REUSE    runs no indexer; attends over the index set in idx_inout (left
 *            by the preceding Full or Reindex layer) with this layer's own
 *            query, window rows and sink.
 *   HCA      a heavily compressed attention layer: no indexer and no
 *            selection; csa2_dense_attn over every visible record of kv
 *            at ratio m (K, idx_inout, blk, P, pool_inout and the indexer
 *            fields are ignored).
 *
 * Every mode computes a fresh output with the layer's own query.
 * ------------------------------------------------------------------------ */
typedef struct csa2_layer_desc {
    int mode;            /* csa2_mode */
    int B, Tq;           /* sequences, query tokens per sequence */
    /* shared store (built by the sharing group's Full layer) */
    int N, m;            /* records per sequence, tokens per record */
    const int32_t* n_rec;           /* [B] or NULL (= N) */
    const void* k_idx;              /* [B][N][Di] indexer keys */
    const void* k_scale;            /* E4M3: [B][N] float; MXFP4: [B][N][Di/32] E8M0; else NULL */
    int k_dtype;
    const void* kv;                 /* [B][N][D] shared latent (K = V); FP4: [B][N][D/2 + D/16] */
    const float* kv_scale;          /* [B][N] for E4M3, else NULL */
    int kv_dtype;
    /* this layer's indexer */
    int Hi, Di;
    const void* q_idx;              /* [B][Tq][Hi][Di] */
    int q_idx_dtype;
    const void* q_idx_scale;        /* MXFP4: [B][Tq][Hi][Di/32] E8M0; else NULL */
    const float* w;                 /* [B][Tq][Hi] */
    /* this layer's attention */
    int H, D;
    const void* q;                  /* [B][Tq][H][D] post-RoPE */
    int q_dtype;
    const void* swa;                /* [B][S][D] local ring */
    const float* swa_scale;         /* [B][S] for E4M3, else NULL */
    int swa_dtype;
    int S, W;
    const float* sink;              /* [H] */
    float sm_scale;                 /* 0 = 1/sqrt(D) */
    int rope_dims;
    float rope_base;
    const int64_t* q_pos;           /* [B][Tq] */
    /* selection */
    int K;
    int32_t* idx_inout;             /* [B][Tq][K] */
    int blk, P;
    int32_t* pool_inout;            /* [B][Tq][P] or NULL */
    /* output and scratch */
    void* out;                      /* [B][Tq][H][D] in out_dtype */
    void* ws;
    size_t ws_bytes;
    int out_dtype;                  /* CSA2_F32 (0, the default) or CSA2_BF16 */
} csa2_layer_desc;

int csa2_layer(const csa2_layer_desc* desc, void* stream);

/* Workspace csa2_layer needs for this descriptor (pointers are ignored). */
size_t csa2_workspace_bytes(const csa2_layer_desc* desc);

/* ------------------------------------------------------------------------
 * csa2_compress -- record construction and the cache write.
 *
 * Turns token rows into global records and their indexer keys ("Create
 * DeepSeek from scratch", "How CSA2 compresses, shares, and selects
 * attention memory": above ratio 1, consecutive token representations are
 * pooled with learned, channel-wise softmax gates; at ratio 1 a normalized
 * projection; "DeepSeek-V4.1-Flash explained", section 2: CSA2 removes
 * overlapping compression groups and derives indexer keys from main KV).
 * For record s of sequence b (token rows m*s .. m*s+m-1, absolute
 * positions t0[b] + m*s ..):
 *
 *   x[d]  = sum_i softmax_i(z[i][d]) * c[i][d]       over the block's rows
 *   x     = x / sqrt(mean_d x[d]^2 + eps) * gain
 *   x     = RoPE of the last rope_dims channels at position t0[b]+m*s+m-1
 *           (adjacent pairs, angle pos*rope_base^(-2j/r), as the output
 *           rotation of csa2_sparse_attn undoes)
 *   kv    = x stored in kv_dtype (quantized after RoPE, the FP4 lesson's
 *           "Quantize after RoPE")
 *   k_idx = (stored kv row, dequantized) @ W_ik, stored in k_dtype
 *
 * The token projections c = h W_c and z = h W_z are ordinary linear layers
 * and are inputs here.  Quantizers round to nearest, ties to even,
 * saturating: e4m3 rows take scale max|x|/448; FP4 groups of 16 take the
 * E4M3 scale nearest max|x|/6; MXFP4 blocks of 32 take 2^(floor(log2
 * max|x|) - 2).
 *
 * Inputs
 *   B, T, m    sequences, token rows per sequence (a multiple of m), ratio
 *   D, Di      latent width (128, 256, 512 or 1024) and key width (64, 128,
 *              192 or 256)
 *   c, z       [B][T][D] candidate latents and gate logits, in_dtype in
 *              {F32, BF16}
 *   t0         [B] int64 absolute position of token row 0 (a multiple of m;
 *              its records go to cache rows t0/m, t0/m + 1, ...; rows at or
 *              past N_out, or a negative t0, are not written)
 *   gain       [D] float32; eps >= 0
 *   w_ik       [D][Di] in w_dtype {F32, BF16}
 *   N_out      records per sequence in the caches
 * Outputs
 *   kv         [B][N_out][D] in kv_dtype {F32, BF16, E4M3, FP4} (FP4:
 *              [B][N_out][D/2 + D/16] bytes); kv_scale [B][N_out] for E4M3
 *   k_idx      [B][N_out][Di] in k_dtype {F32, BF16, E4M3, MXFP4} (MXFP4:
 *              [B][N_out][Di/2] bytes, Di = 128 or 256); k_scale [B][N_out]
 *              float for E4M3, [B][N_out][Di/32] E8M0 bytes for MXFP4
 * Workspace: none.
 * ------------------------------------------------------------------------ */
int csa2_compress(int B, int T, int D, int m, int Di,
                  const void* c, const void* z, int in_dtype,
                  const int64_t* t0, const float* gain, float eps,
                  int rope_dims, float rope_base,
                  const void* w_ik, int w_dtype, int N_out,
                  void* kv, float* kv_scale, int kv_dtype,
                  void* k_idx, void* k_scale, int k_dtype, void* stream);

/* ------------------------------------------------------------------------
 * csa2_group -- a sharing group in one call: layers[0 .. n_layers-1] in
 * order on one stream, e.g. Full (building the pool) -> Reindex ->
 * Reindex -> Reuse -> Reuse over one shared store ("DeepSeek-V4.1-Flash
 * explained", section 2 mode table and section 3 "Hierarchical indexing:
 * search broadly once").  Later layers read the idx_inout / pool_inout
 * their predecessors write, so they must point at the same buffers.  All
 * descriptors (and their workspaces, which layers of one group may share,
 * since the layers run one after another) are validated before anything is
 * enqueued.  The whole group is a fixed sequence of launches, so a caller
 * can capture it in one HIP graph.
 * ------------------------------------------------------------------------ */
int csa2_group(const csa2_layer_desc* layers, int n_layers, void* stream);

/* Static text for a status code; for the last error on the calling thread
 * it includes the detail recorded then. */
const char* csa2_status_str(int status);

/* Library version string. */
const char* csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
