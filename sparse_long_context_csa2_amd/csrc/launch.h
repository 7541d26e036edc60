// Internal interface between the C ABI host code and the kernel translation
// units.  Every launcher only enqueues work on `stream` and returns a
// hipError_t value as int (0 = success).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct IndexArgs {
    int B, Tq, N, Hi, Di, m;
    const void* q_idx;
    int q_dtype;
    const void* q_scale;  // MXFP4 queries: E8M0 scales [B][Tq][Hi][Di/32], else null
    const float* w;
    const void* k_idx;
    const void* k_scale;  // e4m3: float [B][N]; MXFP4: E8M0 bytes [B][N][Di/32]; else null
    int k_dtype;
    const int64_t* q_pos;
    const int32_t* n_rec;
    const int32_t* pool;  // [B][Tq][P] or null
    int P, blk;
    float* scores;        // [B][Tq][ncols]
    int ncols;
};
// True when the MFMA indexer handles these shapes and dtypes.
bool index_scores_mfma_ok(const IndexArgs& a);
int launch_index_scores(const IndexArgs& a, void* stream);

struct TopkArgs {
    int rows, ncols, K;
    const float* scores;
    const int32_t* pool;  // [rows][P] or null
    int P, blk;
    int32_t* idx;         // [rows][K]
    bool sort_by_key;     // output ordered by (score desc, id asc) instead of by column
    void* ws;
    size_t ws_bytes;
};
// Longest Top-K row (columns) the library takes.
constexpr int kTopkMaxCols = 1 << 24;
size_t topk_ws_bytes(int rows, int ncols, int K);
int launch_topk(const TopkArgs& a, void* stream);

size_t block_pool_ws_bytes(int rows, int N, int blk);
int launch_block_pool(int rows, int N, int blk, int P, const float* scores, int32_t* pool,
                      void* ws, size_t ws_bytes, void* stream);

struct AttnArgs {
    int B, Tq, H, D, N, K;
    const void* q;
    int q_dtype;
    const void* kv;
    const float* kv_scale;
    int kv_dtype;
    const int32_t* idx;
    const void* swa;
    const float* swa_scale;
    int swa_dtype;
    int S, W;
    const int64_t* q_pos;
    const float* sink;
    float sm_scale;
    int rope_dims;
    float rope_base;
    void* out;
    int out_dtype;  // DT_F32 or DT_BF16
    void* ws;
    size_t ws_bytes;
    int dense_m = 0;                // > 0: dense mode (no idx; all visible records at ratio dense_m)
    const int32_t* n_rec = nullptr;  // dense mode: [B] or null (= N)
    size_t part_cap = SIZE_MAX;      // most bytes of split partials the splits taken for parallelism may use
};
bool sparse_attn_mfma_ok(const AttnArgs& a);
size_t sparse_attn_ws_bytes(int B, int Tq, int H, int D, int K, int W, size_t part_cap = SIZE_MAX);
size_t dense_attn_ws_bytes(int B, int Tq, int H, int D, int N, int W);
int launch_sparse_attn(const AttnArgs& a, void* stream);
// The allocation-free entry point's static scratch: its size, and its
// address on the current device (looked up on the first call per device;
// err is a hipError_t value, 0 on success).
size_t sparse_attn_scratch_bytes();
void* sparse_attn_scratch(int& err);

struct CompressArgs {
    int B, T, D, m, Di, N_out;
    const void* c;
    const void* z;
    int in_dtype;
    const int64_t* t0;
    const float* gain;
    float eps;
    int rope_dims;
    float rope_base;
    const void* w_ik;
    int w_dtype;
    void* kv;
    float* kv_scale;
    int kv_dtype;
    void* k_idx;
    void* k_scale;
    int k_dtype;
};
int launch_compress(const CompressArgs& a, void* stream);

}  // namespace csa2
