// Top-K record selection and the hierarchical block pool.
//
// Top-K returns the addresses of the K best records, never their scores
// ("Create DeepSeek from scratch", lesson 06, worked example and unit test):
// preference is score descending, then record id ascending.  Exact ties
// really occur (a ReLU sum is exactly 0 whenever every head's product is
// negative), so the tie-break is part of the result.
//
// Each element gets the 64-bit composite key (score_key(score) << 32 |
// ~record_id); with unique record ids the keys are unique and "the K
// largest composite keys" is exactly the required set.
//
// One workgroup (1024 threads) per row:
//  1. min/max of the selectable scores (block reduction);
//  2. histogram of a monotone bucket index b = (score - min) * 2048/(max-min)
//     -- spreading the scores over 2048 LDS bins keeps same-address atomic
//     contention low, unlike the top bits of the float, which cluster in a
//     few exponents;
//  3. the boundary bucket B*: fewer than K elements lie above it;
//  4. the boundary bucket's elements (usually a handful) go to LDS and an
//     exact 8-bit radix select over their composite keys picks the ones
//     still needed;
//  5. ordered compaction writes the chosen record ids in column order (or,
//     for the pool, a bitonic sort orders them by composite key).
// Rows of up to 16384 columns are cached in LDS; longer rows are re-read
// from global memory (L2) in each pass.
//
// The block pool scores block b of a row by the maximum of its members
// ("DeepSeek V4.1-Flash. Every layer, connected.", hierarchy caption) in a
// small kernel, then runs the same selection on the block maxima.
#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kNB = 2048;          // buckets of the first level
constexpr int kLdsCols = 16384;    // rows up to this length are cached in LDS
constexpr int kCandCap = 4096;     // boundary-bucket candidates held in LDS
constexpr int kMaxK = 2048;        // largest K (and P) accepted

struct TopkP {
    int rows, ncols, K, P, blk;
    const float* scores;
    const int32_t* pool;
    int32_t* idx;
    int sort_by_key;
};

struct Shared {
    float vals[kLdsCols];
    int hist[kNB];
    uint32_t cand_hi[kCandCap];
    uint32_t cand_lo[kCandCap];
    uint32_t sel_hi[kMaxK];
    uint32_t sel_lo[kMaxK];
    float red_f[2][kWaves];
    int red_i[kWaves + 1];
    int hist8[256];
    int misc[8];
};

__device__ __forceinline__ int rec_of(const TopkP& p, const int32_t* prow, int c) {
    if (!prow) return c;
    const int pb = prow[c / p.blk];
    return pb < 0 ? -1 : pb * p.blk + c % p.blk;
}

// Block-wide sum; every thread gets the result.
__device__ int block_sum(int v, int* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = warp_sum_i(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += red[i];
    return t;
}

// Finds the digit d of a 256-bin histogram such that the count of larger
// digits is < need <= count of digits >= d.  Returns d and updates need to
// the number still to take among digit d.  Called by all threads after a
// barrier; thread 0 computes, everyone reads.
__device__ int pick_digit(int* hist8, int* misc, int& need) {
    if (threadIdx.x == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
            if (above + hist8[d] >= need) break;
            above += hist8[d];
        }
        misc[0] = d;
        misc[1] = need - above;
    }
    __syncthreads();
    const int d = misc[0];
    need = misc[1];
    __syncthreads();
    return d;
}

// Exact selection of the `need` largest composite keys among the elements
// that `src(i, hi, lo)` yields for i in [0, count); returns the threshold
// (thr_hi, thr_lo): chosen = hi > thr_hi || (hi == thr_hi && lo >= thr_lo).
template <class Src>
__device__ void radix_select(Src src, int count, int need, Shared& sh, uint32_t& thr_hi,
                             uint32_t& thr_lo) {
    uint32_t pre_hi = 0, mask_hi = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kThreads) sh.hist8[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < count; i += kThreads) {
            uint32_t hi, lo;
            if (src(i, hi, lo) && (hi & mask_hi) == pre_hi) atomicAdd(&sh.hist8[(hi >> shift) & 255], 1);
        }
        __syncthreads();
        const int d = pick_digit(sh.hist8, sh.misc, need);
        pre_hi |= static_cast<uint32_t>(d) << shift;
        mask_hi |= 255u << shift;
    }
    thr_hi = pre_hi;
    // how many carry exactly thr_hi?
    int eq = 0;
    for (int i = threadIdx.x; i < count; i += kThreads) {
        uint32_t hi, lo;
        if (src(i, hi, lo) && hi == pre_hi) ++eq;
    }
    eq = block_sum(eq, sh.red_i);
    if (eq == need) {
        thr_lo = 0;
        return;
    }
    uint32_t pre_lo = 0, mask_lo = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kThreads) sh.hist8[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < count; i += kThreads) {
            uint32_t hi, lo;
            if (src(i, hi, lo) && hi == pre_hi && (lo & mask_lo) == pre_lo)
                atomicAdd(&sh.hist8[(lo >> shift) & 255], 1);
        }
        __syncthreads();
        const int d = pick_digit(sh.hist8, sh.misc, need);
        pre_lo |= static_cast<uint32_t>(d) << shift;
        mask_lo |= 255u << shift;
    }
    thr_lo = pre_lo;
}

__global__ __launch_bounds__(kThreads) void topk_row_kernel(TopkP p) {
    __shared__ Shared sh;
    const int row = blockIdx.x;
    const int n = p.ncols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* srow = p.scores + static_cast<size_t>(row) * n;
    const int32_t* prow = p.pool ? p.pool + static_cast<size_t>(row) * p.P : nullptr;
    int32_t* orow = p.idx + static_cast<size_t>(row) * p.K;
    const bool cached = n <= kLdsCols;

    auto value = [&](int c) -> float { return cached ? sh.vals[c] : srow[c]; };
    auto selectable = [&](int c, float v) -> bool {
        return score_key(v) != 0u && rec_of(p, prow, c) >= 0;
    };

    // 1. load, count, min/max
    float vmin = __builtin_huge_valf(), vmax = -__builtin_huge_valf();
    int nvalid = 0;
    for (int c = threadIdx.x; c < n; c += kThreads) {
        const float v = srow[c];
        if (cached) sh.vals[c] = v;
        if (selectable(c, v)) {
            ++nvalid;
            vmin = fminf(vmin, v);
            vmax = fmaxf(vmax, v);
        }
    }
    vmin = -warp_max(-vmin);
    vmax = warp_max(vmax);
    if (lane == 0) { sh.red_f[0][wave] = vmin; sh.red_f[1][wave] = vmax; }
    nvalid = block_sum(nvalid, sh.red_i);  // contains barriers
    vmin = sh.red_f[0][0];
    vmax = sh.red_f[1][0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) {
        vmin = fminf(vmin, sh.red_f[0][i]);
        vmax = fmaxf(vmax, sh.red_f[1][i]);
    }

    const int K = p.K;
    const int take = nvalid < K ? nvalid : K;
    // bucket mapping; degenerate ranges put everything in bucket 0
    const float span = vmax - vmin;
    const float bscale = (span > 0.f && span < __builtin_huge_valf()) ? static_cast<float>(kNB) / span : 0.f;
    auto bucket = [&](float v) -> int {
        const int b = static_cast<int>((v - vmin) * bscale);
        return b < 0 ? 0 : (b >= kNB ? kNB - 1 : b);
    };

    int bstar = -1;  // elements in buckets > bstar are chosen outright
    uint32_t thr_hi = 0, thr_lo = 0;
    if (nvalid > K) {
        // 2. bucket histogram
        for (int i = threadIdx.x; i < kNB; i += kThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int c = threadIdx.x; c < n; c += kThreads) {
            const float v = value(c);
            if (selectable(c, v)) atomicAdd(&sh.hist[bucket(v)], 1);
        }
        __syncthreads();
        // 3. boundary bucket (thread 0 walks down from the top)
        if (threadIdx.x == 0) {
            int above = 0, b = kNB - 1;
            for (; b > 0; --b) {
                if (above + sh.hist[b] >= K) break;
                above += sh.hist[b];
            }
            sh.misc[2] = b;
            sh.misc[3] = K - above;  // still needed from bucket b
            sh.misc[4] = 0;          // candidate count
        }
        __syncthreads();
        bstar = sh.misc[2];
        const int need = sh.misc[3];
        // 4. candidates of the boundary bucket
        for (int c = threadIdx.x; c < n; c += kThreads) {
            const float v = value(c);
            if (selectable(c, v) && bucket(v) == bstar) {
                const int slot = atomicAdd(&sh.misc[4], 1);
                if (slot < kCandCap) {
                    sh.cand_hi[slot] = score_key(v);
                    sh.cand_lo[slot] = ~static_cast<uint32_t>(rec_of(p, prow, c));
                }
            }
        }
        __syncthreads();
        const int ncand = sh.misc[4];
        if (ncand <= kCandCap) {
            auto src = [&](int i, uint32_t& hi, uint32_t& lo) -> bool {
                hi = sh.cand_hi[i];
                lo = sh.cand_lo[i];
                return true;
            };
            radix_select(src, ncand, need, sh, thr_hi, thr_lo);
        } else {
            auto src = [&](int c, uint32_t& hi, uint32_t& lo) -> bool {
                const float v = value(c);
                if (!selectable(c, v) || bucket(v) != bstar) return false;
                hi = score_key(v);
                lo = ~static_cast<uint32_t>(rec_of(p, prow, c));
                return true;
            };
            radix_select(src, n, need, sh, thr_hi, thr_lo);
        }
    }

    auto chosen = [&](int c) -> bool {
        const float v = value(c);
        if (!selectable(c, v)) return false;
        if (bstar < 0) return true;
        const int b = bucket(v);
        if (b != bstar) return b > bstar;
        const uint32_t hi = score_key(v);
        if (hi != thr_hi) return hi > thr_hi;
        return ~static_cast<uint32_t>(rec_of(p, prow, c)) >= thr_lo;
    };

    if (!p.sort_by_key) {
        // 5a. ordered compaction: each wave owns a contiguous column range
        const int span_w = ((n + kWaves - 1) / kWaves + 63) & ~63;
        const int c0 = wave * span_w, c1 = min(n, c0 + span_w);
        int cnt = 0;
        for (int base = c0; base < c1; base += 64) {
            const int c = base + lane;
            const bool s = c < c1 && chosen(c);
            cnt += __popcll(__ballot(s));
        }
        __syncthreads();
        if (lane == 0) sh.red_i[wave] = cnt;
        __syncthreads();
        int off = 0;
        for (int i = 0; i < wave; ++i) off += sh.red_i[i];
        for (int base = c0; base < c1; base += 64) {
            const int c = base + lane;
            const bool s = c < c1 && chosen(c);
            const unsigned long long bal = __ballot(s);
            const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
            if (s && pos < K) orow[pos] = rec_of(p, prow, c);
            off += __popcll(bal);
        }
        for (int i = take + threadIdx.x; i < K; i += kThreads) orow[i] = -1;
    } else {
        // 5b. gather the chosen keys, bitonic sort descending, write ids
        if (threadIdx.x == 0) sh.misc[5] = 0;
        __syncthreads();
        for (int c = threadIdx.x; c < n; c += kThreads) {
            if (chosen(c)) {
                const int slot = atomicAdd(&sh.misc[5], 1);
                if (slot < K) {
                    sh.sel_hi[slot] = score_key(value(c));
                    sh.sel_lo[slot] = ~static_cast<uint32_t>(rec_of(p, prow, c));
                }
            }
        }
        __syncthreads();
        int m2 = 1;
        while (m2 < take) m2 <<= 1;
        for (int i = take + threadIdx.x; i < m2; i += kThreads) { sh.sel_hi[i] = 0; sh.sel_lo[i] = 0; }
        __syncthreads();
        for (int k = 2; k <= m2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = threadIdx.x; i < m2; i += kThreads) {
                    const int ij = i ^ j;
                    if (ij > i) {
                        const unsigned long long a = (static_cast<unsigned long long>(sh.sel_hi[i]) << 32) | sh.sel_lo[i];
                        const unsigned long long b = (static_cast<unsigned long long>(sh.sel_hi[ij]) << 32) | sh.sel_lo[ij];
                        const bool desc = (i & k) == 0;
                        if (desc ? (a < b) : (a > b)) {
                            sh.sel_hi[i] = static_cast<uint32_t>(b >> 32); sh.sel_lo[i] = static_cast<uint32_t>(b);
                            sh.sel_hi[ij] = static_cast<uint32_t>(a >> 32); sh.sel_lo[ij] = static_cast<uint32_t>(a);
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = threadIdx.x; i < K; i += kThreads)
            orow[i] = i < take ? static_cast<int32_t>(~sh.sel_lo[i]) : -1;
    }
}

// Block maxima: beta[row][j] = max over columns [j*blk, min((j+1)*blk, N)).
__global__ __launch_bounds__(256) void block_max_kernel(const float* scores, int N, int blk, int nb,
                                                        float* beta) {
    const int row = blockIdx.y;
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nb) return;
    const float* s = scores + static_cast<size_t>(row) * N + static_cast<size_t>(j) * blk;
    const int len = min(blk, N - j * blk);
    float m = -__builtin_huge_valf();
    for (int i = 0; i < len; ++i) {
        const float v = s[i];
        if (v > m) m = v;  // NaN never raises the maximum
    }
    beta[static_cast<size_t>(row) * nb + j] = m;
}

int launch_rows(const TopkP& p, hipStream_t st) {
    hipLaunchKernelGGL(topk_row_kernel, dim3(p.rows), dim3(kThreads), 0, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t topk_ws_bytes(int, int, int) { return 0; }

int launch_topk(const TopkArgs& a, void* stream) {
    TopkP p;
    p.rows = a.rows; p.ncols = a.ncols; p.K = a.K; p.P = a.P; p.blk = a.blk;
    p.scores = a.scores; p.pool = a.pool; p.idx = a.idx; p.sort_by_key = a.sort_by_key ? 1 : 0;
    return launch_rows(p, static_cast<hipStream_t>(stream));
}

size_t block_pool_ws_bytes(int rows, int N, int blk) {
    const size_t nb = (static_cast<size_t>(N) + blk - 1) / blk;
    return ((static_cast<size_t>(rows) * nb * sizeof(float)) + 255) & ~static_cast<size_t>(255);
}

int launch_block_pool(int rows, int N, int blk, int P, const float* scores, int32_t* pool, void* ws,
                      size_t, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int nb = (N + blk - 1) / blk;
    float* beta = static_cast<float*>(ws);
    hipLaunchKernelGGL(block_max_kernel, dim3((nb + 255) / 256, rows), dim3(256), 0, st, scores, N, blk,
                       nb, beta);
    int e = static_cast<int>(hipGetLastError());
    if (e) return e;
    TopkP p;
    p.rows = rows; p.ncols = nb; p.K = P; p.P = 0; p.blk = 0;
    p.scores = beta; p.pool = nullptr; p.idx = pool; p.sort_by_key = 1;
    return launch_rows(p, st);
}

}  // namespace csa2
