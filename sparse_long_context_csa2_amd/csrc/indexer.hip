// Lightning-indexer scoring kernels.
//
//   I[b,t,s] = sum_h w[b,t,h] * max(0, q_idx[b,t,h,:] . k[b,s,:])
//
// with -inf for records the query may not see ("DeepSeek V4.1-Flash. Every
// layer, connected.", caption "The global and index paths"; "DeepSeek V4
// Inside: One Token Through Every Block", Fig. 10).
//
// Two kernels:
//  * idx_mfma_kernel -- 32 heads x 128 dims, bf16 queries, bf16 or e4m3
//    keys.  The heads are the M side of 16x16x32 bf16 MFMAs (two m-tiles),
//    16 records are the N side, the 128 dims are four k-steps.  Each lane
//    loads its record's key bytes straight into registers: for one load
//    instruction the four lanes that share a record read 64 contiguous
//    bytes, so a wave touches 16 whole 64-byte segments per instruction.
//    The ReLU, head weights and the sum over heads run in the epilogue:
//    a lane holds 8 heads of one record, two xor-shuffles finish the sum.
//    Decode rows (one query token) give each wave its own record tiles.
//  * idx_prefill_kernel -- many tokens of one sequence (no pool): 32x32x16
//    MFMAs over LDS-staged key tiles shared by a workgroup's 8 tokens.
//  * idx_generic_kernel -- any head count/dim and dtype, one thread per
//    (row, column), fp32 FMA; used for small shapes such as the toy.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kHi = 32;
constexpr int kDi = 128;

struct IdxP {
    int B, Tq, N, m, ncols, P, blk;
    const uint16_t* q;   // bf16 [B][Tq][32][128]
    const float* w;      // [B][Tq][32]
    const uint8_t* k;    // key rows, bf16 or e4m3
    const float* ks;     // e4m3 row scales [B][N]
    const int64_t* q_pos;
    const int32_t* n_rec;
    const int32_t* pool;
    float* out;
    int tiles_per_block;
};

__device__ __forceinline__ int visible_count(int64_t t, int m, int nrec) {
    // records s with m*s + m - 1 <= t  <=>  s < floor((t + 1) / m)
    if (t < 0) return 0;
    int64_t v = (t + 1) / m;
    return v < nrec ? static_cast<int>(v) : nrec;
}

// Element offset (in units of 8 values) of k-step `ks` for lane group `g`.
template <int KDT>
__device__ __forceinline__ int chunk8(int g, int ks) {
    if (KDT == DT_BF16) return g + 4 * ks;                 // one 16-byte load per k-step
    return 2 * (g + 4 * (ks >> 1)) + (ks & 1);             // one 16-byte load per two k-steps
}

// Loads the lane's share of one key row as four bf16x8 k-step operands.
// Streaming (decode) reads are marked non-temporal: each key row is used
// once per call.  Prefill reads keep normal caching: every key tile is
// reused by all query-token groups.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int KDT, bool NT>
__device__ __forceinline__ void load_key(const uint8_t* row, int g, bool valid, bf16x8 (&bk)[4]) {
    if (KDT == DT_BF16) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 v = valid ? ld16<NT>(p + g + 4 * ks) : u32x4{0, 0, 0, 0};
            bk[ks] = as_bf16x8(v);
        }
    } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            u32x4 v = valid ? ld16<NT>(p + g + 4 * i) : u32x4{0, 0, 0, 0};
            bk[2 * i] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{v[0], v[1]}));
            bk[2 * i + 1] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{v[2], v[3]}));
        }
    }
}

// TOKW query tokens per wave.  WAVES_ON_TOKENS: the block's four waves take
// different tokens and the same record tiles (prefill); otherwise they take
// the same token and different tiles (decode, or any pooled row).
template <int KDT, int TOKW, bool WAVES_ON_TOKENS>
__global__ __launch_bounds__(256) void idx_mfma_kernel(IdxP p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;

    int b, tok0, ntok;
    if (WAVES_ON_TOKENS) {
        const int gps = (p.Tq + 4 * TOKW - 1) / (4 * TOKW);
        b = blockIdx.y / gps;
        tok0 = (blockIdx.y % gps) * 4 * TOKW + wave * TOKW;
        ntok = p.Tq - tok0;
        ntok = ntok < 0 ? 0 : (ntok > TOKW ? TOKW : ntok);
    } else {
        b = blockIdx.y / p.Tq;
        tok0 = blockIdx.y % p.Tq;
        ntok = 1;
    }
    if (ntok == 0) return;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;

    // A operands (queries), head weights and visibility of the wave's tokens.
    bf16x8 qa[TOKW][2][4];
    float wv[TOKW][2][4];
    int vis[TOKW];
    int vis_max = 0;
#pragma unroll
    for (int tk = 0; tk < TOKW; ++tk) {
        const bool on = tk < ntok;
        const size_t row = static_cast<size_t>(b) * p.Tq + tok0 + (on ? tk : 0);
        vis[tk] = on ? visible_count(p.q_pos[row], p.m, nrec) : 0;
        vis_max = max(vis_max, vis[tk]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const uint16_t* qh = p.q + (row * kHi + 16 * mt + n) * kDi;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4 v = on ? *reinterpret_cast<const u32x4*>(qh + 8 * chunk8<KDT>(g, ks))
                             : u32x4{0, 0, 0, 0};
                qa[tk][mt][ks] = as_bf16x8(v);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) wv[tk][mt][v] = on ? p.w[row * kHi + 16 * mt + 4 * g + v] : 0.f;
        }
    }

    const int ntiles = (p.ncols + 15) / 16;
    const int t_begin = blockIdx.x * p.tiles_per_block;
    const int t_end = min(ntiles, t_begin + p.tiles_per_block);
    const int t_step = WAVES_ON_TOKENS ? 1 : 4;
    const int t_first = t_begin + (WAVES_ON_TOKENS ? 0 : wave);
    const int32_t* prow = p.pool ? p.pool + (static_cast<size_t>(b) * p.Tq + tok0) * p.P : nullptr;
    const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;

    // One record tile in flight ahead of the one being multiplied.
    struct Tile {
        int c, rec;
        bool ld, any;
        bf16x8 bk[4];
        float kscale;
    };
    auto fetch = [&](int ti, Tile& T) {
        T.c = ti * 16 + n;
        T.rec = -1;
        if (T.c < p.ncols) {
            if (prow) {
                const int pb = prow[T.c / p.blk];
                T.rec = pb < 0 ? -1 : pb * p.blk + T.c % p.blk;
            } else {
                T.rec = T.c;
            }
        }
        T.ld = T.rec >= 0 && T.rec < vis_max;
        T.any = __any(T.ld);
        T.kscale = 1.f;
        if (T.any) {
            load_key<KDT, !WAVES_ON_TOKENS>(kbase + static_cast<size_t>(T.ld ? T.rec : 0) * kRowBytes, g, T.ld,
                                            T.bk);
            if (KDT == DT_E4M3) T.kscale = T.ld ? p.ks[static_cast<size_t>(b) * p.N + T.rec] : 0.f;
        }
    };
    Tile cur, nxt;
    if (t_first < t_end) fetch(t_first, cur);
    for (int ti = t_first; ti < t_end; ti += t_step) {
        if (ti + t_step < t_end) fetch(ti + t_step, nxt);
        const int c = cur.c;
        if (!cur.any) {
#pragma unroll
            for (int tk = 0; tk < TOKW; ++tk) {
                if (g == 0 && tk < ntok && c < p.ncols)
                    p.out[(static_cast<size_t>(b) * p.Tq + tok0 + tk) * p.ncols + c] = -__builtin_huge_valf();
            }
        } else {
#pragma unroll
            for (int tk = 0; tk < TOKW; ++tk) {
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc0 = mfma16x16x32(qa[tk][0][ks], cur.bk[ks], acc0);
                    acc1 = mfma16x16x32(qa[tk][1][ks], cur.bk[ks], acc1);
                }
                float part = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float d0 = acc0[v], d1 = acc1[v];
                    if (KDT == DT_E4M3) { d0 *= cur.kscale; d1 *= cur.kscale; }
                    part += wv[tk][0][v] * fmaxf(d0, 0.f);
                    part += wv[tk][1][v] * fmaxf(d1, 0.f);
                }
                part += shfl_xor_f(part, 16);
                part += shfl_xor_f(part, 32);
                if (g == 0 && tk < ntok && c < p.ncols) {
                    const bool ok = cur.rec >= 0 && cur.rec < vis[tk];
                    p.out[(static_cast<size_t>(b) * p.Tq + tok0 + tk) * p.ncols + c] =
                        ok ? part : -__builtin_huge_valf();
                }
            }
        }
        cur = nxt;
    }
}

// Prefill scoring: many query tokens of one sequence against the records
// they may see -- a causal GEMM (tokens x heads) x 128 x records with a
// ReLU and weighted head-sum epilogue.  32x32x16 MFMAs: M = the 32 heads of
// one token, N = 32 records, K = 128 dims in 8 k-steps.  A workgroup takes
// kPfTok consecutive tokens (kPfTokW per wave, their query fragments and
// head weights in registers) and streams the 32-record key tiles they can
// see through LDS (double-buffered, fetched two tiles ahead); each lane
// ends a tile holding 16 heads of one record, so the head sum is a short
// tree and one lane swap.  The grid is (column chunk of kPfChunk, token
// block): later token blocks see more records, and the chunks keep the
// longest workgroup short.  Scores collect in LDS and leave in whole rows
// at the end: no global store sits in the tile loop, so the waits for the
// key prefetches stay exact.
constexpr int kPfTokW = 2;             // tokens per wave
constexpr int kPfTok = 4 * kPfTokW;    // tokens per workgroup
constexpr int kPfRec = 32;             // records per tile
constexpr int kPfPitch = kDi + 8;      // bf16 per LDS key row: 272 B keeps 16 lanes' reads on distinct banks
constexpr int kPfChunk = 512;          // score columns per workgroup

template <int KDT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void idx_prefill_kernel(IdxP p) {
    __shared__ __align__(16) uint16_t kt[2][kPfRec * kPfPitch];
    __shared__ float kts[2][kPfRec];
    __shared__ __align__(16) float scs[kPfTok][kPfChunk];
    __shared__ __align__(16) float wl[kPfTok][kHi];
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;   // record within the tile (B and C column)
    const int kg = lane >> 5;  // k group
    // Workgroup L runs on XCD L % 8 (round-robin dispatch).  The column
    // chunks of one token block get ids that are equal mod 8, so its query
    // rows are fetched into one L2 and shared; later token blocks (more
    // visible records) come first.
    const int gps = (p.Tq + kPfTok - 1) / kPfTok;
    const int nblk = p.B * gps;
    const int nch = (p.ncols + kPfChunk - 1) / kPfChunk;
    const int L = static_cast<int>(blockIdx.x);
    const int mi = L / 8;
    const int tbi = (mi / nch) * 8 + L % 8;
    if (tbi >= nblk) return;  // padding of the id space to a multiple of 8 blocks
    const int blk = nblk - 1 - tbi;
    const int c0 = (mi % nch) * kPfChunk;
    const int cw = min(kPfChunk, p.ncols - c0);
    const int b = blk / gps;
    const int tb = (blk % gps) * kPfTok;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
    const size_t row0 = static_cast<size_t>(b) * p.Tq;

    // Every global read the block needs before its first tile goes out
    // at once: positions (lanes 0..7 of each wave), query fragments, head
    // weights (to LDS) and, below, the first key tiles.
    const int pt = tb + (lane & 7);
    const int64_t pos = pt < p.Tq ? p.q_pos[row0 + pt] : -1;
    bf16x8 qa[kPfTokW][8];
#pragma unroll
    for (int tk = 0; tk < kPfTokW; ++tk) {
        const int t = min(tb + kPfTokW * wave + tk, p.Tq - 1);
        const uint16_t* qh = p.q + ((row0 + t) * kHi + j) * kDi + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qa[tk][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 16 * ks));
    }
    {
        const int t = min(tb + tid / kHi, p.Tq - 1);
        wl[tid / kHi][tid % kHi] = p.w[(row0 + t) * kHi + tid % kHi];  // 256 threads = 8 tokens x 32 heads
    }
    // key tile staging: thread -> (record tid / 8, 16-dim chunk tid % 8)
    const int sr = tid >> 3, sc = tid & 7;
    const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;
    typedef typename std::conditional<KDT == DT_BF16, u32x4, u32x2>::type Raw;
    struct Stage {
        Raw d[2];
        float s;
    };
    auto fetch = [&](int ti, Stage& st) {
        const int rec = ti * kPfRec + sr;
        const bool ok = rec < p.N;  // rows past the visible ones are masked after the product
        const uint8_t* r = kbase + static_cast<size_t>(ok ? rec : 0) * kRowBytes;
        if constexpr (KDT == DT_BF16) {
            st.d[0] = ok ? reinterpret_cast<const u32x4*>(r)[2 * sc] : u32x4{0, 0, 0, 0};
            st.d[1] = ok ? reinterpret_cast<const u32x4*>(r)[2 * sc + 1] : u32x4{0, 0, 0, 0};
            st.s = 1.f;
        } else {
            st.d[0] = ok ? reinterpret_cast<const u32x2*>(r)[2 * sc] : u32x2{0, 0};
            st.d[1] = ok ? reinterpret_cast<const u32x2*>(r)[2 * sc + 1] : u32x2{0, 0};
            st.s = (ok && sc == 0) ? p.ks[static_cast<size_t>(b) * p.N + rec] : 0.f;
        }
    };
    auto land = [&](int buf, const Stage& st) {
        u32x4* d = reinterpret_cast<u32x4*>(&kt[buf][sr * kPfPitch + 16 * sc]);
        if constexpr (KDT == DT_BF16) {
            d[0] = st.d[0];
            d[1] = st.d[1];
        } else {
            d[0] = e4m3x8_to_bf16x8(st.d[0]);
            d[1] = e4m3x8_to_bf16x8(st.d[1]);
            if (sc == 0) kts[buf][sr] = st.s;
        }
    };

    const int it0 = c0 / kPfRec;
    const int it_cap = (c0 + cw + kPfRec - 1) / kPfRec;  // tiles of this chunk
    Stage s0, sa, sb;  // tiles it0, it+1 and it+2
    fetch(it0, s0);
    if (it0 + 1 < it_cap) fetch(it0 + 1, sa);
    if (it0 + 2 < it_cap) fetch(it0 + 2, sb);

    // visibility: lanes 0..7 hold the block's tokens; the block's maximum
    // bounds the tiles, each token masks its own columns
    int v8 = (lane < kPfTok && pt < p.Tq) ? visible_count(pos, p.m, nrec) : 0;
#pragma unroll
    for (int o = 1; o < kPfTok; o <<= 1) v8 = max(v8, __shfl_xor(v8, o, kWave));
    const int vis_blk = min(__builtin_amdgcn_readfirstlane(v8), p.ncols);
    int vis[kPfTokW];
#pragma unroll
    for (int tk = 0; tk < kPfTokW; ++tk) {
        const int i = kPfTokW * wave + tk;
        const int vi = (tb + i < p.Tq) ? visible_count(__shfl(pos, i, kWave), p.m, nrec) : 0;
        vis[tk] = __builtin_amdgcn_readfirstlane(vi);
    }
    // tiles of this chunk that any token of the block can see
    const int it_end = min((min(vis_blk, c0 + cw) + kPfRec - 1) / kPfRec, it_cap);
    if (it0 < it_end) land(0, s0);
    // columns no tile writes stay -inf
    for (int i = tid; i < kPfTok * kPfChunk / 4; i += 256)
        reinterpret_cast<f32x4*>(&scs[0][0])[i] = f32x4{-__builtin_huge_valf(), -__builtin_huge_valf(),
                                                        -__builtin_huge_valf(), -__builtin_huge_valf()};
    {
        for (int it = it0; it < it_end; ++it) {
            const int buf = (it - it0) & 1;
            __syncthreads();  // tile `it` in LDS; tile it-1's buffer free; score rows cleared
            bf16x8 bk[8];
            const uint16_t* kr = &kt[buf][j * kPfPitch + 8 * kg];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) bk[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * ks));
            f32x16 c[kPfTokW];
#pragma unroll
            for (int tk = 0; tk < kPfTokW; ++tk)
#pragma unroll
                for (int v = 0; v < 16; ++v) c[tk][v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int tk = 0; tk < kPfTokW; ++tk) c[tk] = mfma32x32x16(qa[tk][ks], bk[ks], c[tk]);
            const int rec = it * kPfRec + j;
            const float ksc = (KDT == DT_E4M3) ? kts[buf][j] : 1.f;
#pragma unroll
            for (int tk = 0; tk < kPfTokW; ++tk) {
                // head weights of this lane's 16 heads: 8 (v / 4) + 4 kg + v % 4
                float wv[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4*>(&wl[kPfTokW * wave + tk][8 * q4 + 4 * kg]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) wv[4 * q4 + v] = w4[v];
                }
                float pr[8];
#pragma unroll
                for (int v = 0; v < 8; ++v)
                    pr[v] = fmaf(wv[2 * v + 1], fmaxf(c[tk][2 * v + 1], 0.f), wv[2 * v] * fmaxf(c[tk][2 * v], 0.f));
                const float part = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                float x, y;
                pair_xor32(part, x, y);
                const float val = (x + y) * ksc;  // the row scale is >= 0, so it commutes with the ReLU
                if (kg == 0 && rec < c0 + cw && rec < vis[tk]) scs[kPfTokW * wave + tk][rec - c0] = val;
            }
            if (it + 1 < it_end) {
                land(buf ^ 1, sa);
                sa = sb;
                if (it + 3 < it_end) fetch(it + 3, sb);
            }
        }
        __syncthreads();  // score rows complete
        // 16-byte stores when every output row starts 16-byte aligned
        const int cw4 = (p.ncols % 4 == 0) ? cw / 4 : 0;
        for (int i = tid; i < kPfTok * cw4; i += 256) {
            const int tk = i / cw4, q4 = i % cw4;
            if (tb + tk < p.Tq)
                *reinterpret_cast<f32x4*>(&p.out[(row0 + tb + tk) * p.ncols + c0 + 4 * q4]) =
                    reinterpret_cast<const f32x4*>(&scs[tk][0])[q4];
        }
        const int rest = cw - 4 * cw4;  // columns left for single stores
        for (int i = tid; i < kPfTok * rest; i += 256) {
            const int tk = i / rest, col = 4 * cw4 + i % rest;
            if (tb + tk < p.Tq) p.out[(row0 + tb + tk) * p.ncols + c0 + col] = scs[tk][col];
        }
    }
}

struct IdxG {
    int B, Tq, N, Hi, Di, m, ncols, P, blk, qdt, kdt;
    const void* q;
    const float* w;
    const void* k;
    const float* ks;
    const int64_t* q_pos;
    const int32_t* n_rec;
    const int32_t* pool;
    float* out;
};

__global__ __launch_bounds__(256) void idx_generic_kernel(IdxG p) {
    extern __shared__ float sh[];  // q row [Hi*Di] then w [Hi]
    const size_t row = blockIdx.y;
    const int b = static_cast<int>(row / p.Tq);
    const int HD = p.Hi * p.Di;
    for (int i = threadIdx.x; i < HD; i += blockDim.x) sh[i] = load_elem(p.q, row * HD + i, p.qdt);
    for (int i = threadIdx.x; i < p.Hi; i += blockDim.x) sh[HD + i] = p.w[row * p.Hi + i];
    __syncthreads();
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= p.ncols) return;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
    const int vis = visible_count(p.q_pos[row], p.m, nrec);
    int rec = c;
    if (p.pool) {
        const int pb = p.pool[row * p.P + c / p.blk];
        rec = pb < 0 ? -1 : pb * p.blk + c % p.blk;
    }
    float res = -__builtin_huge_valf();
    if (rec >= 0 && rec < vis) {
        const size_t kr = (static_cast<size_t>(b) * p.N + rec) * p.Di;
        const float sc = p.kdt == DT_E4M3 ? p.ks[static_cast<size_t>(b) * p.N + rec] : 1.f;
        res = 0.f;
        for (int h = 0; h < p.Hi; ++h) {
            float dot = 0.f;
            for (int i = 0; i < p.Di; ++i) dot = fmaf(sh[h * p.Di + i], load_elem(p.k, kr + i, p.kdt), dot);
            dot *= sc;
            res += sh[HD + h] * fmaxf(dot, 0.f);
        }
    }
    p.out[row * p.ncols + c] = res;
}

template <int KDT, int TOKW, bool WOT>
int launch_mfma(const IndexArgs& a, int tiles_per_block, hipStream_t st) {
    IdxP p;
    p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.m = a.m; p.ncols = a.ncols; p.P = a.P; p.blk = a.blk;
    p.q = static_cast<const uint16_t*>(a.q_idx);
    p.w = a.w;
    p.k = static_cast<const uint8_t*>(a.k_idx);
    p.ks = a.k_scale;
    p.q_pos = a.q_pos;
    p.n_rec = a.n_rec;
    p.pool = a.pool;
    p.out = a.scores;
    p.tiles_per_block = tiles_per_block;
    const int ntiles = (a.ncols + 15) / 16;
    dim3 grid((ntiles + tiles_per_block - 1) / tiles_per_block,
              WOT ? a.B * ((a.Tq + 4 * TOKW - 1) / (4 * TOKW)) : a.B * a.Tq);
    hipLaunchKernelGGL((idx_mfma_kernel<KDT, TOKW, WOT>), grid, dim3(256), 0, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

bool index_scores_mfma_ok(const IndexArgs& a) {
    return a.Hi == kHi && a.Di == kDi && a.q_dtype == DT_BF16 &&
           (a.k_dtype == DT_BF16 || a.k_dtype == DT_E4M3);
}

int launch_index_scores(const IndexArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (index_scores_mfma_ok(a)) {
        const int ntiles = (a.ncols + 15) / 16;
        const int rows = a.B * a.Tq;
        // Prefill-shaped work (many tokens of one sequence, no pool): waves
        // share record tiles across 16 tokens.
        if (!a.pool && a.Tq >= 16) {
            IdxP p;
            p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.m = a.m; p.ncols = a.ncols; p.P = a.P; p.blk = a.blk;
            p.q = static_cast<const uint16_t*>(a.q_idx);
            p.w = a.w;
            p.k = static_cast<const uint8_t*>(a.k_idx);
            p.ks = a.k_scale;
            p.q_pos = a.q_pos;
            p.n_rec = a.n_rec;
            p.pool = nullptr;
            p.out = a.scores;
            p.tiles_per_block = 0;
            const int nblk8 = (a.B * ((a.Tq + kPfTok - 1) / kPfTok) + 7) / 8 * 8;
            const dim3 grid(nblk8 * ((a.ncols + kPfChunk - 1) / kPfChunk));
            if (a.k_dtype == DT_BF16)
                hipLaunchKernelGGL(idx_prefill_kernel<DT_BF16>, grid, dim3(256), 0, st, p);
            else
                hipLaunchKernelGGL(idx_prefill_kernel<DT_E4M3>, grid, dim3(256), 0, st, p);
            return static_cast<int>(hipGetLastError());
        }
        // Decode rows: pick tiles per block so the grid has >= ~2048 blocks
        // while each wave still streams several tiles.
        int tpb = 32;
        while (tpb > 4 && static_cast<long>(rows) * ((ntiles + tpb - 1) / tpb) < 2048) tpb >>= 1;
        return a.k_dtype == DT_BF16 ? launch_mfma<DT_BF16, 1, false>(a, tpb, st)
                                    : launch_mfma<DT_E4M3, 1, false>(a, tpb, st);
    }
    IdxG p;
    p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.Hi = a.Hi; p.Di = a.Di; p.m = a.m; p.ncols = a.ncols;
    p.P = a.P; p.blk = a.blk; p.qdt = a.q_dtype; p.kdt = a.k_dtype;
    p.q = a.q_idx; p.w = a.w; p.k = a.k_idx; p.ks = a.k_scale; p.q_pos = a.q_pos;
    p.n_rec = a.n_rec; p.pool = a.pool; p.out = a.scores;
    dim3 grid((a.ncols + 255) / 256, a.B * a.Tq);
    const size_t lds = (static_cast<size_t>(a.Hi) * a.Di + a.Hi) * sizeof(float);
    hipLaunchKernelGGL(idx_generic_kernel, grid, dim3(256), lds, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
