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

// Non-temporal 16-byte load: in decode each key row is used once per call.
__device__ __forceinline__ u32x4 ld16_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// The lane's share of one key row, as loaded (bf16: four 16-byte k-step
// chunks; e4m3: two, each holding two k-steps).  Nothing here uses the
// bytes, so no wait follows the loads; key_operands converts them where
// they are multiplied.  `row` is always a real row: for a record the query
// may not see, the caller passes another one and drops that column's score.
template <int KDT>
__device__ __forceinline__ void load_key_raw(const uint8_t* row, int g, u32x4 (&raw)[4]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row);
    constexpr int kLoads = (KDT == DT_BF16) ? 4 : 2;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) raw[i] = ld16_nt(p + g + 4 * i);
}

template <int KDT>
__device__ __forceinline__ void key_operands(const u32x4 (&raw)[4], bf16x8 (&bk)[4]) {
    if constexpr (KDT == DT_BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bk[ks] = as_bf16x8(raw[ks]);
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            bk[2 * i] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{raw[i][0], raw[i][1]}));
            bk[2 * i + 1] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{raw[i][2], raw[i][3]}));
        }
    }
}

// Decode scoring: one query token per row (or any pooled row).  The four
// waves of a workgroup take alternate 16-record tiles of the row's column
// range; each lane loads its record's key bytes straight into registers
// (non-temporal: every key row is read once per call), several tiles
// ahead of the one being multiplied.  Scores collect in LDS and leave as whole
// column runs at the end: no store sits between a prefetch and its wait.
constexpr int kDecTpbMax = 128;  // tiles per workgroup, at most

template <int KDT>
__global__ __launch_bounds__(256) void idx_mfma_kernel(IdxP p) {
    __shared__ float osc[kDecTpbMax * 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;

    const int b = blockIdx.y / p.Tq;
    const int tok = blockIdx.y % p.Tq;
    const size_t row = static_cast<size_t>(b) * p.Tq + tok;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;

    // A operands (the token's queries), head weights and visibility
    bf16x8 qa[2][4];
    float wv[2][4];
    const int vis = visible_count(p.q_pos[row], p.m, nrec);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const uint16_t* qh = p.q + (row * kHi + 16 * mt + n) * kDi;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qa[mt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 8 * chunk8<KDT>(g, ks)));
#pragma unroll
        for (int v = 0; v < 4; ++v) wv[mt][v] = p.w[row * kHi + 16 * mt + 4 * g + v];
    }

    const int ntiles = (p.ncols + 15) / 16;
    const int t_begin = blockIdx.x * p.tiles_per_block;
    const int t_end = min(ntiles, t_begin + p.tiles_per_block);
    const int32_t* prow = p.pool ? p.pool + row * p.P : nullptr;
    const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;

    struct Tile {
        int rec;
        bool any;
        u32x4 raw[4];
        float kscale;
    };
    auto fetch = [&](int ti, Tile& T) {
        const int c = ti * 16 + n;
        T.rec = -1;
        if (c < p.ncols) {
            if (prow) {
                const int pb = prow[c / p.blk];
                T.rec = pb < 0 ? -1 : pb * p.blk + c % p.blk;
            } else {
                T.rec = c;
            }
        }
        const bool ld = T.rec >= 0 && T.rec < vis;
        T.any = __any(ld);
        T.kscale = 1.f;
        if (T.any) {
            load_key_raw<KDT>(kbase + static_cast<size_t>(ld ? T.rec : 0) * kRowBytes, g, T.raw);
            if (KDT == DT_E4M3) T.kscale = ld ? p.ks[static_cast<size_t>(b) * p.N + T.rec] : 0.f;
        }
    };
    auto score = [&](int ti, const Tile& T) {
        float val = -__builtin_huge_valf();
        if (T.any) {
            bf16x8 bk[4];
            key_operands<KDT>(T.raw, bk);
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc0 = mfma16x16x32(qa[0][ks], bk[ks], acc0);
                acc1 = mfma16x16x32(qa[1][ks], bk[ks], acc1);
            }
            float part = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float d0 = acc0[v], d1 = acc1[v];
                if (KDT == DT_E4M3) { d0 *= T.kscale; d1 *= T.kscale; }
                part += wv[0][v] * fmaxf(d0, 0.f);
                part += wv[1][v] * fmaxf(d1, 0.f);
            }
            part += shfl_xor_f(part, 16);
            part += shfl_xor_f(part, 32);
            if (T.rec >= 0 && T.rec < vis) val = part;
        }
        if (g == 0) osc[(ti - t_begin) * 16 + n] = val;
    };
    // tiles wave, wave + 4, ... of the range, through a ring of kRing
    // tiles: kRing - 1 in flight ahead of the one being multiplied (e4m3
    // tiles carry half the bytes, so more of them)
    constexpr int kRing = (KDT == DT_BF16) ? 3 : 4;
    Tile tt[kRing];
    const int ti0 = t_begin + wave;
#pragma unroll
    for (int d = 0; d + 1 < kRing; ++d)
        if (ti0 + 4 * d < t_end) fetch(ti0 + 4 * d, tt[d]);
    for (int base = ti0; base < t_end; base += 4 * kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            const int ti = base + 4 * d;
            if (ti >= t_end) break;
            const int tf = ti + 4 * (kRing - 1);
            if (tf < t_end) fetch(tf, tt[(d + kRing - 1) % kRing]);
            score(ti, tt[d]);
        }
    }
    __syncthreads();
    const int c0 = t_begin * 16;
    const int c1 = min(t_end * 16, p.ncols);
    float* orow = p.out + row * p.ncols;
    for (int c = c0 + static_cast<int>(threadIdx.x); c < c1; c += 256) orow[c] = osc[c - c0];
}

// Prefill scoring: many query tokens of one sequence against the records
// they may see -- a causal GEMM (tokens x heads) x 128 x records with a
// ReLU and weighted head-sum epilogue.  Records are stationary: a
// workgroup owns kP2Rec consecutive records, converts their keys to bf16
// in LDS once, and its waves stream query tokens past them, each token's
// query fragments read straight from global memory by the one wave that
// scores it.  32x32x16 MFMAs: M = the 32 heads of the token, N = 32
// records, K = 128 dims in 8 k-steps.  Lane group kg takes dims
// 64 kg + 8 ks .. +7 at k-step ks in both operands, so a lane's query
// fragments are 128 contiguous bytes of one head row.  Records come in
// pairs of 32-record sets: after the epilogue one lane swap leaves lane l
// holding the score of record 64 sp + l, and a wave stores 256 contiguous
// bytes.  Sets that the token cannot see at all are skipped.
constexpr int kP2Rec = 256;            // records per workgroup
constexpr int kP2TokW = 8;             // tokens per wave
constexpr int kP2Tok = 4 * kP2TokW;    // tokens per workgroup
constexpr int kP2Pitch = kDi * 2 + 16; // bytes per LDS key row: conflict-free operand reads

template <int KDT>
__global__ __launch_bounds__(256, 2) void idx_prefill_kernel(IdxP p) {
    __shared__ __align__(16) uint8_t kl[kP2Rec * kP2Pitch];
    __shared__ float ksl[kP2Rec];
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;
    constexpr int kPairs = kP2Rec / 64;  // 64-record set pairs of the group
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;   // record within a set (B and C column), head (A row)
    const int kg = lane >> 5;  // k group
    // Workgroup L runs on XCD L % 8 (round-robin dispatch).  The record
    // groups of one token block get ids that are equal mod 8 and adjacent in
    // that XCD's order, so the block's query rows are read into one L2;
    // later token blocks (more visible records) come first.
    const int ntb = (p.Tq + kP2Tok - 1) / kP2Tok;
    const int nblk = p.B * ntb;
    const int ngr = (p.ncols + kP2Rec - 1) / kP2Rec;
    const int L = static_cast<int>(blockIdx.x);
    const int mi = L / 8;
    const int tbi = (mi / ngr) * 8 + L % 8;
    if (tbi >= nblk) return;  // padding of the id space to a multiple of 8 blocks
    const int blk = nblk - 1 - tbi;
    const int b = blk / ntb;
    const int t0 = (blk % ntb) * kP2Tok;
    const int R0 = (mi % ngr) * kP2Rec;
    const int nr = min(kP2Rec, p.ncols - R0);  // columns of this group
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
    const size_t row0 = static_cast<size_t>(b) * p.Tq;

    // this wave's tokens: visibility (lane i holds token i's), and the
    // first token's query fragments and head weights
    const int tw0 = t0 + kP2TokW * wave;
    const int tw1 = min(tw0 + kP2TokW, p.Tq);
    const int vis_l = (lane < tw1 - tw0) ? visible_count(p.q_pos[row0 + tw0 + lane], p.m, nrec) : 0;
    struct Tok {
        bf16x8 a[8];
        f32x4 w[4];
    };
    auto tload = [&](int t, Tok& x) {
        const u32x4* qh = reinterpret_cast<const u32x4*>(p.q + ((row0 + t) * kHi + j) * kDi + 64 * kg);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) x.a[ks] = as_bf16x8(qh[ks]);
        // weights of this lane's 16 heads: 8 (v / 4) + 4 kg + v % 4
        const float* wr = p.w + (row0 + t) * kHi + 4 * kg;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) x.w[q4] = *reinterpret_cast<const f32x4*>(wr + 8 * q4);
    };
    Tok cur;
    if (tw0 < tw1) tload(tw0, cur);

    // keys of the group -> bf16 rows in LDS (records past N are zero rows,
    // masked below like every record the token cannot see)
    {
        typedef typename std::conditional<KDT == DT_BF16, u32x4, u32x2>::type Raw;
        constexpr int kChunkBytes = (KDT == DT_BF16) ? 16 : 8;  // 8 dims
        const uint8_t* kb = p.k + static_cast<size_t>(b) * p.N * kRowBytes;
        // all loads first and unconditional (a clamped row, zeroed after):
        // a branch around each load would serialise them
        Raw raw[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = i * 256 + tid;  // 16 chunks per record
            const int rec = min(R0 + (c >> 4), p.N - 1);
            raw[i] = *reinterpret_cast<const Raw*>(kb + static_cast<size_t>(rec) * kRowBytes + kChunkBytes * (c & 15));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = i * 256 + tid;
            u32x4 v;
            if constexpr (KDT == DT_BF16) v = raw[i];
            else v = e4m3x8_to_bf16x8(raw[i]);
            if (R0 + (c >> 4) >= p.N) v = u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(kl + (c >> 4) * kP2Pitch + 16 * (c & 15)) = v;
        }
        if constexpr (KDT == DT_E4M3)
            ksl[tid] = R0 + tid < p.N ? p.ks[static_cast<size_t>(b) * p.N + R0 + tid] : 0.f;
    }
    __syncthreads();

    // Set pairs 0 .. NP-1 of one token in one branch-free block (their
    // MFMAs, operand reads and epilogues interleave); pairs past NP are
    // out of the token's sight and score -inf.
    float sc[kP2TokW][kPairs];
    auto score_pairs = [&](auto np_tag, const Tok& x, int vis, float (&out)[kPairs]) {
        constexpr int NP = decltype(np_tag)::value;
        float wv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) wv[v] = x.w[v / 4][v % 4];
#pragma unroll
        for (int sp = 0; sp < kPairs; ++sp) {
            out[sp] = -__builtin_huge_valf();
            if (sp < NP) {  // folds: sp is unrolled, NP a constant
                const int rb = 64 * sp;
                const uint8_t* k0 = kl + (rb + j) * kP2Pitch + 128 * kg;
                const uint8_t* k1 = k0 + 32 * kP2Pitch;
                f32x16 c0, c1;
#pragma unroll
                for (int v = 0; v < 16; ++v) c0[v] = c1[v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8 b0 = as_bf16x8(*reinterpret_cast<const u32x4*>(k0 + 16 * ks));
                    const bf16x8 b1 = as_bf16x8(*reinterpret_cast<const u32x4*>(k1 + 16 * ks));
                    c0 = mfma32x32x16(x.a[ks], b0, c0);
                    c1 = mfma32x32x16(x.a[ks], b1, c1);
                }
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    s0 = fmaf(wv[v], fmaxf(c0[v], 0.f), s0);
                    s1 = fmaf(wv[v], fmaxf(c1[v], 0.f), s1);
                }
                // lanes 0..31 finish set 0 (records rb + l), lanes 32..63 set 1
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
                float tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                if constexpr (KDT == DT_E4M3) tot *= ksl[rb + lane];  // the row scale is >= 0: it commutes with the ReLU
                if (R0 + rb + lane < vis) out[sp] = tot;
            }
        }
    };
    // Scores stay in registers until the wave's tokens are done: a store
    // inside the loop would make every wait for the next token's loads wait
    // for the stores as well.
#pragma unroll
    for (int i = 0; i < kP2TokW; ++i) {
        const int t = tw0 + i;
        if (t >= tw1) break;
        Tok nxt;
        if (t + 1 < tw1) tload(t + 1, nxt);
        const int vis = __builtin_amdgcn_readlane(vis_l, i);
        // set pairs holding a record the token sees (all of them hold columns)
        const int np = min(max(vis - R0 + 63, 0) >> 6, (nr + 63) >> 6);
        switch (np) {
            case 0: score_pairs(std::integral_constant<int, 0>{}, cur, vis, sc[i]); break;
            case 1: score_pairs(std::integral_constant<int, 1>{}, cur, vis, sc[i]); break;
            case 2: score_pairs(std::integral_constant<int, 2>{}, cur, vis, sc[i]); break;
            case 3: score_pairs(std::integral_constant<int, 3>{}, cur, vis, sc[i]); break;
            default: score_pairs(std::integral_constant<int, 4>{}, cur, vis, sc[i]); break;
        }
        cur = nxt;
    }
#pragma unroll
    for (int i = 0; i < kP2TokW; ++i) {
        const int t = tw0 + i;
        if (t >= tw1) break;
        float* orow = p.out + (row0 + t) * p.ncols + R0;
#pragma unroll
        for (int sp = 0; sp < kPairs; ++sp)
            if (64 * sp + lane < nr) orow[64 * sp + lane] = sc[i][sp];
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

template <int KDT>
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
    dim3 grid((ntiles + tiles_per_block - 1) / tiles_per_block, a.B * a.Tq);
    hipLaunchKernelGGL(idx_mfma_kernel<KDT>, grid, dim3(256), 0, st, p);
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
            const int nblk8 = (a.B * ((a.Tq + kP2Tok - 1) / kP2Tok) + 7) / 8 * 8;
            const dim3 grid(nblk8 * ((a.ncols + kP2Rec - 1) / kP2Rec));
            if (a.k_dtype == DT_BF16)
                hipLaunchKernelGGL(idx_prefill_kernel<DT_BF16>, grid, dim3(256), 0, st, p);
            else
                hipLaunchKernelGGL(idx_prefill_kernel<DT_E4M3>, grid, dim3(256), 0, st, p);
            return static_cast<int>(hipGetLastError());
        }
        // Decode rows: the largest tiles per block that still gives >= 1024
        // blocks (four per CU), so each wave streams many tiles and the
        // start-up latency is paid rarely.
        int tpb = kDecTpbMax;
        while (tpb > 4 && static_cast<long>(rows) * ((ntiles + tpb - 1) / tpb) < 1024) tpb >>= 1;
        return a.k_dtype == DT_BF16 ? launch_mfma<DT_BF16>(a, tpb, st) : launch_mfma<DT_E4M3>(a, tpb, st);
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
