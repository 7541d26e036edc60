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
//    MFMAs, one token per wave with its query in registers, key tiles
//    streamed through LDS and shared by the workgroup's 8 tokens.
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
    const uint16_t* q;   // bf16 [B][Tq][32][128], or MXFP4 codes [B][Tq][32][64]
    const uint8_t* qsc;  // MXFP4 queries: E8M0 scales [B][Tq][32][4], else null
    const float* w;      // [B][Tq][32]
    const uint8_t* k;    // key rows: bf16, e4m3, or MXFP4 codes (64 bytes)
    const void* ks;      // e4m3 row scales float [B][N]; MXFP4 E8M0 scales uint8 [B][N][4]
    const int64_t* q_pos;
    const int32_t* n_rec;
    const int32_t* pool;
    float* out;
    int tiles_per_block;
};

// LDS hand-off barrier: this wave's LDS accesses are complete, then all
// waves meet (global loads in flight are not waited for)
__device__ __forceinline__ void lds_sync_all() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
    if (KDT == DT_MXFP4) return 4 * g + ks;                // one 16-byte load (= one MX block) per row
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
    if constexpr (KDT == DT_MXFP4) {  // dims 32g .. 32g+31: one MX block, 16 bytes
        raw[0] = ld16_nt(p + g);
        return;
    }
    constexpr int kLoads = (KDT == DT_BF16) ? 4 : 2;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) raw[i] = ld16_nt(p + g + 4 * i);
}

// `scale`: the lane's MX block scale (MXFP4 keys; unused otherwise).
template <int KDT>
__device__ __forceinline__ void key_operands(const u32x4 (&raw)[4], float scale, bf16x8 (&bk)[4]) {
    if constexpr (KDT == DT_BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bk[ks] = as_bf16x8(raw[ks]);
    } else if constexpr (KDT == DT_MXFP4) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bk[ks] = as_bf16x8(fp4x8_to_bf16x8(raw[0][ks], scale));
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
// range.  A tile's 16 key rows are loaded into registers as whole rows: load
// i of the wave reads 1 KiB, lane l taking 16 bytes (chunk l mod C of row
// 64 i / C + l / C, C = 16-byte chunks per row; non-temporal, as every key
// row is read once per call), several tiles ahead of the one being
// multiplied.  Before its MFMAs the wave passes the tile through its own
// LDS buffer into the operand layout (lane (n, g) takes record n's chunks
// of lane group g), chunk c of row r at slot c ^ (r mod C) so that neither
// pass has bank conflicts.  (Loading the operand layout directly -- 16
// rows x 64 bytes per instruction -- streams about 13% slower.)  MXFP4 rows
// are 64 bytes, so a lane's operand chunk (record n, MX block g) is loaded
// directly: one instruction then reads the tile's contiguous 1 KiB.  Scores
// collect in LDS and leave as whole column runs at the end: no store sits
// between a prefetch and its wait.
constexpr int kDecTpbMax = 128;  // tiles per workgroup, at most

// QMX (MXFP4 queries and keys): the scores come from gfx950's block-scaled
// MFMA, v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1: one
// instruction per 16 heads x 16 records covers all 128 dims, products are
// exact and each lane's E8M0 scale applies to its 32 dims (lane l holds row
// l % 16, dims 32 (l / 16) .. +31, element e in nibble e, low nibble first),
// which is the stored MX block of that lane group; nothing is converted.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_mx4(const u32x4& a, int sa, const u32x4& b, int sb, f32x4 c) {
    const i32x8 A = {static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                     0, 0, 0, 0};
    const i32x8 Bv = {static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3]),
                      0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bv, c, 4, 4, 0, sa, 0, sb);
}

// POOL: the row's columns are pooled blocks of records (p.pool); otherwise
// column c is record c and a tile's loads form one straight-line sequence,
// so that the waits before each tile's multiply count only that tile's
// loads (an invisible row is read from record 0 and its score dropped).
template <int KDT, bool QMX, bool POOL>
__global__ __launch_bounds__(256) void idx_mfma_kernel(IdxP p) {
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : (KDT == DT_MXFP4 ? kDi / 2 : kDi);
    constexpr int kCPR = kRowBytes / 16;  // 16-byte chunks per key row
    constexpr int kRPI = 64 / kCPR;       // rows per 1 KiB load
    constexpr int kLI = 16 / kRPI;        // loads per 16-row tile
    constexpr bool kTr = KDT != DT_MXFP4;  // tiles pass through LDS into the operand layout
    __shared__ float osc[kDecTpbMax * 16];
    __shared__ __align__(16) uint8_t ktr[kTr ? 4 : 1][kTr ? 16 * kRowBytes : 16];  // per-wave tile transpose
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int lr = lane / kCPR;  // the lane's row within a load
    const int lc = lane % kCPR;  // and its chunk

    const int b = blockIdx.y / p.Tq;
    const int tok = blockIdx.y % p.Tq;
    const size_t row = static_cast<size_t>(b) * p.Tq + tok;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;

    // A operands (the token's queries), head weights and visibility
    bf16x8 qa[2][4];
    u32x4 qmx[2];  // QMX: the lane's 32 query codes (one MX block) per m-tile
    int qmxs[2];   // QMX: their E8M0 scale
    float wv[2][4];
    const int vis = visible_count(p.q_pos[row], p.m, nrec);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        if constexpr (QMX) {  // MXFP4 queries: the head's block g and its scale
            const size_t hrow = row * kHi + 16 * mt + n;
            qmx[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.q) + hrow * (kDi / 2) + 16 * g);
            qmxs[mt] = p.qsc[hrow * (kDi / 32) + g];
        } else {
            const uint16_t* qh = p.q + (row * kHi + 16 * mt + n) * kDi;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 8 * chunk8<KDT>(g, ks)));
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) wv[mt][v] = p.w[row * kHi + 16 * mt + 4 * g + v];
    }

    const int ntiles = (p.ncols + 15) / 16;
    const int t_begin = blockIdx.x * p.tiles_per_block;
    const int t_end = min(ntiles, t_begin + p.tiles_per_block);
    const int32_t* prow = POOL ? p.pool + row * p.P : nullptr;
    const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;
    const int lim = min(vis, t_end * 16);  // !POOL: records this workgroup reads (vis <= N = ncols)

    struct Tile {
        int rec;
        bool any;
        u32x4 raw[4];
        float kscale;
        uint32_t kblk;  // MXFP4: the row's four E8M0 block scales
    };
    auto fetch = [&](int ti, Tile& T) {
        const int c = ti * 16 + n;
        bool ld;
        if constexpr (POOL) {
            T.rec = -1;
            if (c < p.ncols) {
                const int pb = prow[c / p.blk];
                T.rec = pb < 0 ? -1 : pb * p.blk + c % p.blk;
            }
            ld = T.rec >= 0 && T.rec < vis;
            T.any = __any(ld);
        } else {
            T.rec = c;
            ld = c < lim;
            T.any = ti * 16 < lim;
        }
        T.kscale = 1.f;
        T.kblk = 0;
        if (POOL && !T.any) return;
        if constexpr (!kTr) {  // MXFP4: the lane's operand chunk
            load_key_raw<KDT>(kbase + static_cast<size_t>(ld ? T.rec : 0) * kRowBytes, g, T.raw);
        } else {
            // whole rows: load i brings rows kRPI i .. +kRPI-1
#pragma unroll
            for (int i = 0; i < kLI; ++i) {
                const int r = kRPI * i + lr;
                const int rr = POOL ? __shfl(T.rec, r, 64) : ti * 16 + r;
                const bool ok = rr >= 0 && rr < (POOL ? vis : lim);
                T.raw[i] = ld16_nt(reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(ok ? rr : 0) * kRowBytes) + lc);
            }
        }
        // the scales of an invisible row are read from record 0 as well
        if (KDT == DT_E4M3) T.kscale = static_cast<const float*>(p.ks)[static_cast<size_t>(b) * p.N + (ld ? T.rec : 0)];
        if (KDT == DT_MXFP4)
            T.kblk = static_cast<const uint32_t*>(p.ks)[static_cast<size_t>(b) * p.N + (ld ? T.rec : 0)];
    };
    uint8_t* const tb = ktr[kTr ? wave : 0];
    auto score = [&](int ti, const Tile& T) {
        float val = -__builtin_huge_valf();
        if (T.any) {
            u32x4 kr[4];  // the lane's chunks of record n, as load_key_raw lays them out
            if constexpr (kTr) {
                // rows -> operand layout through the wave's LDS buffer (one
                // wave's LDS accesses complete in order: no wait between them)
#pragma unroll
                for (int i = 0; i < kLI; ++i) {
                    const int r = kRPI * i + lr;
                    *reinterpret_cast<u32x4*>(tb + r * kRowBytes + 16 * (lc ^ (r % kCPR))) = T.raw[i];
                }
                asm volatile("" ::: "memory");  // the reads below stay after the writes
                constexpr int kChunks = (KDT == DT_BF16) ? 4 : 2;
#pragma unroll
                for (int j = 0; j < kChunks; ++j) {
                    const int ch = g + 4 * j;
                    kr[j] = *reinterpret_cast<const u32x4*>(tb + n * kRowBytes + 16 * (ch ^ (n % kCPR)));
                }
                asm volatile("" ::: "memory");  // and before the next tile's writes
            } else {
                kr[0] = T.raw[0];
            }
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (QMX) {
                const int ksc = static_cast<int>((T.kblk >> (8 * g)) & 0xFFu);
                acc0 = mfma_mx4(qmx[0], qmxs[0], kr[0], ksc, acc0);
                acc1 = mfma_mx4(qmx[1], qmxs[1], kr[0], ksc, acc1);
            } else {
                bf16x8 bk[4];
                key_operands<KDT>(kr, KDT == DT_MXFP4 ? e8m0_to_f32(T.kblk >> (8 * g)) : 1.f, bk);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc0 = mfma16x16x32(qa[0][ks], bk[ks], acc0);
                    acc1 = mfma16x16x32(qa[1][ks], bk[ks], acc1);
                }
            }
            // an e4m3 row's scale is >= 0, so it leaves the ReLU and is
            // applied once to the head sum: relu(s d) w = s w relu(d)
            float part = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                part += wv[0][v] * relu(acc0[v]);
                part += wv[1][v] * relu(acc1[v]);
            }
            part += shfl_xor_f(part, 16);
            part += shfl_xor_f(part, 32);
            if (KDT == DT_E4M3) part *= T.kscale;
            if (T.rec >= 0 && T.rec < vis) val = part;
        }
        if (g == 0) osc[(ti - t_begin) * 16 + n] = val;
    };
    // tiles wave, wave + 4, ... of the range, through a ring of kRing
    // tiles: kRing - 1 in flight ahead of the one being multiplied (e4m3
    // tiles carry half the bytes, so more of them)
    constexpr int kRing = (KDT == DT_BF16) ? 3 : 4;  // MXFP4 tiles: a quarter of the bytes
    Tile tt[kRing];
    const int ti0 = t_begin + wave;
    if constexpr (!POOL) {
        // Every ring slot is always filled -- a tile past the range reads
        // record 0 (an L2 hit) -- so no load is conditional and the wait
        // before each tile's multiply leaves the later tiles' loads in
        // flight (with conditional prefetches the compiler's count covers
        // nearly all of them).
#pragma unroll
        for (int d = 0; d + 1 < kRing; ++d) fetch(ti0 + 4 * d, tt[d]);
        for (int base = ti0; base < t_end; base += 4 * kRing) {
#pragma unroll
            for (int d = 0; d < kRing; ++d) {
                const int ti = base + 4 * d;
                fetch(ti + 4 * (kRing - 1), tt[(d + kRing - 1) % kRing]);
                if (ti < t_end) score(ti, tt[d]);
            }
        }
    } else {
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
    }
    __syncthreads();
    const int c0 = t_begin * 16;
    const int c1 = min(t_end * 16, p.ncols);
    float* orow = p.out + row * p.ncols;
    for (int c = c0 + static_cast<int>(threadIdx.x); c < c1; c += 256) __builtin_nontemporal_store(osc[c - c0], &orow[c]);
}

// Multi-query decode scoring: several query tokens of one sequence (2 .. 8,
// e.g. the positions a speculative draft asks the model to verify, "Create
// DeepSeek from scratch", "How DSpark drafts and verifies several tokens")
// against all its records, no pool.  A key tile is loaded once, as whole
// rows through a per-wave LDS transpose as in idx_mfma_kernel (with the same
// unconditional prefetch ring), and multiplied against every token: the
// M side of the products is Tq x 32 heads, so the keys cross HBM once per
// sequence instead of once per token.  The tokens' queries sit in LDS (a
// 256-byte head row keeps its 16-byte chunk c at slot c ^ (row mod 16), so
// the 16 rows one operand read touches fill all banks) and their scores
// collect in LDS until the workgroup's column run is done.
constexpr int kMultiMax = 8;     // query tokens per sequence, at most
constexpr int kMultiTpbMax = 64; // tiles per workgroup, at most

template <int KDT>
__global__ __launch_bounds__(256) void idx_multi_kernel(IdxP p) {
    extern __shared__ __align__(16) uint8_t msh[];
    const int Tq = p.Tq;
    uint8_t* qsh = msh;                                          // [Tq][32 heads][256 B], swizzled
    float* wsh = reinterpret_cast<float*>(msh + Tq * kHi * 256);  // [Tq][32]
    float* osc = wsh + Tq * kHi;                                 // [Tq][tpb * 16]
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;
    constexpr int kCPR = kRowBytes / 16;  // 16-byte chunks per key row
    constexpr int kRPI = 64 / kCPR;       // rows per 1 KiB load
    constexpr int kLI = 16 / kRPI;        // loads per 16-row tile
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int lr = lane / kCPR;  // the lane's row within a load
    const int lc = lane % kCPR;  // and its chunk
    // per-wave tile transpose, after the scores
    uint8_t* const tb = reinterpret_cast<uint8_t*>(osc + Tq * p.tiles_per_block * 16) + wave * 16 * kRowBytes;
    const int b = blockIdx.y;
    const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
    const int tpb = p.tiles_per_block;

    // the tokens' queries and head weights into LDS
    for (int c = tid; c < Tq * kHi * 16; c += 256) {
        const int r = c >> 4, ch = c & 15;  // head row (token * 32 + head), chunk
        const u32x4 v = *reinterpret_cast<const u32x4*>(p.q + (static_cast<size_t>(b) * Tq * kHi + r) * kDi + 8 * ch);
        *reinterpret_cast<u32x4*>(qsh + r * 256 + 16 * (ch ^ (r & 15))) = v;
    }
    for (int c = tid; c < Tq * kHi; c += 256) wsh[c] = p.w[static_cast<size_t>(b) * Tq * kHi + c];
    __shared__ int vsh[kMultiMax];  // records each token may see
    if (tid < kMultiMax) vsh[tid] = tid < Tq ? visible_count(p.q_pos[static_cast<size_t>(b) * Tq + tid], p.m, nrec) : 0;
    __syncthreads();
    int vmax = 0;
    for (int t = 0; t < Tq; ++t) vmax = max(vmax, vsh[t]);

    const int ntiles = (p.ncols + 15) / 16;
    const int t_begin = blockIdx.x * tpb;
    const int t_end = min(ntiles, t_begin + tpb);
    const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;

    struct Tile {
        int rec;
        bool any;
        u32x4 raw[4];
        float kscale;
    };
    const int lim = min(vmax, t_end * 16);  // records this workgroup reads (vmax <= N = ncols)
    auto fetch = [&](int ti, Tile& T) {
        const int c = ti * 16 + n;
        T.rec = c;
        const bool ld = c < lim;
        T.any = ti * 16 < lim;
        // whole rows (a row no token may see is read from record 0)
#pragma unroll
        for (int i = 0; i < kLI; ++i) {
            const int rr = ti * 16 + kRPI * i + lr;
            T.raw[i] = ld16_nt(reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(rr < lim ? rr : 0) * kRowBytes) + lc);
        }
        T.kscale = 1.f;
        if (KDT == DT_E4M3) T.kscale = static_cast<const float*>(p.ks)[static_cast<size_t>(b) * p.N + (ld ? c : 0)];
    };
    auto score = [&](int ti, const Tile& T) {
        bf16x8 bk[4];
        if (T.any) {
            // rows -> operand layout through the wave's LDS buffer
#pragma unroll
            for (int i = 0; i < kLI; ++i) {
                const int r = kRPI * i + lr;
                *reinterpret_cast<u32x4*>(tb + r * kRowBytes + 16 * (lc ^ (r % kCPR))) = T.raw[i];
            }
            asm volatile("" ::: "memory");  // the reads below stay after the writes
            u32x4 kr[4];
            constexpr int kChunks = (KDT == DT_BF16) ? 4 : 2;
#pragma unroll
            for (int j = 0; j < kChunks; ++j) {
                const int ch = g + 4 * j;
                kr[j] = *reinterpret_cast<const u32x4*>(tb + n * kRowBytes + 16 * (ch ^ (n % kCPR)));
            }
            asm volatile("" ::: "memory");  // and before the next tile's writes
            key_operands<KDT>(kr, 1.f, bk);
        }
        for (int t = 0; t < Tq; ++t) {
            float val = -__builtin_huge_valf();
            if (T.any) {
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
                const uint8_t* q0 = qsh + (t * kHi + n) * 256;       // head n (m-tile 0)
                const uint8_t* q1 = q0 + 16 * 256;                    // head 16 + n
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int ch = chunk8<KDT>(g, ks) ^ n;           // rows n and 16 + n share the swizzle
                    acc0 = mfma16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(q0 + 16 * ch)), bk[ks], acc0);
                    acc1 = mfma16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(q1 + 16 * ch)), bk[ks], acc1);
                }
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(wsh + t * kHi + 4 * g);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(wsh + t * kHi + 16 + 4 * g);
                float part = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    part += w0[v] * relu(acc0[v]);
                    part += w1[v] * relu(acc1[v]);
                }
                part += shfl_xor_f(part, 16);
                part += shfl_xor_f(part, 32);
                if (KDT == DT_E4M3) part *= T.kscale;
                if (T.rec >= 0 && T.rec < vsh[t]) val = part;
            }
            if (g == 0) osc[t * tpb * 16 + (ti - t_begin) * 16 + n] = val;
        }
    };
    constexpr int kRing = (KDT == DT_BF16) ? 3 : 4;
    Tile tt[kRing];
    const int ti0 = t_begin + wave;
    // every ring slot is always filled (tiles past the range read record 0)
#pragma unroll
    for (int d = 0; d + 1 < kRing; ++d) fetch(ti0 + 4 * d, tt[d]);
    for (int base = ti0; base < t_end; base += 4 * kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            const int ti = base + 4 * d;
            fetch(ti + 4 * (kRing - 1), tt[(d + kRing - 1) % kRing]);
            if (ti < t_end) score(ti, tt[d]);
        }
    }
    __syncthreads();
    const int c0 = t_begin * 16;
    const int c1 = min(t_end * 16, p.ncols);
    for (int t = 0; t < Tq; ++t) {
        float* orow = p.out + (static_cast<size_t>(b) * Tq + t) * p.ncols;
        for (int c = c0 + tid; c < c1; c += 256) __builtin_nontemporal_store(osc[t * tpb * 16 + c - c0], &orow[c]);
    }
}

// Prefill scoring: many query tokens of one sequence against the records
// they may see -- a causal GEMM (tokens x heads) x 128 x records with a
// ReLU and weighted head-sum epilogue.
//
// Tokens are stationary: a workgroup of 8 waves takes a block of 8
// consecutive tokens of one sequence, one token per wave, whose query
// fragments stay in registers, and streams the key rows the block can see
// through LDS in tiles of 64 records.  Blocks are numbered by position, and
// workgroup w takes blocks nb-1-w and w: under causal visibility every
// workgroup then has about the same number of tiles.  32x32x16 MFMAs:
// M = the 32 heads of the token, N = 32 records, K = 128 dims in 8 k-steps.
// Lane group kg takes dims 64 kg + 8 ks .. +7 at k-step ks in both
// operands.  After the epilogue one lane swap leaves lane l holding the
// score of record 64 k + l of tile k; a wave keeps eight tiles' scores in
// registers and then stores them.
//
// Memory: the block's queries and head weights, and the key tiles, are
// copied global -> LDS with global_load_lds (e4m3 key rows go through
// registers and are converted exactly to bf16); the second block's queries
// are copied while the first block runs.  Tiles come in periods of two, one
// barrier each, the next period's copies in flight during the current one.
// In LDS a 256-byte row (one head's query, one record's key) keeps its
// 16-byte chunk c at slot c ^ (r mod 16), so the 16 rows that one phase of
// an operand read touches fill all banks.
constexpr int kPWaves = 8;               // waves per workgroup = tokens per block
constexpr int kPTile = 64;               // records per tile
constexpr int kPRing = 4;                // tile buffers: two periods of two tiles
constexpr int kPRowB = kDi * 2;          // bytes per LDS row (bf16)
constexpr int kPChunk = 8;               // tiles whose scores are stored together
constexpr int kPQBytes = kHi * kPRowB;   // one token's queries

__device__ __forceinline__ uint32_t lds_u32(const void* ptr) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((const __attribute__((address_space(3))) uint8_t*)(ptr)));
}

// One 1 KiB global -> LDS copy: lane l moves the 16 bytes at base + off to
// LDS byte address lds + 16 l (gfx950 global_load_lds_dwordx4, LDS address
// in M0).  Completion is awaited with explicit vmcnt waits.
__device__ __forceinline__ void copy_lds16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}

template <int KDT>
__global__ __launch_bounds__(kPWaves * 64, 1) void idx_prefill_kernel(IdxP p, int nb) {
    __shared__ __align__(16) uint8_t kt[kPRing][kPTile * kPRowB];
    __shared__ __align__(16) uint8_t qs[kPWaves][kPQBytes];
    __shared__ __align__(16) float wsh[kPWaves][kHi];
    __shared__ float kst[kPRing][kPTile];  // e4m3 row scales
    constexpr int kRowBytes = (KDT == DT_BF16) ? kDi * 2 : kDi;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;   // record within a set (B and C column), head (A row)
    const int kg = lane >> 5;  // k group
    const int sw = j & 15;     // chunk swizzle of rows j and 32 + j
    const int w0 = static_cast<int>(blockIdx.x);
    // a heavy block, then a light one (whose queries arrive meanwhile)
    const int npass = nb - 1 - w0 > w0 ? 2 : 1;
    const int jbs[2] = {nb - 1 - w0, w0};

    // queries of block jb -> LDS (wave w: token t0 + w, eight 4-row
    // copies), and wave 0 the eight tokens' head weights (one copy)
    auto qcopy = [&](int jb) {
        const int b = jb % p.B;
        const int t0 = (jb / p.B) * kPWaves;
        const size_t row0 = static_cast<size_t>(b) * p.Tq;
        const int tq = min(t0 + wave, p.Tq - 1);  // past the end: a valid row, never stored
        const uint16_t* qrow = p.q + (row0 + tq) * kHi * kDi;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            copy_lds16(qrow, static_cast<uint32_t>(r * kPRowB + 16 * ((lane & 15) ^ (r & 15))),
                       lds_u32(&qs[wave][0]) + i * 4 * kPRowB);
        }
        if (wave == 0) {
            const int tw = min(t0 + (lane >> 3), p.Tq - 1) - t0;
            copy_lds16(p.w + (row0 + t0) * kHi, static_cast<uint32_t>((tw * kHi + 4 * (lane & 7)) * 4), lds_u32(&wsh[0][0]));
        }
    };
    qcopy(jbs[0]);

#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            if (npass < 2) break;
            lds_sync_all();  // every wave is done with the previous block's tiles
        }
        const int jb = jbs[pass];
        const int b = jb % p.B;
        const int t0 = (jb / p.B) * kPWaves;
        const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
        const size_t row0 = static_cast<size_t>(b) * p.Tq;
        // visibility: lane i (mod 8) holds token t0 + i's; the block's tiles
        // cover the most that any of its tokens sees
        const int ti = t0 + (lane & 7);
        const int vis_l = ti < p.Tq ? visible_count(p.q_pos[row0 + ti], p.m, nrec) : 0;
        int vmax = vis_l;
        vmax = max(vmax, __shfl_xor(vmax, 1));
        vmax = max(vmax, __shfl_xor(vmax, 2));
        vmax = max(vmax, __shfl_xor(vmax, 4));
        vmax = __builtin_amdgcn_readfirstlane(vmax);
        const int nt = (min(vmax, p.ncols) + kPTile - 1) / kPTile;
        const int t = t0 + wave;
        const bool live = t < p.Tq;
        const int vis = __builtin_amdgcn_readlane(vis_l, wave);
        const uint8_t* kbase = p.k + static_cast<size_t>(b) * p.N * kRowBytes;

        // bf16 key tile k -> buffer k % kPRing: wave w copies rows 8w .. 8w+7
        // (two 4-row copies; lane l takes row 4i + l/16, chunk slot l % 16)
        auto issue = [&](int k) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * wave + ii;
                const int r = 4 * i + (lane >> 4);
                const int rec0 = k * kPTile;
                const int rr = min(rec0 + r, p.N - 1) - rec0;  // rows past N repeat the last (masked)
                copy_lds16(kbase + static_cast<size_t>(rec0) * kRowBytes,
                           static_cast<uint32_t>(rr * kRowBytes + 16 * ((lane & 15) ^ (r & 15))),
                           lds_u32(&kt[k % kPRing][0]) + i * 4 * kPRowB);
            }
        };
        // e4m3 key tiles: thread tid stages 16 dims (two chunks) of row
        // tid / 8, threads 0..63 the row scales; even and odd tiles have a
        // register set each
        u32x4 eraw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        float esc[2] = {0.f, 0.f};
        auto eload = [&](int k, int par) {
            const int r = tid >> 3;
            const int rec = min(k * kPTile + r, p.N - 1);
            eraw[par] = *reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(rec) * kRowBytes + 16 * (tid & 7));
            if (tid < kPTile)
                esc[par] = static_cast<const float*>(p.ks)[static_cast<size_t>(b) * p.N + min(k * kPTile + tid, p.N - 1)];
        };
        auto eland = [&](int k, int par) {
            const int r = tid >> 3;
            const int c = 2 * (tid & 7);
            uint8_t* row = &kt[k % kPRing][r * kPRowB];
            *reinterpret_cast<u32x4*>(row + 16 * (c ^ (r & 15))) = e4m3x8_to_bf16x8(u32x2{eraw[par][0], eraw[par][1]});
            *reinterpret_cast<u32x4*>(row + 16 * ((c + 1) ^ (r & 15))) = e4m3x8_to_bf16x8(u32x2{eraw[par][2], eraw[par][3]});
            if (tid < kPTile) kst[k % kPRing][tid] = esc[par];
        };
        // Period of tiles k, k+1 (k even, > 0): its tiles are visible to
        // every wave after the barrier; the next period's tiles go out
        // into the buffers of the previous period.
        auto period = [&](int k) {
            if constexpr (KDT == DT_BF16) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                lds_sync_all();
                if (k + 2 < nt) issue(k + 2);
                if (k + 3 < nt) issue(k + 3);
            } else {
                lds_sync_all();
                if (k + 2 < nt) eland(k + 2, 0);
                if (k + 3 < nt) eland(k + 3, 1);
                if (k + 4 < nt) eload(k + 4, 0);
                if (k + 5 < nt) eload(k + 5, 1);
            }
        };

        // Period 0: tiles 0, 1 and the queries land; the fragments move to
        // registers; the next block's queries and the tiles of period 1 go out.
        if constexpr (KDT == DT_BF16) {
            if (nt > 0) issue(0);
            if (nt > 1) issue(1);
        } else {
            if (nt > 0) eload(0, 0);
            if (nt > 1) eload(1, 1);
            if (nt > 0) eland(0, 0);
            if (nt > 1) eland(1, 1);
            if (nt > 2) eload(2, 0);
            if (nt > 3) eload(3, 1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_sync_all();
        bf16x8 qa[8];
        float wv[16];
        {
            const uint8_t* qr = &qs[wave][j * kPRowB];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * ((8 * kg + ks) ^ sw)));
            // weights of this lane's 16 heads: 8 (v / 4) + 4 kg + v % 4
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(&wsh[wave][8 * q4 + 4 * kg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[4 * q4 + e] = w4[e];
            }
        }
        if (pass == 0 && npass == 2) {
            lds_sync_all();  // every wave holds its fragments: the query buffer is free
            qcopy(jbs[1]);
        }
        if constexpr (KDT == DT_BF16) {
            if (nt > 2) issue(2);
            if (nt > 3) issue(3);
        } else {
            if (nt > 2) eland(2, 0);
            if (nt > 3) eland(3, 1);
            if (nt > 4) eload(4, 0);
            if (nt > 5) eload(5, 1);
        }

        // epilogue of a tile's MFMA results: lane l gets the score of record
        // 64k + l
        auto epi = [&](int k, const f32x16 (&c)[2], float scl) -> float {
            float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s0[v & 3] = fmaf(wv[v], relu(c[0][v]), s0[v & 3]);
                s1[v & 3] = fmaf(wv[v], relu(c[1][v]), s1[v & 3]);
            }
            const float a0 = (s0[0] + s0[1]) + (s0[2] + s0[3]);
            const float a1 = (s1[0] + s1[1]) + (s1[2] + s1[3]);
            // lanes 0..31 finish set 0 (records 64k + l), lanes 32..63 set 1
            const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
            float tot = __uint_as_float(rs[0]) + __uint_as_float(rs[1]);
            if constexpr (KDT == DT_E4M3) tot *= scl;  // the row scale is >= 0: it commutes with the ReLU
            return k * kPTile + lane < vis ? tot : -__builtin_huge_valf();
        };
        // MFMAs of tile k (set 0: rows j, set 1: rows 32 + j) with the
        // epilogue of tile kp (results cp, row scale sp) spread between them:
        // all operand reads first, then one MFMA and four VALU instructions at
        // a time.  The row scale of tile k is read now, before the barrier
        // that lets its buffer be refilled.
        auto mma_epi = [&](int k, f32x16 (&c)[2], float& scl, int kp, const f32x16 (&cp)[2], float sp) -> float {
            if constexpr (KDT == DT_E4M3) scl = kst[k % kPRing][lane];
            const uint8_t* r0p = &kt[k % kPRing][j * kPRowB];
            const uint8_t* r1p = r0p + 32 * kPRowB;
            bf16x8 bop[8][2];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int cs = 16 * ((8 * kg + ks) ^ sw);
                bop[ks][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(r0p + cs));
                bop[ks][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(r1p + cs));
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) c[0][v] = c[1][v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                c[0] = mfma32x32x16(qa[ks], bop[ks][0], c[0]);
                c[1] = mfma32x32x16(qa[ks], bop[ks][1], c[1]);
            }
            const float e = epi(kp, cp, sp);
            __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
            }
            return e;
        };

        // Tile k's MFMAs and tile k-1's epilogue form one block, so the
        // epilogue's VALU work fills the matrix pipeline's shadow.
        float* orow = p.out + (row0 + (live ? t : t0)) * p.ncols;
        float sc[kPChunk];
        auto flush = [&](int kb, int cnt) {  // scores of tiles kb .. kb+cnt-1
            if (live) {
#pragma unroll
                for (int u = 0; u < kPChunk; ++u) {
                    const int c = (kb + u) * kPTile + lane;
                    if (u < cnt && c < p.ncols) __builtin_nontemporal_store(sc[u], &orow[c]);
                }
            }
        };
        f32x16 cc[2][2];
        float cscl[2] = {1.f, 1.f};  // e4m3 row scale of the record each lane scores
        for (int k0 = 0; k0 < nt; k0 += kPChunk) {
#pragma unroll
            for (int i = 0; i < kPChunk; ++i) {
                const int k = k0 + i;
                if (k < nt) {
                    if ((i & 1) == 0 && k > 0) period(k);
                    // (for k = 0 the epilogue runs on stale registers; unused)
                    const float e = mma_epi(k, cc[i & 1], cscl[i & 1], k - 1, cc[(i + 1) & 1], cscl[(i + 1) & 1]);
                    if (k > 0) sc[(i + kPChunk - 1) % kPChunk] = e;
                    if (i == 0 && k > 0) flush(k0 - kPChunk, kPChunk);
                    if (k == nt - 1) {
                        sc[i] = epi(k, cc[i & 1], cscl[i & 1]);
                        flush(k0, i + 1);
                    }
                }
            }
        }
        // columns past the block's tiles: nothing there is visible
        if (live)
            for (int c = nt * kPTile + lane; c < p.ncols; c += 64) __builtin_nontemporal_store(-__builtin_huge_valf(), &orow[c]);
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

template <int KDT, bool QMX = false>
int launch_mfma(const IndexArgs& a, int tiles_per_block, hipStream_t st) {
    IdxP p;
    p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.m = a.m; p.ncols = a.ncols; p.P = a.P; p.blk = a.blk;
    p.q = static_cast<const uint16_t*>(a.q_idx);
    p.qsc = static_cast<const uint8_t*>(a.q_scale);
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
    if (a.pool) hipLaunchKernelGGL((idx_mfma_kernel<KDT, QMX, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((idx_mfma_kernel<KDT, QMX, false>), grid, dim3(256), 0, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

bool index_scores_mfma_ok(const IndexArgs& a) {
    if (a.Hi != kHi || a.Di != kDi) return false;
    if (a.k_dtype == DT_MXFP4) return a.q_dtype == DT_BF16 || a.q_dtype == DT_MXFP4;
    return a.q_dtype == DT_BF16 && (a.k_dtype == DT_BF16 || a.k_dtype == DT_E4M3);
}

int launch_index_scores(const IndexArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (index_scores_mfma_ok(a)) {
        const int ntiles = (a.ncols + 15) / 16;
        const int rows = a.B * a.Tq;
        // Prefill-shaped work (many tokens of one sequence, no pool): blocks of
        // 8 tokens, two blocks (a light and a heavy one) per workgroup.
        if (!a.pool && a.Tq >= 16 && a.k_dtype != DT_MXFP4) {
            IdxP p;
            p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.m = a.m; p.ncols = a.ncols; p.P = a.P; p.blk = a.blk;
            p.q = static_cast<const uint16_t*>(a.q_idx);
            p.qsc = nullptr;
            p.w = a.w;
            p.k = static_cast<const uint8_t*>(a.k_idx);
            p.ks = a.k_scale;
            p.q_pos = a.q_pos;
            p.n_rec = a.n_rec;
            p.pool = nullptr;
            p.out = a.scores;
            p.tiles_per_block = 0;
            const int nb = a.B * ((a.Tq + kPWaves - 1) / kPWaves);
            const dim3 grid((nb + 1) / 2);
            if (a.k_dtype == DT_BF16)
                hipLaunchKernelGGL(idx_prefill_kernel<DT_BF16>, grid, dim3(kPWaves * 64), 0, st, p, nb);
            else
                hipLaunchKernelGGL(idx_prefill_kernel<DT_E4M3>, grid, dim3(kPWaves * 64), 0, st, p, nb);
            return static_cast<int>(hipGetLastError());
        }
        // Several decode tokens per sequence (and no pool): each key tile is
        // read once for all of them.  Tiles per workgroup: the largest that
        // still gives >= 512 workgroups.
        if (!a.pool && a.Tq >= 2 && a.Tq <= kMultiMax && a.q_dtype == DT_BF16 && a.k_dtype != DT_MXFP4) {
            int tpb = kMultiTpbMax;
            while (tpb > 4 && static_cast<long>(a.B) * ((ntiles + tpb - 1) / tpb) < 512) tpb >>= 1;
            IdxP p;
            p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.m = a.m; p.ncols = a.ncols; p.P = 0; p.blk = 0;
            p.q = static_cast<const uint16_t*>(a.q_idx);
            p.qsc = nullptr;
            p.w = a.w;
            p.k = static_cast<const uint8_t*>(a.k_idx);
            p.ks = a.k_scale;
            p.q_pos = a.q_pos;
            p.n_rec = a.n_rec;
            p.pool = nullptr;
            p.out = a.scores;
            p.tiles_per_block = tpb;
            const size_t lds = static_cast<size_t>(a.Tq) * (kHi * 256 + kHi * 4 + tpb * 16 * 4) +
                               4 * 16 * static_cast<size_t>(a.k_dtype == DT_BF16 ? kDi * 2 : kDi);
            const dim3 grid((ntiles + tpb - 1) / tpb, a.B);
            if (a.k_dtype == DT_BF16)
                hipLaunchKernelGGL(idx_multi_kernel<DT_BF16>, grid, dim3(256), lds, st, p);
            else
                hipLaunchKernelGGL(idx_multi_kernel<DT_E4M3>, grid, dim3(256), lds, st, p);
            return static_cast<int>(hipGetLastError());
        }
        // Decode rows: the largest tiles per block that still gives >= 512
        // blocks (two per CU), so each wave streams many tiles and the
        // start-up latency is paid rarely.  (Measured on the 64-row bf16
        // decode: two blocks per CU beat four, 57 -> 53 us; one per CU is
        // slower again.)
        int tpb = kDecTpbMax;
        while (tpb > 4 && static_cast<long>(rows) * ((ntiles + tpb - 1) / tpb) < 512) tpb >>= 1;
        if (a.k_dtype == DT_MXFP4)
            return a.q_dtype == DT_MXFP4 ? launch_mfma<DT_MXFP4, true>(a, tpb, st) : launch_mfma<DT_MXFP4>(a, tpb, st);
        return a.k_dtype == DT_BF16 ? launch_mfma<DT_BF16>(a, tpb, st) : launch_mfma<DT_E4M3>(a, tpb, st);
    }
    IdxG p;
    p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.Hi = a.Hi; p.Di = a.Di; p.m = a.m; p.ncols = a.ncols;
    p.P = a.P; p.blk = a.blk; p.qdt = a.q_dtype; p.kdt = a.k_dtype;
    p.q = a.q_idx; p.w = a.w; p.k = a.k_idx; p.q_pos = a.q_pos;
    p.n_rec = a.n_rec; p.pool = a.pool; p.out = a.scores;
    p.ks = static_cast<const float*>(a.k_scale);
    dim3 grid((a.ncols + 255) / 256, a.B * a.Tq);
    const size_t lds = (static_cast<size_t>(a.Hi) * a.Di + a.Hi) * sizeof(float);
    hipLaunchKernelGGL(idx_generic_kernel, grid, dim3(256), lds, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
