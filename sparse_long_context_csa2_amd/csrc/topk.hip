// Top-K record selection and the hierarchical block pool.
//
// Top-K returns the addresses of the K best records, never their scores
// ("Create DeepSeek from scratch", lesson 06, worked example and unit test):
// preference is score descending, then record id ascending.  Exact ties
// really occur (a ReLU sum is exactly 0 whenever every head's product is
// negative), so the tie-break is part of the result.
//
// Every element has the 64-bit composite key (score_key(score) << 32 |
// ~record_id); with unique record ids the keys are unique, and "the K
// largest composite keys" is exactly the required set.  Selection runs in
// two levels:
//  1. a 4096-bin histogram of the top 12 key bits (sign, exponent, 3
//     mantissa bits) finds the boundary bin B*: fewer than K elements lie
//     in higher bins, which are all chosen;
//  2. an exact 8-bit-digit radix select over the composite keys of the
//     boundary bin's elements (usually a few dozen) picks the rest.
// All bin searches are parallel block scans.
//
// Rows of up to 4096 columns (score order only for K <= 64): one wave per
// row, keys in registers, the boundary key by binary search over key
// values.  Other rows of up to 4096 columns: one 256-thread workgroup per
// row with the keys cached in LDS.
// Longer rows whose candidates fit one row (sub-rows x K <= 16384, no
// score order): two passes of the one-workgroup row kernel.  The first
// keeps each 8192-column sub-row's K best (key, record) pairs, in column
// order; the second selects the row's K best among them.  This is exact:
// the composite keys are a strict order, so each of the row's K best is
// among the K best of its own sub-row.  The scores are read once, and no
// workspace has to start cleared.
// Other long rows: the row is split into 4096-column chunks over many
// workgroups.  A histogram kernel accumulates the row histogram (LDS-
// private per workgroup, merged with global atomics after a kernel that
// clears it; rows of at most four chunks instead keep each chunk's
// histogram, which the select kernel sums, and need no clearing).  A
// select kernel then classifies each chunk -- keys above the boundary bin
// are chosen outright, keys inside it are candidates -- places both lists
// with one block scan and appends them to the row's with one atomic.  The last
// workgroup to finish a row (atomic ticket) resolves the boundary bin
// exactly and writes the row, sorted in LDS.  Output ids are sorted by
// column, so results are deterministic whatever the order in which
// workgroups ran.
//
// The block pool scores block b by the maximum of its members ("DeepSeek
// V4.1-Flash. Every layer, connected.", hierarchy caption) -- one wave per
// block -- then runs the same selection on the block maxima with the
// output ordered by (block maximum desc, block id asc).
#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kNT = 256;             // threads per workgroup
constexpr int kNW = kNT / kWave;     // waves per workgroup
constexpr int kBins = 4096;          // first-level bins: key >> 20
constexpr int kBinShift = 20;
constexpr int kSmallCols = 4096;     // short rows: one workgroup per row
constexpr int kChunk = 4096;         // columns per workgroup on long rows
constexpr int kCandCap = 2048;       // boundary candidates held in LDS
constexpr int kMaxK = 2048;
constexpr int kFewChunks = 4;        // rows of up to this many chunks keep per-chunk histograms

struct TopkP {
    int rows, ncols, K, P, blk, nchunks;
    const float* scores;
    const int32_t* pool;
    int32_t* idx;
    int sort_by_key;
    // long-row workspace
    int* ghist;      // [rows][kBins]: histogram of the keys' top 12 bits; with at most
                     // kFewChunks chunks per row, [rows][nchunks][kBins]: each chunk's own
    int* cnt;        // [rows][4]: finished chunks (word 2)
    int* ccnt;       // [rows][nchunks]: entries of each chunk
    uint32_t* ckey;  // [rows][ncols]: entries (key, column) -- keys in the boundary bin or above,
    int* ccol;       //   chunk c's at [c kChunk, c kChunk + count), in column order
    // two-pass rows: [rows][nchunks][K] keys and record ids of each
    // sub-row's K best, in column order (key 0 and id -1 pad a short list)
    uint32_t* cand_k;
    int32_t* cand_i;
};

__device__ __forceinline__ int rec_of(const TopkP& p, const int32_t* prow, int c) {
    if (!prow) return c;
    const int pb = prow[c / p.blk];
    return pb < 0 ? -1 : pb * p.blk + c % p.blk;
}


// Keys of columns c0 + i * kNT + threadIdx.x, i < N (0 past c1).  All
// loads are issued before any key is formed: branches between a load and
// the next would make each load wait for the one before.
template <int N>
__device__ __forceinline__ void load_keys(const TopkP& p, const int32_t* prow, const float* srow, int c0, int c1,
                                          uint32_t (&kk)[N]) {
    float sv[N];
    int pv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) sv[i] = srow[min(c0 + i * kNT + static_cast<int>(threadIdx.x), c1 - 1)];
    if (prow) {  // one uniform branch around all the pool loads
#pragma unroll
        for (int i = 0; i < N; ++i) pv[i] = prow[min(c0 + i * kNT + static_cast<int>(threadIdx.x), c1 - 1) / p.blk];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) pv[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = c0 + i * kNT + static_cast<int>(threadIdx.x);
        const uint32_t k = score_key(sv[i]);
        kk[i] = (c < c1 && pv[i] >= 0) ? k : 0u;
    }
}

__device__ __forceinline__ unsigned long long composite(uint32_t key, int rec) {
    return (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(rec));
}

struct Scan {
    int wave_tot[kNW];
    int res[3];
};

// Exclusive prefix sum over the block (thread order); returns this
// thread's exclusive prefix, and the block total in *total.
__device__ int block_excl_scan(int v, Scan& s, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s.wave_tot[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
        if (i < wave) off += s.wave_tot[i];
        tot += s.wave_tot[i];
    }
    *total = tot;
    return off + x - v;
}

// Finds, scanning bins from the top, the bin where the running count first
// reaches `need`; returns it and sets *rest to the number still needed
// from that bin.  hist has nbins = kNT * PER entries.  If the total is
// below `need` the result is -1 (everything is chosen).
template <int PER>
__device__ int find_from_top(const int* hist, int need, Scan& s, int* rest, int* bin_count = nullptr) {
    int loc[PER];
    int sum = 0;
    const int top = kNT * PER - 1 - threadIdx.x * PER;  // this thread's highest bin
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        loc[j] = hist[top - j];
        sum += loc[j];
    }
    int total;
    const int excl = block_excl_scan(sum, s, &total);
    if (threadIdx.x == 0) { s.res[0] = -1; s.res[1] = 0; s.res[2] = 0; }
    __syncthreads();
    if (excl < need && excl + sum >= need) {
        int acc = excl;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (acc + loc[j] >= need) {
                s.res[0] = top - j;
                s.res[1] = need - acc;
                s.res[2] = loc[j];
                break;
            }
            acc += loc[j];
        }
    }
    __syncthreads();
    const int bin = s.res[0];
    *rest = s.res[1];
    if (bin_count) *bin_count = s.res[2];
    __syncthreads();
    return bin;
}

// Exact radix select of the `need` largest composite keys among the
// elements src(i) yields, i in [0, count).  Returns the threshold:
// chosen = composite >= thr.  src(i, key, rec) returns false to skip.
// The digits above `shift0` must be the same for all elements (`known`
// holds them; bits of `known` below those digits are ignored).
template <class Src>
__device__ unsigned long long radix_select(Src src, int count, int need, int* hist8, Scan& s,
                                           int shift0 = 56, unsigned long long known = 0) {
    unsigned long long mask = shift0 >= 56 ? 0ull : ~0ull << (shift0 + 8);
    unsigned long long prefix = known & mask;
    for (int shift = shift0; shift >= 0; shift -= 8) {
        // stop as soon as the remaining prefix class holds exactly `need`
        hist8[threadIdx.x] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < count; i += kNT) {
            uint32_t key;
            int rec;
            if (!src(i, key, rec)) continue;
            const unsigned long long ck = composite(key, rec);
            if ((ck & mask) == prefix) atomicAdd(&hist8[(ck >> shift) & 255], 1);
        }
        __syncthreads();
        int rest, cnt_d;
        const int d = find_from_top<1>(hist8, need, s, &rest, &cnt_d);
        prefix |= static_cast<unsigned long long>(d) << shift;
        mask |= 255ull << shift;
        if (cnt_d == rest) {
            need = rest;
            break;  // the whole digit class is chosen: threshold is its prefix
        }
        need = rest;
    }
    return prefix;
}

// ---------------------------------------------------------------- rows <= 4096, one wave each

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const int lo = __shfl_xor(static_cast<int>(v & 0xFFFFFFFFull), m, kWave);
    const int hi = __shfl_xor(static_cast<int>(v >> 32), m, kWave);
    return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// One wave per row, the row's keys in registers: lane l owns columns
// 64 i + l, so each load instruction reads 256 contiguous bytes.  The K-th
// largest score key k* comes from a 32-step binary search over key values,
// counting with ballots (no cross-lane data movement); every key above k*
// is chosen, and of the keys equal to k* the ones with the smallest record
// ids (the larger composite keys): in the lowest columns without a pool,
// by a second binary search over record ids with one.  Column order comes
// from ballot prefixes; score order (K <= 64) from a bitonic sort across
// the wave's lanes.
__device__ __forceinline__ uint32_t warp_min_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave)));
    return v;
}
__device__ __forceinline__ uint32_t warp_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave)));
    return v;
}

template <int KPL, bool POOL>
__global__ __launch_bounds__(kNT) void topk_wave_kernel(TopkP p) {
    __shared__ unsigned long long slot[kNW][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kNW + wave;
    if (row >= p.rows) return;
    const int n = p.ncols;
    const int K = p.K;
    const float* srow = p.scores + static_cast<size_t>(row) * n;
    const int32_t* prow = POOL ? p.pool + static_cast<size_t>(row) * p.P : nullptr;
    int32_t* orow = p.idx + static_cast<size_t>(row) * K;
    uint32_t kk[KPL];
    int rr[KPL];  // record ids (the column itself without a pool)
    {
        float sv[KPL];
        int pv[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) sv[i] = srow[min(64 * i + lane, n - 1)];  // all loads at once
        if constexpr (POOL) {
#pragma unroll
            for (int i = 0; i < KPL; ++i) pv[i] = prow[min(64 * i + lane, n - 1) / p.blk];
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int c = 64 * i + lane;
            rr[i] = POOL ? (pv[i] < 0 ? -1 : pv[i] * p.blk + c % p.blk) : c;
            kk[i] = (c < n && rr[i] >= 0) ? score_key(sv[i]) : 0u;
        }
    }
    auto count_ge = [&](uint32_t x) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) c += __popcll(__ballot(kk[i] >= x));
        return c;
    };
    const int nvalid = count_ge(1u);
    uint32_t kstar = 1u;  // with nvalid <= K every valid key is chosen
    int need_tie = KPL * 64;
    if (nvalid > K) {
        // Largest x with count(key >= x) >= K.  The K-th key lies between
        // the smallest and the largest valid key, so the bits above their
        // highest differing bit are known; and once a probe counts exactly
        // K keys at or above it, those K keys are the selection (every key
        // equal to the probe is then needed), so the search can stop.
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            if (kk[i]) lo = min(lo, kk[i]);
            hi = max(hi, kk[i]);
        }
        lo = warp_min_u32(lo);
        hi = warp_max_u32(hi);
        const uint32_t diff = lo ^ hi;
        const int top = diff ? 31 - __builtin_clz(diff) : -1;
        uint32_t x = top >= 0 ? (hi & ~((2u << top) - 1u)) : hi;  // the common prefix (<= lo)
        if (top == 31) x = 0u;
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t cand = x | (1u << bit);
            const int c = count_ge(cand);
            if (c >= K) x = cand;
            if (c == K) break;
        }
        kstar = x;
        need_tie = K - (kstar == 0xFFFFFFFFu ? 0 : count_ge(kstar + 1u));  // keys equal to k* still needed
    }
    int rstar = 0x7FFFFFFF;  // with a pool: ties chosen when rec <= rstar
    if (POOL && nvalid > K) {
        // the need_tie-th smallest record id among the ties
        auto ties_below = [&](int y) {
            int c = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i) c += __popcll(__ballot(kk[i] == kstar && rr[i] < y));
            return c;
        };
        int r = 0;
        for (int bit = 30; bit >= 0; --bit)
            if (ties_below(r + (1 << bit)) < need_tie) r += 1 << bit;
        rstar = r;
    }
    // column order: row i of the register array holds columns 64 i .. 64 i + 63
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0, tseen = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const unsigned long long tie = __ballot(kk[i] == kstar);
        const bool tie_in = POOL ? rr[i] <= rstar : tseen + __popcll(tie & below) < need_tie;
        const bool ch = kk[i] > kstar || (((tie >> lane) & 1ull) && tie_in);
        const unsigned long long cm = __ballot(ch);
        if (ch) {
            const int pos = base + __popcll(cm & below);
            if (p.sort_by_key) slot[wave][pos] = composite(kk[i], rr[i]);  // pos < K <= 64
            else orow[pos] = rr[i];
        }
        base += __popcll(cm);
        tseen += __popcll(tie);
    }
    if (p.sort_by_key) {
        __builtin_amdgcn_wave_barrier();
        unsigned long long v = lane < base ? slot[wave][lane] : 0ull;
        for (int k = 2; k <= 64; k <<= 1)
            for (int j = k >> 1; j > 0; j >>= 1) {
                const unsigned long long o = shfl_xor_u64(v, j);
                const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
                v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
            }
        if (lane < K) orow[lane] = lane < base ? static_cast<int32_t>(~static_cast<uint32_t>(v)) : -1;
        return;
    }
    for (int i = base + lane; i < K; i += kWave) orow[i] = -1;
}

// ---------------------------------------------------------------- rows <= 4096

// Ordered compaction of a block's flagged columns, taken in rounds: thread
// t holds the flag of column r * kNT + t in round r.  Each wave counts a
// round with one ballot; one wave scans the R * kNW counts in (round, wave)
// order; emit(r, pos) then gets each flagged column's place in column
// order.  Strided columns keep the LDS reads around it free of bank
// conflicts, and no counter is shared.  Returns the number flagged.
// cnt needs 2 * R * kNW + 1 ints, and R * kNW <= 64.
template <int R, class Emit>
__device__ int block_compact(const bool (&flag)[R], int* cnt, Emit emit) {
    static_assert(R * kNW <= 64, "one wave scans the counts");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long bal[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        bal[r] = __ballot(flag[r]);
        if (lane == 0) cnt[r * kNW + wave] = __popcll(bal[r]);
    }
    __syncthreads();
    if (wave == 0) {
        const int v = lane < R * kNW ? cnt[lane] : 0;
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, kWave);
            if (lane >= o) x += y;
        }
        if (lane < R * kNW) cnt[R * kNW + lane] = x - v;
        if (lane == 63) cnt[2 * R * kNW] = x;  // the total
    }
    __syncthreads();
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (flag[r]) emit(r, cnt[R * kNW + r * kNW + wave] + __popcll(bal[r] & lt));
    const int total = cnt[2 * R * kNW];
    __syncthreads();  // cnt may be reused
    return total;
}

template <int CAP>
struct SmallShared {
    uint32_t keys[CAP];
    union {                       // the histogram is dead once the bin is found
        int hist[kBins];
        unsigned long long fin[kMaxK];
    };
    int cand[kCandCap];
    int pool[CAP];                // the row's pool (block ids; P <= columns), when it has one
    int hist8[256];
    int ccnt[2 * (CAP / kNT) * kNW + 1];
    Scan scan;
    int misc[4];
};

template <int CAP>
__global__ __launch_bounds__(kNT) void topk_small_kernel(TopkP p) {
    __shared__ SmallShared<CAP> sh;
    const int row = blockIdx.x;
    const int n = p.ncols;
    const int K = p.K;
    const float* srow = p.scores + static_cast<size_t>(row) * n;
    const int32_t* prow = p.pool ? p.pool + static_cast<size_t>(row) * p.P : nullptr;
    int32_t* orow = p.idx + static_cast<size_t>(row) * K;
    // The row's pool goes to LDS first: every record id below is then an
    // LDS read (a global read would wait, at each use, for the stores and
    // loads issued before it).  Column c's block c / blk comes from one
    // multiply by ceil(2^32 / blk), exact while c * blk < 2^32 (here both
    // are at most 4096), not from an integer division per use.
    const bool pooled = prow != nullptr;
    if (pooled) {
        for (int i = threadIdx.x; i < p.P; i += kNT) sh.pool[i] = prow[i];
        __syncthreads();
    }
    const unsigned long long bmul = pooled ? ((1ull << 32) + p.blk - 1) / p.blk : 0ull;
    auto recl = [&](int c) -> int {
        if (!pooled) return c;
        const int q = static_cast<int>((static_cast<unsigned long long>(c) * bmul) >> 32);
        const int pb = sh.pool[q];
        return pb < 0 ? -1 : pb * p.blk + (c - q * p.blk);
    };

    int nvalid = 0;
    for (int c0 = 0; c0 < n; c0 += 4 * kNT) {  // four keys per thread per round, loads issued together
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = srow[min(c0 + i * kNT + static_cast<int>(threadIdx.x), n - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * kNT + static_cast<int>(threadIdx.x);
            uint32_t k = score_key(sv[i]);
            if (c >= n || (k != 0u && recl(c) < 0)) k = 0u;
            if (c < n) sh.keys[c] = k;
            nvalid += k != 0u;
        }
    }
    for (int i = threadIdx.x; i < kBins; i += kNT) sh.hist[i] = 0;
    int total;
    block_excl_scan(nvalid, sh.scan, &total);  // barriers inside
    nvalid = total;

    int bstar = -1;
    unsigned long long thr = 0;
    if (nvalid > K) {
        for (int c = threadIdx.x; c < n; c += kNT) {
            const uint32_t k = sh.keys[c];
            if (k) atomicAdd(&sh.hist[k >> kBinShift], 1);
        }
        __syncthreads();
        int need;
        bstar = find_from_top<kBins / kNT>(sh.hist, K, sh.scan, &need);
        constexpr int kR = CAP / kNT;
        bool inb[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int c = r * kNT + static_cast<int>(threadIdx.x);
            const uint32_t k = c < n ? sh.keys[c] : 0u;
            inb[r] = k && static_cast<int>(k >> kBinShift) == bstar;
        }
        const int ncand = block_compact(inb, sh.ccnt, [&](int r, int pos) {
            if (pos < kCandCap) sh.cand[pos] = r * kNT + static_cast<int>(threadIdx.x);
        });
        // every candidate shares the key's top 12 bits (bin bstar)
        const unsigned long long known = static_cast<unsigned long long>(static_cast<uint32_t>(bstar) << kBinShift) << 32;
        if (ncand <= kCandCap) {
            auto src = [&](int i, uint32_t& key, int& rec) -> bool {
                const int c = sh.cand[i];
                key = sh.keys[c];
                rec = recl(c);
                return true;
            };
            thr = radix_select(src, ncand, need, sh.hist8, sh.scan, 48, known);
        } else {
            auto src = [&](int c, uint32_t& key, int& rec) -> bool {
                key = sh.keys[c];
                if (!key || static_cast<int>(key >> kBinShift) != bstar) return false;
                rec = recl(c);
                return true;
            };
            thr = radix_select(src, n, need, sh.hist8, sh.scan, 48, known);
        }
    }
    auto chosen = [&](int c) -> bool {
        const uint32_t k = sh.keys[c];
        if (!k) return false;
        const int b = static_cast<int>(k >> kBinShift);
        if (b != bstar) return b > bstar;
        return composite(k, recl(c)) >= thr;
    };
    const int take = nvalid < K ? nvalid : K;

    if (!p.sort_by_key) {
        // ordered compaction of the chosen records into LDS (the
        // histogram's space, dead by now); one coalesced pass then writes
        // the row
        constexpr int kR = CAP / kNT;
        bool ch[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int c = r * kNT + static_cast<int>(threadIdx.x);
            ch[r] = c < n && chosen(c);
        }
        int* outr = sh.hist;
        block_compact(ch, sh.ccnt, [&](int r, int pos) {
            if (pos < K) outr[pos] = recl(r * kNT + static_cast<int>(threadIdx.x));
        });
        for (int i = threadIdx.x; i < K; i += kNT) orow[i] = i < take ? outr[i] : -1;
    } else {
        if (threadIdx.x == 0) sh.misc[1] = 0;
        __syncthreads();
        for (int c = threadIdx.x; c < n; c += kNT) {
            if (chosen(c)) {
                const int slot = atomicAdd(&sh.misc[1], 1);
                if (slot < K) sh.fin[slot] = composite(sh.keys[c], recl(c));
            }
        }
        __syncthreads();
        int m2 = 1;
        while (m2 < take) m2 <<= 1;
        for (int i = take + threadIdx.x; i < m2; i += kNT) sh.fin[i] = 0ull;
        __syncthreads();
        for (int k = 2; k <= m2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = threadIdx.x; i < m2; i += kNT) {
                    const int ij = i ^ j;
                    if (ij > i) {
                        const unsigned long long a = sh.fin[i], b = sh.fin[ij];
                        const bool desc = (i & k) == 0;
                        if (desc ? (a < b) : (a > b)) { sh.fin[i] = b; sh.fin[ij] = a; }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = threadIdx.x; i < K; i += kNT)
            orow[i] = i < take ? static_cast<int32_t>(~static_cast<uint32_t>(sh.fin[i])) : -1;
    }
}

// ---------------------------------------------------------------- rows up to 16384 columns, one workgroup each

// One workgroup of NT threads per row (1024 threads of 16 keys for rows up
// to 16384 columns; 512 of 8 for rows up to 4096, whose eight waves meet
// faster at the kernel's many barriers: 7% faster than 1024 threads of 4
// keys, while 256 of 16 were 18% slower), the row's keys in registers:
// thread t owns the KPT consecutive columns KPT*t .. KPT*t+KPT-1.  One LDS
// histogram of the top 12 key bits finds the boundary bin; an exact radix
// select over the composite keys of that bin runs straight over the
// registers (8-bit digits below the bin's 12 known bits, each pass one LDS
// histogram and one scan, stopping once a digit class holds exactly the
// elements still needed); the chosen columns leave in column order through
// one block scan of per-thread counts.  No candidate list, no workspace and
// one launch: for the few long rows of decode this replaces a chain of
// kernels that hand lists from workgroup to workgroup.
constexpr int kRT = 1024;
constexpr int kRowCols = kRT * 16;  // columns per row at most (16 keys per thread fit the registers)
constexpr int kRTShort = 512;       // threads per row for rows up to kRTShort * 8 columns
// two-pass long rows: sub-rows of kSubKPT x kSubNT columns (8192 on 512
// threads measured faster than 16384 on 1024: C4 20.0 against 24.1 us per
// call, C5 and C7 within 2%)
constexpr int kSubKPT = 16, kSubNT = 512, kSubCols = kSubKPT * kSubNT;

template <int NT>
struct RowScan {
    static constexpr int kRW = NT / kWave;
    int wave_tot[kRW];
    int res[3];
    uint32_t lo[kRW], hi[kRW];
};

template <int NT>
__device__ int row_excl_scan(int v, RowScan<NT>& s, int* total) {
    constexpr int kRW = NT / kWave;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s.wave_tot[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kRW; ++i) {
        const int w = s.wave_tot[i];
        off += i < wave ? w : 0;
        tot += w;
    }
    *total = tot;
    return off + x - v;
}

// Scanning nb = NT * PER (PER > 0) or 256 (PER = 0: threads below 256 hold
// one bin each) bins from the top, the bin where the running count first
// reaches `need`: returns it (-1 if the total is below need) and the number
// still needed from it, and that bin's count.
template <int PER, int NT>
__device__ int row_find(const int* hist, int need, RowScan<NT>& s, int* rest, int* bin_count) {
    constexpr int P = PER ? PER : 1;
    constexpr int NB = PER ? NT * PER : 256;
    int loc[P];
    int sum = 0;
    const int t = threadIdx.x;
    const int top = NB - 1 - t * P;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        loc[j] = (PER || t < NB) ? hist[top - j] : 0;
        sum += loc[j];
    }
    int total;
    const int excl = row_excl_scan(sum, s, &total);
    if (t == 0) { s.res[0] = -1; s.res[1] = 0; s.res[2] = 0; }
    __syncthreads();
    if (excl < need && excl + sum >= need) {
        int acc = excl;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (acc + loc[j] >= need) {
                s.res[0] = top - j;
                s.res[1] = need - acc;
                s.res[2] = loc[j];
                break;
            }
            acc += loc[j];
        }
    }
    __syncthreads();
    const int bin = s.res[0];
    *rest = s.res[1];
    *bin_count = s.res[2];
    __syncthreads();
    return bin;
}

template <int NT>
struct __align__(16) RowShared {
    int hist[kBins];
    int hist8[256];
    int pool[NT * 4];  // the row's pool (NT * 16 columns, blocks of at least 4 records)
    RowScan<NT> scan;
};

// Modes of the row kernel:
//  kRowIds  -- a row of scores -> its K best record ids;
//  kRowSub  -- sub-row (blockIdx.x mod nchunks) of KPT x NT columns of a row
//              -> its K best (key, record) pairs into cand_k / cand_i;
//  kRowCand -- a row of such pairs (p.ncols = nchunks x K) -> the K best
//              record ids.
constexpr int kRowIds = 0, kRowSub = 1, kRowCand = 2;

template <int KPT, bool POOL, int NT, int MODE = kRowIds>
__global__ __launch_bounds__(NT) void topk_row_kernel(TopkP p) {
    constexpr int kRW = NT / kWave;
    constexpr int kSub = KPT * NT;  // kRowSub: columns per sub-row
    static_assert(!(MODE == kRowSub && POOL) || KPT <= 16, "the pool slice (blocks of >= 4) fits sh.pool");
    static_assert(MODE != kRowCand || !POOL, "candidates carry their record ids");
    __shared__ RowShared<NT> sh;
    __shared__ int32_t cid[MODE == kRowCand ? KPT * NT : 1];  // the candidates' record ids
    const int row = MODE == kRowSub ? static_cast<int>(blockIdx.x) / p.nchunks : static_cast<int>(blockIdx.x);
    const int sub = MODE == kRowSub ? static_cast<int>(blockIdx.x) % p.nchunks : 0;
    const int cbase = sub * kSub;  // the sub-row's first column
    const int n = MODE == kRowSub ? min(kSub, p.ncols - cbase) : p.ncols;
    const int K = p.K;
    const int t = threadIdx.x;
    const float* srow = p.scores + static_cast<size_t>(row) * p.ncols + cbase;
    const uint32_t* krow = MODE == kRowCand ? p.cand_k + static_cast<size_t>(row) * n : nullptr;
    const int32_t* irow = MODE == kRowCand ? p.cand_i + static_cast<size_t>(row) * n : nullptr;
    int32_t* orow = p.idx + static_cast<size_t>(row) * K;
    if constexpr (POOL) {
        // the blocks of the sub-row's columns (a sub-row starts at a block:
        // its width is a multiple of blk on this path)
        const int q0 = cbase / p.blk;
        const int32_t* prow = p.pool + static_cast<size_t>(row) * p.P + q0;
        const int np = min(p.P - q0, (n + p.blk - 1) / p.blk);
        for (int i = t; i < np; i += NT) sh.pool[i] = prow[i];
    }
    for (int i = t; i < kBins; i += NT) sh.hist[i] = 0;
    const int lane = t & 63, wave = t >> 6;
    // the thread's scores, all loads in flight at once
    const int c0 = KPT * t;
    uint32_t kk[KPT];  // scores' bits (candidate keys), then keys
    const uint32_t* src = MODE == kRowCand ? krow : reinterpret_cast<const uint32_t*>(srow);
    if ((p.ncols & 3) == 0 && c0 + KPT <= n) {  // whole and 16-byte aligned (the row base is)
#pragma unroll
        for (int i = 0; i < KPT; i += 4) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + c0 + i);
            kk[i] = v[0]; kk[i + 1] = v[1]; kk[i + 2] = v[2]; kk[i + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) kk[i] = src[min(c0 + i, n - 1)];
    }
    if constexpr (MODE == kRowCand)
        for (int c = t; c < n; c += NT) cid[c] = irow[c];
    __syncthreads();  // pool, candidate ids and cleared histogram visible
    auto rec_of_col = [&](int c) -> int {
        if constexpr (MODE == kRowCand) return cid[c];
        if constexpr (!POOL) return cbase + c;
        const int q = c / p.blk;
        const int pb = sh.pool[q];
        return pb < 0 ? -1 : (pb * p.blk + (c - q * p.blk));
    };
    int nv = 0;
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int c = c0 + i;
        uint32_t k = MODE == kRowCand ? kk[i] : score_key(__uint_as_float(kk[i]));
        if (c >= n || (POOL && k != 0u && rec_of_col(c) < 0)) k = 0u;
        kk[i] = k;
        nv += k != 0u;
        if (k) klo = min(klo, k);
        khi = max(khi, k);
    }
    // The row's valid keys share every bit above the highest bit in which
    // its smallest and largest differ; the histogram takes the 12 bits
    // below that common prefix, so the keys spread over the bins (the top
    // 12 bits would put most of a row into a few bins, whose LDS atomics
    // serialise).
    for (int o = 32; o > 0; o >>= 1) {
        klo = min(klo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(klo), o, kWave)));
        khi = max(khi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(khi), o, kWave)));
    }
    if (lane == 0) {
        sh.scan.lo[wave] = klo;
        sh.scan.hi[wave] = khi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRW; ++w) {
        klo = min(klo, sh.scan.lo[w]);
        khi = max(khi, sh.scan.hi[w]);
    }
    const uint32_t diff = klo ^ khi;
    const int top = (diff && klo <= khi) ? 31 - __builtin_clz(diff) : -1;
    const int bsh = top > 11 ? top - 11 : 0;                                 // bin = (key >> bsh) & 4095
    // the shared high bits (all of them when every valid key is equal)
    const uint32_t common = top < 0 ? khi : (top >= 31 ? 0u : (khi & ~((2u << top) - 1u)));
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (kk[i]) atomicAdd(&sh.hist[(kk[i] >> bsh) & (kBins - 1)], 1);
    int nvalid;
    row_excl_scan(nv, sh.scan, &nvalid);  // barriers inside: the histogram is complete

    int b1 = -1;
    unsigned long long thr = 0ull;
    if (nvalid > K) {
        int need, bc;
        b1 = row_find<kBins / NT>(sh.hist, K, sh.scan, &need, &bc);
        // radix select of the `need` largest composite keys of bin b1, over
        // the registers; the common prefix and the bin fix the composite's
        // bits from 32 + bsh up
        const uint32_t kb = common | (static_cast<uint32_t>(b1) << bsh);  // the bin's key bits
        unsigned long long prefix = static_cast<unsigned long long>(kb) << 32;
        unsigned long long mask = ~0ull << (32 + bsh);
        auto in_bin = [&](uint32_t k) { return k && (k >> bsh) == (kb >> bsh); };
        for (int shift = 32 + bsh - 8;; shift -= 8) {
            const int sh8 = shift > 0 ? shift : 0;
            if (t < 256) sh.hist8[t] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                if (in_bin(kk[i])) {
                    const unsigned long long ck = composite(kk[i], rec_of_col(c0 + i));
                    if ((ck & mask) == prefix) atomicAdd(&sh.hist8[(ck >> sh8) & 255], 1);
                }
            }
            __syncthreads();
            int rest, cnt_d;
            const int d = row_find<0>(sh.hist8, need, sh.scan, &rest, &cnt_d);
            prefix |= static_cast<unsigned long long>(d) << sh8;
            mask |= 255ull << sh8;
            need = rest;
            if (cnt_d == rest || sh8 == 0) break;  // the whole class is chosen, or the key is exact
        }
        thr = prefix;
    }
    // chosen columns, in column order: the composite key reaches the
    // threshold, i.e. the key is above the threshold's key part, or equal
    // to it with ~record reaching the low part (with at most K valid keys
    // the threshold is 1 << 32: every valid key).  Decided once per key, as
    // a bit mask, with 32-bit compares.
    const uint32_t thr_k = b1 >= 0 ? static_cast<uint32_t>(thr >> 32) : 1u;
    const uint32_t thr_lo = b1 >= 0 ? static_cast<uint32_t>(thr) : 0u;
    uint32_t chosen = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const uint32_t k = kk[i];
        bool ch = k > thr_k;
        if (k == thr_k) ch = ~static_cast<uint32_t>(rec_of_col(c0 + i)) >= thr_lo;
        chosen |= static_cast<uint32_t>(ch) << i;
    }
    int take;
    int pos = row_excl_scan(__popc(chosen), sh.scan, &take);
    if constexpr (MODE == kRowSub) {
        const size_t slot = (static_cast<size_t>(row) * p.nchunks + sub) * K;
        uint32_t* ck = p.cand_k + slot;
        int32_t* ci = p.cand_i + slot;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (((chosen >> i) & 1u) && pos < K) {
                ck[pos] = kk[i];
                ci[pos++] = rec_of_col(c0 + i);
            }
        for (int i = take + t; i < K; i += NT) {
            ck[i] = 0u;  // never selectable
            ci[i] = -1;
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (((chosen >> i) & 1u) && pos < K) orow[pos++] = rec_of_col(c0 + i);
        for (int i = take + t; i < K; i += NT) orow[i] = -1;
    }
}

// ---------------------------------------------------------------- long rows

// The row lists that the workgroups of a row hand to its last workgroup
// are written and read as device-scope relaxed atomics: those bypass the
// per-XCD L2s, so the hand-off needs only this wave's stores to be
// complete before the ticket -- not a device-wide fence, which on this
// chip writes back and invalidates the whole L2.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }  // vmcnt(0)

__global__ __launch_bounds__(kNT) void topk_zero_kernel(TopkP p) {
    const int row = blockIdx.x;
    int* h = p.ghist + static_cast<size_t>(row) * kBins;
    for (int i = threadIdx.x; i < kBins; i += kNT) h[i] = 0;
    if (threadIdx.x < 4) p.cnt[row * 4 + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kNT) void topk_hist_kernel(TopkP p) {
    __shared__ int hist[kBins];
    const int row = blockIdx.y;
    const int c0 = blockIdx.x * kChunk;
    const int c1 = min(p.ncols, c0 + kChunk);
    const float* srow = p.scores + static_cast<size_t>(row) * p.ncols;
    const int32_t* prow = p.pool ? p.pool + static_cast<size_t>(row) * p.P : nullptr;
    // the chunk's keys first, all loads in flight at once
    uint32_t kk[kChunk / kNT];
    load_keys(p, prow, srow, c0, c1, kk);
    for (int i = threadIdx.x; i < kBins; i += kNT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kChunk / kNT; ++i)
        if (kk[i]) atomicAdd(&hist[kk[i] >> kBinShift], 1);
    __syncthreads();
    if (p.nchunks <= kFewChunks) {
        // the chunk's own histogram (the select kernel sums the row's few);
        // the row's counters are cleared here, before the select kernel runs
        int* g = p.ghist + (static_cast<size_t>(row) * p.nchunks + blockIdx.x) * kBins;
        for (int i = threadIdx.x; i < kBins; i += kNT) g[i] = hist[i];
        if (blockIdx.x == 0 && threadIdx.x < 4) p.cnt[row * 4 + threadIdx.x] = 0;
        return;
    }
    int* g = p.ghist + static_cast<size_t>(row) * kBins;
    for (int i = threadIdx.x; i < kBins; i += kNT)
        if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// The last workgroup of a row holds the row's entries (keys in bin b1 or
// above, at most kEntCap) in LDS; more go through the slower path that
// reads them from the lists.
constexpr int kEntCap = 4096;
static_assert(kEntCap / kNT == kChunk / kNT, "entry rows and load rows share the per-wave count table");
constexpr int kMaxChunks = 16 * kNT;  // rows up to 16M columns
struct __align__(16) LongShared {
    union {
        int hist[kBins];          // the row histogram, until the boundary bin is known
        uint32_t key[kEntCap];    // last workgroup: the row's entries in column order
    } a;
    int col[kEntCap];             // their columns (with sort_by_key, reused for the chosen composites)
    int rec[kEntCap];             // their records
    int hist8[256];
    int cbase[kMaxChunks + 1];    // first entry of each chunk
    int cnt_wi[kChunk / kNT][kNW];  // entries per (load row, wave)
    Scan scan;
    int misc[4];
};

__global__ __launch_bounds__(kNT) void topk_select_kernel(TopkP p) {
    __shared__ LongShared sh;
    constexpr int kPer = kChunk / kNT;
    const int row = blockIdx.y;
    const int chunk = blockIdx.x;
    const int K = p.K;
    const int nch = p.nchunks;
    const int c0 = chunk * kChunk;
    const int c1 = min(p.ncols, c0 + kChunk);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* srow = p.scores + static_cast<size_t>(row) * p.ncols;
    const int32_t* prow = p.pool ? p.pool + static_cast<size_t>(row) * p.P : nullptr;
    int* cnt = p.cnt + row * 4;
    int* ccnt = p.ccnt + static_cast<size_t>(row) * nch;
    uint32_t* gkey = p.ckey + static_cast<size_t>(row) * p.ncols;
    int* gcol = p.ccol + static_cast<size_t>(row) * p.ncols;

    // the chunk's keys and the row histogram, all loads in flight at once
    uint32_t kk[kPer];
    load_keys(p, prow, srow, c0, c1, kk);
    if (nch <= kFewChunks) {
        // the row histogram is the sum of its chunks' (all loads in flight at once)
        const int* g = p.ghist + static_cast<size_t>(row) * nch * kBins;
        int hv[kFewChunks][kBins / kNT];
#pragma unroll
        for (int c = 0; c < kFewChunks; ++c)
#pragma unroll
            for (int j = 0; j < kBins / kNT; ++j)
                hv[c][j] = g[static_cast<size_t>(min(c, nch - 1)) * kBins + j * kNT + threadIdx.x];
#pragma unroll
        for (int j = 0; j < kBins / kNT; ++j) {
            int t = 0;
#pragma unroll
            for (int c = 0; c < kFewChunks; ++c) t += c < nch ? hv[c][j] : 0;
            sh.a.hist[j * kNT + threadIdx.x] = t;
        }
    } else {
        const int* g = p.ghist + static_cast<size_t>(row) * kBins;
        int hv[kBins / kNT];
#pragma unroll
        for (int j = 0; j < kBins / kNT; ++j) hv[j] = g[j * kNT + threadIdx.x];
#pragma unroll
        for (int j = 0; j < kBins / kNT; ++j) sh.a.hist[j * kNT + threadIdx.x] = hv[j];
    }
    __syncthreads();
    int need1;
    const int b1 = find_from_top<kBins / kNT>(sh.a.hist, K, sh.scan, &need1);
    // The chunk's entries -- keys in bin b1 or above (every valid key when
    // the row holds fewer than K) -- go to the chunk's own columns' slots of
    // the row's lists, in column order: column c0 + i kNT + t comes after
    // those of the earlier load rows i, of the earlier waves in row i, and
    // of the earlier lanes of its own wave (one ballot per load row).
    auto entry = [&](uint32_t k) { return k != 0u && static_cast<int>(k >> kBinShift) >= b1; };
    unsigned long long bal[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) bal[i] = __ballot(entry(kk[i]));
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) sh.cnt_wi[i][wave] = __popcll(bal[i]);
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    int run = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            const int n = sh.cnt_wi[i][w];
            before += w < wave ? n : 0;
            tot += n;
        }
        if ((bal[i] >> lane) & 1ull) {
            const int at = c0 + run + before + __popcll(bal[i] & below);
            st_dev(gkey + at, kk[i]);
            st_dev(gcol + at, c0 + i * kNT + static_cast<int>(threadIdx.x));
        }
        run += tot;
    }
    if (threadIdx.x == 0) st_dev(ccnt + chunk, run);
    wait_stores();  // this wave's list entries are visible device-wide
    __syncthreads();
    if (threadIdx.x == 0) sh.misc[2] = atomicAdd(&cnt[2], 1) == nch - 1;
    __syncthreads();
    if (!sh.misc[2]) return;

    // ---- last workgroup of this row ----
    // chunk c's entries sit at [c kChunk, c kChunk + n_c) of the lists;
    // thread t sums the counts of its (contiguous) chunks, one scan places them
    // (the counts are loaded once, all at once, and kept for the placing)
    const int cpt = (nch + kNT - 1) / kNT;
    constexpr int kCpt = kMaxChunks / kNT;
    int cv[kCpt];
    int csum = 0;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        const int c = static_cast<int>(threadIdx.x) * cpt + j;
        cv[j] = j < cpt && c < nch ? ld_dev(ccnt + c) : 0;
    }
#pragma unroll
    for (int j = 0; j < kCpt; ++j) csum += cv[j];
    int total;
    int cb = block_excl_scan(csum, sh.scan, &total);
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        const int c = static_cast<int>(threadIdx.x) * cpt + j;
        if (j < cpt && c < nch) {
            sh.cbase[c] = cb;
            cb += cv[j];
        }
    }
    if (threadIdx.x == 0) sh.cbase[nch] = total;
    __syncthreads();
    // list slot of entry e: its chunk is the last one starting at or below e
    // (a binary search: the crowded path's; the LDS path uses a table)
    auto slot_of = [&](int e) {
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.cbase[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        return lo * kChunk + (e - sh.cbase[lo]);
    };
    // every candidate shares the key's top 12 bits (bin b1)
    const unsigned long long known = static_cast<unsigned long long>(static_cast<uint32_t>(b1 < 0 ? 0 : b1) << kBinShift) << 32;
    int32_t* orow = p.idx + static_cast<size_t>(row) * K;
    int take = 0;
    if (total == 0) {
        // nothing selectable in the row
    } else if (total <= kEntCap) {
        // Entry e = j kNT + t is thread t's j-th (LDS accesses by consecutive
        // threads hit consecutive words).  Its chunk comes from a table that
        // each wave fills for its chunks, 64 entries at a time; then every
        // entry's list loads go out at once.
        constexpr int kEP = kEntCap / kNT;
        int* owner = sh.col;  // the column array is filled only after the loads
        for (int c = wave; c < nch; c += kNW) {
            const int b0 = sh.cbase[c], n = sh.cbase[c + 1] - b0;
            for (int i = lane; i < n; i += kWave) owner[b0 + i] = c;
        }
        __syncthreads();
        uint32_t ek[kEP];
        int ec[kEP];
#pragma unroll
        for (int j = 0; j < kEP; ++j) {
            const int e = min(j * kNT + static_cast<int>(threadIdx.x), total - 1);
            const int c = owner[e];
            const int s = c * kChunk + (e - sh.cbase[c]);
            ek[j] = ld_dev(gkey + s);
            ec[j] = ld_dev(gcol + s);
        }
        int er[kEP];
#pragma unroll
        for (int j = 0; j < kEP; ++j) er[j] = rec_of(p, prow, ec[j]);
        __syncthreads();  // the histogram (overlaid by the key array) and the table are no longer read
#pragma unroll
        for (int j = 0; j < kEP; ++j) {
            const int e = j * kNT + static_cast<int>(threadIdx.x);
            if (e < total) {
                sh.a.key[e] = ek[j];
                sh.col[e] = ec[j];
                sh.rec[e] = er[j];
            }
        }
        __syncthreads();
        // the threshold among the boundary bin's entries (every entry is
        // chosen when the row holds fewer than K)
        unsigned long long thr = 0ull;
        if (b1 >= 0) {
            auto src = [&](int i, uint32_t& key, int& rec) -> bool {
                key = sh.a.key[i];
                rec = sh.rec[i];
                return static_cast<int>(key >> kBinShift) == b1;
            };
            thr = radix_select(src, total, need1, sh.hist8, sh.scan, 48, known);
        }
        // chosen entries in column order (= entry order): entry j kNT + t
        // goes after the chosen ones of the earlier rows j, of the earlier
        // waves in row j and of the earlier lanes of its wave (ballots)
        bool cf[kEP];
        unsigned long long cbal[kEP];
#pragma unroll
        for (int j = 0; j < kEP; ++j) {
            const int e = j * kNT + static_cast<int>(threadIdx.x);
            const int ei = min(e, total - 1);
            const uint32_t k = sh.a.key[ei];
            const int r = sh.rec[ei];
            cf[j] = e < total && (static_cast<int>(k >> kBinShift) > b1 || composite(k, r) >= thr);
            cbal[j] = __ballot(cf[j]);
        }
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < kEP; ++j) sh.cnt_wi[j][wave] = __popcll(cbal[j]);
        }
        __syncthreads();
        const unsigned long long below = (1ull << lane) - 1ull;
        int run2 = 0;
        int at[kEP];
#pragma unroll
        for (int j = 0; j < kEP; ++j) {
            int before = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < kNW; ++w) {
                const int n = sh.cnt_wi[j][w];
                before += w < wave ? n : 0;
                tot += n;
            }
            at[j] = run2 + before + __popcll(cbal[j] & below);
            run2 += tot;
        }
        take = min(run2, K);
        if (!p.sort_by_key) {
#pragma unroll
            for (int j = 0; j < kEP; ++j)
                if (cf[j] && at[j] < K) orow[at[j]] = sh.rec[j * kNT + static_cast<int>(threadIdx.x)];
        } else {
            // score order: the chosen composites, then a bitonic sort
            unsigned long long cv[kEP];
#pragma unroll
            for (int j = 0; j < kEP; ++j) {
                const int e = min(j * kNT + static_cast<int>(threadIdx.x), total - 1);
                cv[j] = composite(sh.a.key[e], sh.rec[e]);
            }
            __syncthreads();  // the column array becomes the composite array
            unsigned long long* fo = reinterpret_cast<unsigned long long*>(sh.col);
#pragma unroll
            for (int j = 0; j < kEP; ++j)
                if (cf[j] && at[j] < K) fo[at[j]] = cv[j];
        }
    } else {
        // a crowded boundary: select and filter straight from the lists
        unsigned long long thr2 = 0ull;
        if (b1 >= 0) {
            auto src = [&](int i, uint32_t& key, int& rec) -> bool {
                const int s = slot_of(i);
                key = ld_dev(gkey + s);
                if (static_cast<int>(key >> kBinShift) != b1) return false;
                rec = rec_of(p, prow, ld_dev(gcol + s));
                return true;
            };
            thr2 = radix_select(src, total, need1, sh.hist8, sh.scan, 48, known);
        }
        unsigned long long* fin = reinterpret_cast<unsigned long long*>(sh.col);
        for (int base = 0; base < total; base += kNT) {
            const int e = base + static_cast<int>(threadIdx.x);
            bool f = false;
            int r = 0;
            uint32_t k = 0u;
            if (e < total) {
                const int s = slot_of(e);
                k = ld_dev(gkey + s);
                r = rec_of(p, prow, ld_dev(gcol + s));
                f = static_cast<int>(k >> kBinShift) > b1 || composite(k, r) >= thr2;
            }
            int nt;
            const int at = take + block_excl_scan(f ? 1 : 0, sh.scan, &nt);
            if (f && at < K) {
                if (p.sort_by_key) fin[at] = composite(k, r);
                else orow[at] = r;
            }
            take += nt;
        }
        take = min(take, K);
    }
    for (int i = take + threadIdx.x; i < K; i += kNT) orow[i] = -1;
    if (!p.sort_by_key) return;
    // score order: bitonic sort of the chosen composites (log^2 stages, one
    // block pass each), descending
    __syncthreads();
    unsigned long long* fin = reinterpret_cast<unsigned long long*>(sh.col);
    int m2 = 1;
    while (m2 < take) m2 <<= 1;
    for (int i = take + threadIdx.x; i < m2; i += kNT) fin[i] = 0ull;  // padding sorts last
    __syncthreads();
    for (int k = 2; k <= m2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < m2; i += kNT) {
                const int ij = i ^ j;
                if (ij > i) {
                    const unsigned long long a = fin[i], b = fin[ij];
                    const bool first = (i & k) == 0;
                    if (first ? a < b : a > b) { fin[i] = b; fin[ij] = a; }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < take; i += kNT) orow[i] = static_cast<int32_t>(~static_cast<uint32_t>(fin[i]));
}

// One wave per block: beta[row][j] = max over columns [j*blk, min((j+1)*blk, N)).
__global__ __launch_bounds__(256) void block_max_kernel(const float* scores, int N, int blk, int nb,
                                                        float* beta) {
    const int row = blockIdx.y;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= nb) return;
    const float* s = scores + static_cast<size_t>(row) * N + static_cast<size_t>(j) * blk;
    const int len = min(blk, N - j * blk);
    float m = -__builtin_huge_valf();
    for (int i = lane; i < len; i += 64) {
        const float v = s[i];
        if (v > m) m = v;  // NaN never raises the maximum
    }
    m = warp_max(m);
    if (lane == 0) beta[static_cast<size_t>(row) * nb + j] = m;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct LongLayout {
    size_t hist, cnt, ccnt, ckey, ccol, total;
};

LongLayout long_layout(int rows, int ncols, int K) {
    LongLayout L;
    size_t off = 0;
    const size_t nchk = (static_cast<size_t>(ncols) + kChunk - 1) / kChunk;
    L.hist = off;
    off += align256(static_cast<size_t>(rows) * (nchk <= kFewChunks ? nchk : 1) * kBins * sizeof(int));
    L.cnt = off;
    off += align256(static_cast<size_t>(rows) * 4 * sizeof(int));
    L.ccnt = off;
    off += align256(static_cast<size_t>(rows) * nchk * sizeof(int));
    L.ckey = off;
    off += align256(static_cast<size_t>(rows) * ncols * sizeof(uint32_t));
    L.ccol = off;
    off += align256(static_cast<size_t>(rows) * ncols * sizeof(int));
    L.total = off;
    return L;
}

int run_topk(TopkP p, void* ws, hipStream_t st) {
    // one wave per row pays off when rows are many or short: a few long rows
    // are faster with a whole workgroup each (the LDS path below)
    if (p.ncols <= 64 * 64 && (!p.sort_by_key || p.K <= 64) && (p.ncols <= 64 * 16 || p.rows >= 1024)) {
        const dim3 grid((p.rows + kNW - 1) / kNW);
        if (p.pool) {
            if (p.ncols <= 64 * 16) hipLaunchKernelGGL((topk_wave_kernel<16, true>), grid, dim3(kNT), 0, st, p);
            else if (p.ncols <= 64 * 32) hipLaunchKernelGGL((topk_wave_kernel<32, true>), grid, dim3(kNT), 0, st, p);
            else hipLaunchKernelGGL((topk_wave_kernel<64, true>), grid, dim3(kNT), 0, st, p);
        } else {
            if (p.ncols <= 64 * 16) hipLaunchKernelGGL((topk_wave_kernel<16, false>), grid, dim3(kNT), 0, st, p);
            else if (p.ncols <= 64 * 32) hipLaunchKernelGGL((topk_wave_kernel<32, false>), grid, dim3(kNT), 0, st, p);
            else hipLaunchKernelGGL((topk_wave_kernel<64, false>), grid, dim3(kNT), 0, st, p);
        }
        return static_cast<int>(hipGetLastError());
    }
    if (!p.sort_by_key && p.ncols <= kRowCols && (!p.pool || p.blk >= 4)) {
        // rows up to 16384 columns (record ids or pooled): one workgroup each
#define CSA2_ROW(KPT, NT)                                                                                \
    if (p.pool) hipLaunchKernelGGL((topk_row_kernel<KPT, true, NT>), dim3(p.rows), dim3(NT), 0, st, p);  \
    else hipLaunchKernelGGL((topk_row_kernel<KPT, false, NT>), dim3(p.rows), dim3(NT), 0, st, p);
        if (p.ncols <= 8 * kRTShort) {
            CSA2_ROW(8, kRTShort)
        } else {
            CSA2_ROW(16, kRT)
        }
#undef CSA2_ROW
        return static_cast<int>(hipGetLastError());
    }
    if (p.ncols <= kSmallCols) {
        hipLaunchKernelGGL(topk_small_kernel<kSmallCols>, dim3(p.rows), dim3(kNT), 0, st, p);
        return static_cast<int>(hipGetLastError());
    }
    const LongLayout L = long_layout(p.rows, p.ncols, p.K);
    uint8_t* base = static_cast<uint8_t*>(ws);
    const int nsub = (p.ncols + kSubCols - 1) / kSubCols;
    if (!p.sort_by_key && static_cast<long>(nsub) * p.K <= kRowCols &&
        (!p.pool || (p.blk >= 4 && kSubCols % p.blk == 0))) {
        // two passes of the row kernel: each sub-row's K best, then the
        // row's K best of those (the pairs fit the long-row workspace,
        // whose entry lists hold 8 bytes per column)
        const size_t nc = static_cast<size_t>(p.rows) * nsub * p.K;
        p.cand_k = reinterpret_cast<uint32_t*>(base);
        p.cand_i = reinterpret_cast<int32_t*>(base + align256(nc * sizeof(uint32_t)));
        p.nchunks = nsub;
        if (p.pool)
            hipLaunchKernelGGL((topk_row_kernel<kSubKPT, true, kSubNT, kRowSub>), dim3(p.rows * nsub), dim3(kSubNT), 0, st, p);
        else
            hipLaunchKernelGGL((topk_row_kernel<kSubKPT, false, kSubNT, kRowSub>), dim3(p.rows * nsub), dim3(kSubNT), 0, st, p);
        const int e = static_cast<int>(hipGetLastError());
        if (e) return e;
        TopkP q = p;
        q.ncols = nsub * p.K;
        q.pool = nullptr;
        q.P = 0;
        q.blk = 0;
        if (q.ncols <= 8 * kRTShort)
            hipLaunchKernelGGL((topk_row_kernel<8, false, kRTShort, kRowCand>), dim3(q.rows), dim3(kRTShort), 0, st, q);
        else
            hipLaunchKernelGGL((topk_row_kernel<16, false, kRT, kRowCand>), dim3(q.rows), dim3(kRT), 0, st, q);
        return static_cast<int>(hipGetLastError());
    }
    p.ghist = reinterpret_cast<int*>(base + L.hist);
    p.cnt = reinterpret_cast<int*>(base + L.cnt);
    p.ccnt = reinterpret_cast<int*>(base + L.ccnt);
    p.ckey = reinterpret_cast<uint32_t*>(base + L.ckey);
    p.ccol = reinterpret_cast<int*>(base + L.ccol);
    p.nchunks = (p.ncols + kChunk - 1) / kChunk;
    if (p.nchunks > kMaxChunks) return static_cast<int>(hipErrorInvalidValue);
    if (p.nchunks > kFewChunks) hipLaunchKernelGGL(topk_zero_kernel, dim3(p.rows), dim3(kNT), 0, st, p);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(p.nchunks, p.rows), dim3(kNT), 0, st, p);
    hipLaunchKernelGGL(topk_select_kernel, dim3(p.nchunks, p.rows), dim3(kNT), 0, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t topk_ws_bytes(int rows, int ncols, int K) {
    if (ncols <= kSmallCols) return 0;
    return long_layout(rows, ncols, K).total;
}

int launch_topk(const TopkArgs& a, void* stream) {
    TopkP p = {};
    p.rows = a.rows; p.ncols = a.ncols; p.K = a.K; p.P = a.P; p.blk = a.blk;
    p.scores = a.scores; p.pool = a.pool; p.idx = a.idx; p.sort_by_key = a.sort_by_key ? 1 : 0;
    return run_topk(p, a.ws, static_cast<hipStream_t>(stream));
}

size_t block_pool_ws_bytes(int rows, int N, int blk) {
    const size_t nb = (static_cast<size_t>(N) + blk - 1) / blk;
    return align256(static_cast<size_t>(rows) * nb * sizeof(float)) + topk_ws_bytes(rows, static_cast<int>(nb),
                                                                                     kMaxK);
}

int launch_block_pool(int rows, int N, int blk, int P, const float* scores, int32_t* pool, void* ws,
                      size_t, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int nb = (N + blk - 1) / blk;
    float* beta = static_cast<float*>(ws);
    hipLaunchKernelGGL(block_max_kernel, dim3((nb + 3) / 4, rows), dim3(256), 0, st, scores, N, blk, nb, beta);
    int e = static_cast<int>(hipGetLastError());
    if (e) return e;
    TopkP p = {};
    p.rows = rows; p.ncols = nb; p.K = P; p.P = 0; p.blk = 0;
    p.scores = beta; p.pool = nullptr; p.idx = pool; p.sort_by_key = 1;
    void* tws = static_cast<uint8_t*>(ws) + align256(static_cast<size_t>(rows) * nb * sizeof(float));
    return run_topk(p, tws, st);
}

}  // namespace csa2
