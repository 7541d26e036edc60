// Sparse shared-latent attention with a sliding window and a sink: the
// MFMA kernel template.  attn.hip instantiates its 64-head layout, attn_dec.hip
// its 16-head decode layout.
//
// For a query token at position t and head h, the entries are the selected
// global records (shared latent rows, used as both key and value) followed
// by the local window rows of positions max(0, t-W+1) .. t ("DeepSeek V4
// Inside: One Token Through Every Block", Fig. 11: the compressed entry is
// both K and V, and the window is joined to it in one softmax):
//
//   z_j   = sm * q_h . x_j
//   ctx_h = sum_j e^{z_j} x_j / (sum_j e^{z_j} + e^{sink_h})     (eq. (27))
//
// and the last r channels of ctx_h are rotated by position -t ("DeepSeek
// V4.1-Flash. Every layer, connected.", caption "The query and output
// paths").
//
// attn_mfma_kernel (64 heads x 512 dims, bf16 queries, bf16 or e4m3 rows):
//  * persistent: one workgroup of 4 waves per compute unit walks the work
//    items.  With many queries (prefill) an item is a query: wave w owns
//    heads 16w .. 16w+15 over all 512 channels, so O stays in its 128
//    accumulation registers and no partial sums cross waves.  With few
//    queries (decode) an item is one group of 16 heads of a query (or of a
//    split of its entries): every wave forms the same logits for those
//    heads and owns 128 channels of their output, and the four head groups
//    of a query run on one XCD, so the rows they all gather come from HBM
//    once and from that XCD's L2 for the other three;
//  * the valid selected records are compacted into an LDS list, so -1
//    padding costs nothing, and a table of row addresses is built per item;
//  * entries are processed in tiles of 32 rows, copied global -> LDS
//    row-major (bf16 directly with global_load_lds; e4m3 converted exactly
//    to bf16 in registers on the way) two tiles ahead of their use;
//  * S^T = X Q^T with 16x16x32 bf16 MFMAs (entries on M, heads on N), so
//    each lane holds 8 logits of ONE head, which are exactly the B operand
//    of the P.V MFMA; O^T += X^T P^T reads X^T with the transposing LDS
//    load.  P is split into bf16 hi + lo parts (two MFMAs) so that rounding
//    P to bf16 costs no accuracy;
//  * the P.V of tile t, the S^T of tile t+1 and its softmax form one
//    branch-free MFMA stream per iteration; each head keeps a lazy
//    reference maximum that moves (with a rescale of O and l) only when a
//    tile exceeds it by a wide margin, checked once per tile;
//  * e4m3 per-row scales multiply the logit and the probability;
//  * with one split the workgroup finishes (sink, normalisation, inverse
//    RoPE) itself; otherwise it writes (max, sum, unnormalised O) and
//    attn_combine_kernel merges the splits.  Splits are used only while the
//    items alone would leave most compute units idle.
// attn_generic_kernel: any head count and dim (one workgroup per query and
// head, fp32 throughout); used for small shapes such as the toy.
//
// Dense mode (heavily compressed attention, "DeepSeek V4 Inside", section
// "What does HCA change?": no indexer, dense attention over every visible
// compressed entry plus the window): no index list; the selected records
// of a query are all records s < min(n_rec, (t+1)/m), in id order.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "launch.h"
namespace csa2 {

// Arguments of attn_mfma_kernel and attn_combine_kernel (built by the host
// launch in attn.hip).
struct AttnP {
    int B, Tq, N, K, S, W, nsplit, per_split;
    int n_items;              // work items (decode layout: padded, see decode_item)
    int dense_m;              // > 0: dense mode, every record visible at compression dense_m (no idx)
    const int32_t* n_rec;     // dense mode: [B] records written per sequence, or null for N
    const uint16_t* q;        // bf16 [B][Tq][64][512]
    const uint8_t* kv;        // rows, bf16 or e4m3
    const float* kv_scale;
    const int32_t* idx;       // [B][Tq][K]
    const uint8_t* swa;
    const float* swa_scale;
    const int64_t* q_pos;
    const float* sink;
    float sm;
    int rope_dims;
    float rope_base;
    void* out;                // [B][Tq][64][512], float32 or bf16 (out_bf16)
    int out_bf16;
    float* part_o;            // [Q][nsplit][64][512]
    float* part_ml;           // [Q][nsplit][64][2]
};

// Launches attn_mfma_kernel's 16-head decode layout (attn_dec.hip, whose
// matrix instructions accumulate in VGPRs) for records of kv_dtype on grid
// workgroups; returns the launch status.
int launch_attn_decode(const AttnP& p, unsigned grid, int kv_dtype, hipStream_t st);

namespace {


constexpr int kH = 64;
constexpr int kD = 512;
constexpr int kTile = 32;
constexpr int kMaxKList = 2048;
constexpr int kMaxRope = kD / 2;
constexpr int kMaxSplits = 32;
constexpr float kJump = 64.f;
// sched_barrier mask: VALU, SALU and transcendental instructions may be
// scheduled across; memory and MFMA instructions keep their order
constexpr int kMayCross = 0x0002 | 0x0004 | 0x0400;  // log2 units: largest probability is 2^kJump

constexpr int kXPitch = kD * 2 + 32;  // bytes per LDS tile row (bf16); 32-byte skew per row
constexpr int kBuf = kTile * kXPitch;   // one tile buffer
constexpr int kMaxWin = 256;
constexpr int kMaxEnt = kMaxKList + kMaxWin;  // entries of one split (multiple of kTile)
constexpr float kLog2e = 1.4426950408889634f;

// Four output channels at element e of the output: float32, or bf16
// rounded to nearest even (8 bytes; e is a multiple of 4).
__device__ __forceinline__ void store_out4(void* out, size_t e, f32x4 v, bool bf16) {
    if (bf16) {
        const u32x2 w = {cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e));
    } else {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(out) + e));
    }
}

// Barrier for LDS hand-offs: this wave's LDS accesses are complete, then
// all waves meet.  Unlike __syncthreads() it does not wait for outstanding
// global loads (the tile prefetches keep flowing across it); the asm is
// also a compiler memory barrier.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Every tile copy of this wave except the newest eight (one tile's) has
// completed.
__device__ __forceinline__ void wait_copies_but_8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ void wait_copies_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copies the 1 KiB row at rp (a wave-uniform address, held in SGPRs)
// straight into LDS at byte address lds: lane l moves the 16 bytes at
// rp + voff with voff = 16 l (gfx950 global_load_lds_dwordx4, LDS address
// in M0).  Issued as asm so that the compiler does not serialise later LDS
// reads of the other tile buffers behind it: completion is awaited
// explicitly with the waits above.
__device__ __forceinline__ void row_copy16(const uint8_t* rp, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(rp)
                 : "memory", "m0");
}

__device__ __forceinline__ float max8(const float (&d)[8]) {
    return fmaxf(fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3])), fmaxf(fmaxf(d[4], d[5]), fmaxf(d[6], d[7])));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((const __attribute__((address_space(3))) uint8_t*)(p)));
}

// 64-bit address held by the first lane, as a wave-uniform (SGPR) value.
// readfirstlane returns a signed int: both halves go through uint32_t so
// that the low half is not sign-extended into the high one.
__device__ __forceinline__ const uint8_t* uniform_ptr(uint32_t lo, uint32_t hi) {
    const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lo)));
    const uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(hi)));
    return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(h) << 32) | l);
}

constexpr int kWaves = 4;   // one wave per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kIdsPerThread = kMaxKList / kThreads;
constexpr int kRowsPerWave = kTile / kWaves;  // tile rows each wave copies
constexpr int kStagePitch = 1040;  // finish: padded LDS row (bytes) staging 256 f32 channels

template <int KVDT>
struct __align__(16) AttnShared {
    // tile buffers: P.V on tile t, S^T on t+1, copies of t+2 (and, for
    // bf16, t+3) in flight
    static constexpr int kNB = (KVDT == DT_BF16) ? 4 : 3;
    static constexpr int kScaled = (KVDT != DT_BF16) ? kMaxEnt : 4;
    // bf16 keeps the compacted id list in the last tile buffer: it is only
    // live while an item is set up, when no copy is in flight
    static constexpr int kListOwn = (KVDT == DT_BF16) ? 4 : kMaxKList;
    uint8_t xb[kNB][kBuf];                  // tile buffers (row-major: entry, channel)
    uint64_t eptr[kMaxEnt];                 // row address of each entry of the work item
    float ezf[kScaled];                     // e4m3: logit factor sm * log2(e) * row scale
    float epf[kScaled];                     // e4m3: row scale (weights the probability)
    int32_t list_own[kListOwn];             // compacted valid record ids (e4m3)
    float rope_cs[kD / 2][2];               // (cos, sin) per channel pair; (1, 0) off the rotary channels
    double rope_inv[kMaxRope];              // base^(-2j/r), once per workgroup
    int cnt[kIdsPerThread][kWaves];         // valid ids per (chunk, wave)
    f32x4 spart[kWaves][64];                // decode: each wave's partial S^T, one f32x4 per lane
    __device__ __forceinline__ int32_t* list() {
        if constexpr (KVDT == DT_BF16) return reinterpret_cast<int32_t*>(xb[kNB - 1]);
        else return list_own;
    }
};

// The next work item's inputs, fetched into registers while the current
// item runs: its slice of the index row and its position (during the first
// tile), and the wave's query fragments (head h, k-step i covering channels
// 32i .. 32i+31, lane group g taking 8 of them; in the decode layout only the
// eight k-steps of the wave's channel half) once the tile loop is done, so
// that they occupy no registers during it.
struct ItemFetch {
    int ids[kIdsPerThread];
    int64_t t;
    float sink;  // the lane's head's sink logit
    bf16x8 q[16];
};

// Waits for the next item's ids, position and sink now, at the end of an
// item (its last copies have landed, the next query loads are not yet out).
// The compiler's waits count only its own loads, so the first use of these
// values in the next item's set-up would get a full wait that also covers
// the query loads issued in between.  Reading them in an asm statement
// moves that wait here without changing where the values live.
__device__ __forceinline__ void settle_fetch(const ItemFetch& f) {
    int s = static_cast<int>(f.t) ^ __float_as_int(f.sink);
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) s |= f.ids[j];
    asm volatile("; fetched %0" ::"v"(s));
}

// The same for the query fragments, in the first tile of an item once its
// own copies have landed (the query loads went out before them): without
// it the first S^T waits for everything issued since, including the next
// item's fetch and the copies of tile 2.  AGPR: where the prefill MFMAs
// read them from; VGPR: the decode layout's.
template <bool AGPR, int N>
__device__ __forceinline__ void settle_q_regs(const bf16x8 (&q)[16]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (AGPR) asm volatile("; query %0" ::"a"(q[i]));
        else asm volatile("; query %0" ::"v"(q[i]));
    }
}

// Work items are (query, split) pairs; with one split, item i is query
// Q-1-i so that later positions (more entries) come first.  Persistent
// workgroup g takes the item of round r at r*G + g for even r and
// r*G + G-1-g for odd r, which evens out the per-workgroup totals.  It
// walks the rounds starting at round g mod R (wrapping): workgroups that
// all finished an item at the same moment would write their outputs in one
// burst that saturates HBM while the matrix units idle; staggered starts
// spread those writes over the run.
__device__ __forceinline__ int item_of(int round, int g, int G) {
    return round * G + ((round & 1) ? (G - 1 - g) : g);
}

// Compacts the item's valid record ids (0 <= id < N, in index order) into
// sh.list() and returns their count (wave-uniform).  ids: this thread's
// chunks of the index row (-1 past its end); sh.cnt holds the per-(chunk,
// wave) counts.
template <class SH>
__device__ __forceinline__ int compact_ids(SH& sh, const int (&ids)[kIdsPerThread], int nids, int N, int wave,
                                           int lane) {
    int ok_bits = 0;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
        if (j < nids) {
            const int rec = ids[j];
            const bool ok = rec >= 0 && rec < N;
            const unsigned long long bal = __ballot(ok);
            if (ok) ok_bits |= 1 << j;
            if (lane == 0) sh.cnt[j][wave] = __popcll(bal);
        }
    }
    lds_sync();
    int nsel = 0;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
        if (j < nids) {
            int before = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) before += (w < wave) ? sh.cnt[j][w] : 0;
            const bool ok = (ok_bits >> j) & 1;
            const unsigned long long bal = __ballot(ok);
            if (ok) sh.list()[nsel + before + __popcll(bal & ((1ull << lane) - 1ull))] = ids[j];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) nsel += sh.cnt[j][w];
        }
    }
    return __builtin_amdgcn_readfirstlane(nsel);
}

// Persistent: gridDim.x workgroups of 4 waves (one per SIMD) walk the work
// items.  Wave w owns heads 16w .. 16w+15 over all 512 channels, so each
// wave has the complete logits of its heads and no partial sums cross
// waves.  Per work item:
//  * the valid selected records are compacted in order and, for the
//    item's entries [j0, j1), a table of row addresses is built (entries
//    past j1 up to the next multiple of the tile repeat the last row, so
//    every tile is a full one; their probabilities are zeroed);
//  * tile rows are copied global -> LDS in row-major order (entry,
//    channel), two tiles ahead of the one being multiplied; each wave
//    copies eight rows per tile from wave-uniform addresses;
//  * S^T = X Q^T reads 16-byte row chunks (entries on M, heads on N);
//    O^T += X^T P^T reads its operand with the gfx950 transposing LDS load:
//    within each 16-lane group, lane j receives element j%4 of the 64-bit
//    chunk addressed by lane 4k+j/4 (k = 0..3), so pointing lane s of group
//    g at X[4g + s/4][d0 + 4(s%4) ..] hands lane j the four entries
//    4g..4g+3 of channel d0 + j -- the MFMA A operand;
//  * logits are kept in log2 units (exp2 on the VALU).
// While an item runs, the next item's index slice, position and query
// fragments are loaded into registers, so an item starts without waiting
// for global memory.
// Decode layout: item i of a grid whose size is a multiple of 8 runs on XCD
// i mod 8 (workgroups are dispatched to the 8 XCDs in turn); the four head
// groups of one (query, split) get items on the same XCD, in the same
// round, so the rows they all gather are fetched from HBM once and read
// from that XCD's L2 by the other three.
struct DecItem {
    int qs, hg;  // (query, split) index and head group
};
__device__ __forceinline__ DecItem decode_item(int i) {
    const int k = i >> 3;
    return DecItem{8 * (k >> 2) + (i & 7), k & 3};
}

template <int KVDT, int NHG>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(AttnP p) {
    __shared__ AttnShared<KVDT> sh;
    constexpr int kRowBytes = (KVDT == DT_BF16) ? kD * 2 : kD;  // window rows (e4m3 when records are fp4)
    // record rows: fp4 holds D/2 code bytes then D/16 E4M3 group scales
    constexpr int kGRowBytes = (KVDT == DT_FP4) ? kD / 2 + kD / 16 : kRowBytes;
    // NHG = 64: wave w owns heads 16w .. 16w+15 over all 512 channels.
    // NHG = 16 (decode): the workgroup owns one group of 16 heads; every
    // wave computes the same logits and softmax for them and owns channels
    // 128w .. 128w+127 of their P.V (O is then 32 registers).
    constexpr bool kDec = NHG == 16;
    constexpr int kU = kDec ? 8 : 32;      // 16-channel blocks of O per wave
    constexpr int kUG = kU / 8;            // blocks per channel group of the MFMA stream
    // S^T k-steps of each wave: NHG = 64, all 16 of its heads' 512 channels;
    // decode, 8: wave w forms the partial S^T of tile entries 16 (w & 1) ..
    // +15 over channels 256 (w >> 1) .. +255, and the four partials are
    // summed through LDS (every wave then holds the whole S^T, as in the
    // NHG = 64 layout, at a quarter of the matrix work and row reads)
    constexpr int kQS = kDec ? 8 : 16;
    static_assert(NHG == 16 || NHG == 64, "head groups of 16 or 64");
    // 64-head layout: an operand in an accumulation register tells the
    // compiler that this kernel uses them, so it selects the MFMA form whose
    // accumulator lives in AGPRs: O (128 registers) then stays there across
    // the tile loop instead of being copied to and from VGPRs on every
    // iteration.  The decode layout's O is 32 registers; its translation
    // unit selects the VGPR form, which keeps O and the logits in VGPRs
    // (with AGPR accumulators the logits displaced O into VGPRs and back on
    // every tile).
    if constexpr (!kDec) asm volatile("" ::"a"(0.f));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int ch0 = kDec ? 128 * wave : 0;  // first channel of the wave's O
    const int kb = kDec ? 8 * (wave >> 1) : 0;  // first k-step of the wave's S^T
    const int mt = kDec ? (wave & 1) : 0;       // decode: the wave's 16 entries of a tile
    const int Q = p.B * p.Tq;
    const int n_items = p.n_items;
    const int G = gridDim.x;
    const float cz = p.sm * kLog2e;
    const int nids = p.dense_m ? 0 : (p.K + kThreads - 1) / kThreads;  // index chunks per thread
    const uint32_t voff = 16u * lane;

    auto item_ok = [&](int item) { return !kDec || decode_item(item).qs < Q * p.nsplit; };
    auto query_of = [&](int item) {
        if constexpr (kDec) return decode_item(item).qs / p.nsplit;
        return p.nsplit == 1 ? Q - 1 - item : item / p.nsplit;
    };
    auto split_of = [&](int item) {
        if constexpr (kDec) return decode_item(item).qs % p.nsplit;
        return p.nsplit == 1 ? 0 : item % p.nsplit;
    };
    auto head_of = [&](int item) {  // this lane's head
        if constexpr (kDec) return 16 * decode_item(item).hg + l16;
        return 16 * wave + l16;
    };
    auto fetch = [&](int item, ItemFetch& f) {
        const int qr = query_of(item);
        const int32_t* irow = nids ? p.idx + static_cast<size_t>(qr) * p.K : nullptr;
#pragma unroll
        for (int j = 0; j < kIdsPerThread; ++j) {
            const int c = j * kThreads + tid;
            f.ids[j] = (j < nids && c < p.K) ? irow[c] : -1;
        }
        f.t = p.q_pos[qr];
        f.sink = p.sink[head_of(item)];
    };
    auto fetch_q = [&](int item, ItemFetch& f) {
        const uint16_t* qh = p.q + (static_cast<size_t>(query_of(item)) * kH + head_of(item)) * kD;
#pragma unroll
        for (int i = 0; i < kQS; ++i) f.q[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 8 * (4 * (kb + i) + g)));
    };

    ItemFetch nx;
    const int R = (n_items + G - 1) / G;  // rounds
    // decode: rounds in order, item r*G + g (G is a multiple of 8, so a
    // workgroup stays on its XCD's share of the items)
    const int rot = kDec ? 0 : static_cast<int>(blockIdx.x) % R;
    int k_next = 0;  // position in this workgroup's round order
    auto next_item = [&]() -> int {
        while (k_next < R) {
            const int r = k_next + rot < R ? k_next + rot : k_next + rot - R;
            ++k_next;
            const int it = kDec ? r * G + static_cast<int>(blockIdx.x) : item_of(r, blockIdx.x, G);
            if (it < n_items && item_ok(it)) return it;  // only the last round is partial
        }
        return n_items;
    };
    int item = next_item();
    if (item < n_items) {
        fetch(item, nx);
        fetch_q(item, nx);
    }
    // the pow() is far costlier than the per-item angle, so it runs once,
    // while the first item's inputs are on their way
    for (int i = tid; i < p.rope_dims / 2; i += kThreads) sh.rope_inv[i] = rope_inv_freq(i, p.rope_dims, p.rope_base);
    settle_fetch(nx);

    // Output of an item.  It runs once the next item's first tile copies
    // are in flight (its stores then drain while those copies land), so O,
    // m and l persist across items.
    f32x4 acc[kU];
    float m_run = -__builtin_huge_valf();  // running max, log2 units (same in the 4 lanes of a head)
    float l_run = 0.f;                     // this lane's share of the running sum
    int prev_qr = -1, prev_split = 0, prev_h = 0;  // the item whose output is pending
    float prev_sink = 0.f;
    // the sink logit was fetched with the item's inputs: a load here would
    // wait for every copy and load in flight, including the next item's
    auto finish = [&](int qr_f, int split_f, int h_f) {
        const int hb = h_f - l16;  // first head of the wave's 16
        float f = 1.f;  // normalisation (one split) or none (partials)
        void* dst;      // output (one split) or the split's partials, as elements from dst0
        size_t dst0;
        bool obf = false;
        if (p.nsplit == 1) {
            const float sk = prev_sink * kLog2e;  // the head's sink logit, log2 units
            const float a = fmaxf(m_run, sk);
            f = 0.f;
            if (a != -__builtin_huge_valf()) {
                const float em = __builtin_amdgcn_exp2f(m_run - a);
                const float es = __builtin_amdgcn_exp2f(sk - a);
                const float den = l_run * em + es;
                f = den > 0.f ? em / den : 0.f;
            }
            dst = p.out;
            dst0 = (static_cast<size_t>(qr_f) * kH + hb) * kD;
            obf = p.out_bf16;
        } else {
            const size_t slot0 = (static_cast<size_t>(qr_f) * p.nsplit + split_f) * kH + hb;
            dst = p.part_o;
            dst0 = slot0 * kD;
            if (g == 0 && (!kDec || wave == 0)) {  // decode: every wave holds the same m and l
                p.part_ml[2 * (slot0 + l16)] = m_run;  // log2 units
                p.part_ml[2 * (slot0 + l16) + 1] = l_run;
            }
        }
        // rotary channels [r0, kD) get the inverse rotation (one split
        // only); the table holds (cos, sin) for every channel pair, (1, 0)
        // below r0.  Lane (head hb + l16, group g) holds channels ch0 + 16u
        // + 4g .. +3, whose two rotary pairs are its own.
        int r0 = p.nsplit == 1 ? kD - p.rope_dims : kD;
        asm volatile("" : "+s"(r0));  // tested per block here, not hoisted out of the item loop
        if constexpr (kDec) {
            // decode: straight from the accumulators (each store writes
            // 64-byte runs of 16 heads' rows; the wave's 8 stores complete
            // every 512-byte run)
            const size_t e0 = dst0 + static_cast<size_t>(l16) * kD + ch0 + 4 * g;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                f32x4 v = acc[u] * f;
                if (ch0 + 16 * u + 16 > r0) {  // wave-uniform: the block holds rotary channels
                    const f32x4 cs = *reinterpret_cast<const f32x4*>(&sh.rope_cs[(ch0 + 16 * u + 4 * g) / 2][0]);
                    const float x0 = v[0], y0 = v[1], x1 = v[2], y1 = v[3];
                    v[0] = x0 * cs[0] + y0 * cs[1];
                    v[1] = y0 * cs[0] - x0 * cs[1];
                    v[2] = x1 * cs[2] + y1 * cs[3];
                    v[3] = y1 * cs[2] - x1 * cs[3];
                }
                store_out4(dst, e0 + 16 * u, v, obf);
            }
            return;
        }
        // prefill: 256 channels of the wave's 16 heads at a time go through
        // LDS (the last two tile buffers; the next item's first copies target
        // the first two; rows padded so that the lanes of one write pass hit
        // distinct banks), so that every store writes whole 1 KB runs of one
        // head's row (measured faster than the 64-byte runs of storing from
        // the accumulators, for this layout's larger outputs)
        static_assert(kWaves * 16 * kStagePitch <= 2 * kBuf, "staging fits the last two tile buffers");
        uint8_t* stage = &sh.xb[AttnShared<KVDT>::kNB - 2][0] + wave * 16 * kStagePitch;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int u = 0; u < 16; ++u)
                *reinterpret_cast<f32x4*>(stage + l16 * kStagePitch + 4 * (16 * u + 4 * g)) = acc[16 * half + u] * f;
            const bool rot = 256 * half + 256 > r0;  // wave-uniform: this half holds rotary channels
            // this lane's channels 256*half + 4*lane .. +3: pairs p0, p0 + 1
            const f32x4 cs = *reinterpret_cast<const f32x4*>(&sh.rope_cs[128 * half + 2 * lane][0]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // staged rows visible to the wave
            f32x4 rows[16];  // all reads in flight at once
#pragma unroll
            for (int r = 0; r < 16; ++r) rows[r] = *reinterpret_cast<const f32x4*>(stage + r * kStagePitch + 16 * lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                f32x4 v = rows[r];
                if (rot) {
                    const float x0 = v[0], y0 = v[1], x1 = v[2], y1 = v[3];
                    v[0] = x0 * cs[0] + y0 * cs[1];
                    v[1] = y0 * cs[0] - x0 * cs[1];
                    v[2] = x1 * cs[2] + y1 * cs[3];
                    v[3] = y1 * cs[2] - x1 * cs[3];
                }
                store_out4(dst, dst0 + r * kD + 256 * half + 4 * lane, v, obf);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next half overwrites
        }
    };


    while (item < n_items) {
        const int qr = query_of(item);
        const int split = split_of(item);
        const int hh = head_of(item);
        const int b = qr / p.Tq;
        const int64_t t = nx.t;
        const float sink = nx.sink;
        const int rd = p.rope_dims;
        bf16x8 qf[16];  // filled from nx just before the first S^T (its loads land meanwhile)
        auto settle_q = [](const bf16x8 (&q)[16]) { settle_q_regs<!kDec, kQS>(q); };

        // ---- compact the valid selected records (in order) ----
        int nsel = compact_ids(sh, nx.ids, nids, p.N, wave, lane);
        if (p.dense_m) {  // dense: every visible record, in id order
            const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
            const int64_t v = t < 0 ? 0 : (t + 1) / p.dense_m;
            nsel = static_cast<int>(v < nrec ? v : nrec);
        }
        const int nwin = t < 0 ? 0 : static_cast<int>(t + 1 < p.W ? t + 1 : p.W);
        const int slot0 = static_cast<int>((t - nwin + 1) % p.S);  // ring slot of the first window row
        const int E = nsel + nwin;
        const int j0 = split * p.per_split;
        const int j1 = min(E, j0 + p.per_split);
        const int nvalid = j1 - j0;  // entries of this item
        const int ntile = nvalid > 0 ? (nvalid + kTile - 1) / kTile : 0;
        lds_sync();  // list complete

        // ---- entry table ----
        for (int e = tid; e < ntile * kTile; e += kThreads) {
            const int ge = min(j0 + e, j1 - 1);
            const uint8_t* rp;
            float sc = 1.f;
            if (ge < nsel) {
                const size_t r = static_cast<size_t>(b) * p.N + (p.dense_m ? ge : sh.list()[ge]);
                if constexpr (KVDT == DT_E4M3) sc = p.kv_scale[r];
                rp = p.kv + r * kGRowBytes;
            } else {
                int slot = slot0 + (ge - nsel);  // < 2S since the window has at most S rows
                if (slot >= p.S) slot -= p.S;
                const size_t r = static_cast<size_t>(b) * p.S + slot;
                if constexpr (KVDT != DT_BF16) sc = p.swa_scale[r];
                rp = p.swa + r * kRowBytes;
            }
            sh.eptr[e] = reinterpret_cast<uint64_t>(rp);
            if constexpr (KVDT != DT_BF16) {
                sh.ezf[e] = cz * sc;
                sh.epf[e] = sc;
            }
        }
        lds_sync();  // table visible

        // Tile staging: wave w fills rows 8w .. 8w+7 of the tile.  bf16 rows
        // go straight from global memory into LDS; e4m3 rows are converted to
        // bf16 in registers on the way (staged one tile ahead); so are fp4
        // record rows (lane l: the code dword of channels 8l .. 8l+7 and the
        // E4M3 scale of their group), whose window rows are e4m3.  Entry e of
        // the item is a record while e < ng (padding repeats the last entry).
        typedef typename std::conditional<KVDT == DT_BF16, u32x4, u32x2>::type Raw;
        Raw stg[kRowsPerWave];
        const int ng = max(0, min(nsel - j0, nvalid));
        auto rec4 = [&](int e) { return KVDT == DT_FP4 && min(e, nvalid - 1) < ng; };
        auto issue = [&](int it, int k) {
            const u32x4* ep = reinterpret_cast<const u32x4*>(&sh.eptr[it * kTile + kRowsPerWave * wave]);
            if constexpr (KVDT == DT_BF16) {
                // all addresses first: each copy is asm with a memory clobber,
                // which no later LDS read may pass
                u32x4 pa[kRowsPerWave / 2];
#pragma unroll
                for (int i = 0; i < kRowsPerWave / 2; ++i) pa[i] = ep[i];
                const uint32_t dst = lds_addr(sh.xb[k]) + kRowsPerWave * wave * kXPitch;
#pragma unroll
                for (int i = 0; i < kRowsPerWave; i += 2) {
                    row_copy16(uniform_ptr(pa[i / 2][0], pa[i / 2][1]), voff, dst + i * kXPitch);
                    row_copy16(uniform_ptr(pa[i / 2][2], pa[i / 2][3]), voff, dst + (i + 1) * kXPitch);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kRowsPerWave; i += 2) {
                    const u32x4 pa = ep[i / 2];
                    // global (not flat) loads: a flat load would also count
                    // against the LDS wait counter, so every LDS wait would
                    // wait for these staging loads as well
                    typedef const __attribute__((address_space(1))) Raw GRaw;
                    typedef const __attribute__((address_space(1))) uint32_t G32;
                    typedef const __attribute__((address_space(1))) uint8_t G8;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const uint8_t* rp = uniform_ptr(pa[2 * h2], pa[2 * h2 + 1]);
                        if (rec4(it * kTile + kRowsPerWave * wave + i + h2)) {  // wave-uniform
                            stg[i + h2][0] = *(G32*)(rp + 4 * lane);
                            stg[i + h2][1] = *(G8*)(rp + kD / 2 + (lane >> 1));
                        } else {
                            stg[i + h2] = *(GRaw*)(rp + 8 * lane);
                        }
                    }
                }
            }
        };
        auto land = [&](int it, int k) {  // e4m3 and fp4: staged registers -> LDS
            if constexpr (KVDT != DT_BF16) {
                uint8_t* xb = sh.xb[k];
#pragma unroll
                for (int i = 0; i < kRowsPerWave; ++i) {
                    u32x4 v;
                    if (rec4(it * kTile + kRowsPerWave * wave + i))
                        v = fp4x8_to_bf16x8(stg[i][0], e4m3_to_f32(static_cast<uint8_t>(stg[i][1])));
                    else
                        v = e4m3x8_to_bf16x8(stg[i]);
                    *reinterpret_cast<u32x4*>(xb + (kRowsPerWave * wave + i) * kXPitch + 16 * lane) = v;
                }
            }
        };


        // Pipeline over tiles: iteration t runs the P.V of tile t with the
        // S^T and the softmax of tile t+1 interleaved (independent work in one
        // basic block, so the matrix units stay busy while the LDS reads and
        // the VALU softmax proceed).  Copies run two tiles ahead of the S^T:
        // bf16 copies tile t+3 into tile t-1's buffer (4 buffers); e4m3
        // stages the next tile in registers (3 buffers).
        //
        // Each head keeps a reference max, set by the first tile: it only
        // moves when a tile exceeds it by more than kJump (log2 units), so
        // probabilities stay below 2^kJump and the usual per-tile rescale of
        // O and l happens only on such a (rare) move.
        constexpr int NB = AttnShared<KVDT>::kNB;
        const int nxt = next_item();
        if (ntile > 0) issue(0, 0);
        if constexpr (KVDT == DT_BF16) {
            if (ntile > 1) issue(1, 1);
        }
        if (prev_qr >= 0) {
            finish(prev_qr, prev_split, prev_h);
            lds_sync();  // every wave is done with the previous item's rope table
        }
        m_run = -__builtin_huge_valf();
        l_run = 0.f;
#pragma unroll
        for (int i = 0; i < kU; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.nsplit == 1)
            for (int i = tid; i < kD / 2; i += kThreads) {
                const int j = i - (kD - rd) / 2;  // rotary pair index of channel pair i
                float c = 1.f, sn = 0.f;
                if (j >= 0) rope_cos_sin(t, sh.rope_inv[j], c, sn);
                sh.rope_cs[i][0] = c;
                sh.rope_cs[i][1] = sn;
            }

        // tile `it` visible in LDS to every wave; the copies of the tile two
        // ahead go out.  The next item's inputs are fetched in tile 0, after
        // its wait and before those copies: the copy waits then cover the
        // fetch only from tile 1 on, one tile after it was issued.
        auto tile_ready = [&](int it) {
            const int buf = it % NB;
            if constexpr (KVDT == DT_BF16) {
                if (it + 1 < ntile) wait_copies_but_8();
                else wait_copies_all();
                lds_sync();  // tile `it` landed; the buffer two tiles ahead is free
                if (it == 0) settle_q(qf);
                if (it == 0 && nxt < n_items) fetch(nxt, nx);
                // later copies go out from inside the MFMA stream (below)
                if (it == 0 && it + 2 < ntile) issue(it + 2, (it + 2) % NB);
            } else {
                land(it, buf);
                if (it == 0 && nxt < n_items) fetch(nxt, nx);
                if (it + 1 < ntile) issue(it + 1, (it + 1) % NB);
                lds_sync();
            }
        };
        // S^T of tile `it` (entries 0..15: s[0], s[2]; 16..31: s[1], s[3]) in
        // four steps of two k-step pairs each, which the P.V of the previous
        // tile interleaves with its MFMAs; the row chunks of pair i+2 are
        // read before the MFMAs of pair i (two pairs in flight hide the LDS
        // latency).  Decode: four steps of one pair each for the wave's 16
        // entries (s[0], s[1]: even and odd k-steps); qk_share publishes
        // their sum and, past a barrier, qk_gather reads the four partials
        // back into s[0] .. s[3] in the layout above.  qk_end forms d = z - m for the lane's entries 16*mt +
        // 4g + v of head h (z in log2 units, m the head's reference) and
        // reports whether any of them exceeds the lazy threshold.  Padding
        // entries repeat a real row, so they may take part in a maximum; only
        // their probabilities are dropped.
        struct Qk {
            f32x4 s[4];
            u32x4 ka[3][4];
            const uint8_t* r0;
        };
        auto kload = [&](const Qk& q, int i, u32x4* d) {
            if constexpr (kDec) {
                d[0] = *reinterpret_cast<const u32x4*>(q.r0 + 64 * i);
                d[1] = *reinterpret_cast<const u32x4*>(q.r0 + 64 * (i + 1));
                return;
            }
            const uint8_t* r1 = q.r0 + 16 * kXPitch;
            d[0] = *reinterpret_cast<const u32x4*>(q.r0 + 64 * i);
            d[1] = *reinterpret_cast<const u32x4*>(r1 + 64 * i);
            d[2] = *reinterpret_cast<const u32x4*>(q.r0 + 64 * (i + 1));
            d[3] = *reinterpret_cast<const u32x4*>(r1 + 64 * (i + 1));
        };
        auto qk_begin = [&](int it, Qk& q) {
            q.r0 = sh.xb[it % NB] + (16 * mt + l16) * kXPitch + 16 * g + 64 * kb;
#pragma unroll
            for (int m = 0; m < 4; ++m) q.s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            kload(q, 0, q.ka[0]);
            kload(q, 2, q.ka[1]);
        };
        auto qk_step = [&](Qk& q, int j) {
            if constexpr (kDec) {
                const int i = 2 * j;  // k-step pair i, i+1 of the wave's eight
                const int k = j % 3;
                if (i + 4 < kQS) kload(q, i + 4, q.ka[(j + 2) % 3]);
                q.s[0] = mfma16x16x32(as_bf16x8(q.ka[k][0]), qf[i], q.s[0]);
                q.s[1] = mfma16x16x32(as_bf16x8(q.ka[k][1]), qf[i + 1], q.s[1]);
                return;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 4 * j + 2 * e;  // k-step pair i, i+1
                const int k = (i / 2) % 3;
                if (i + 4 < 16) kload(q, i + 4, q.ka[(i / 2 + 2) % 3]);
                q.s[0] = mfma16x16x32(as_bf16x8(q.ka[k][0]), qf[i], q.s[0]);
                q.s[1] = mfma16x16x32(as_bf16x8(q.ka[k][1]), qf[i], q.s[1]);
                q.s[2] = mfma16x16x32(as_bf16x8(q.ka[k][2]), qf[i + 1], q.s[2]);
                q.s[3] = mfma16x16x32(as_bf16x8(q.ka[k][3]), qf[i + 1], q.s[3]);
            }
        };
        auto qk_share = [&](const Qk& q) { sh.spart[wave][lane] = q.s[0] + q.s[1]; };
        auto qk_gather = [&](Qk& q) {  // partials of waves 0, 2 (entries 0..15) and 1, 3 (16..31)
#pragma unroll
            for (int w = 0; w < kWaves; ++w) q.s[(w & 1) + 2 * (w >> 1)] = sh.spart[w][lane];
        };
        auto qk_end = [&](int it, Qk& q, float m, float (&d)[8]) -> bool {
            const f32x4 s0 = q.s[0] + q.s[2];
            const f32x4 s1 = q.s[1] + q.s[3];
            if constexpr (KVDT != DT_BF16) {  // per-entry scales (fp4 records: 1)
                const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sh.ezf[it * kTile + 4 * g]);
                const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sh.ezf[it * kTile + 16 + 4 * g]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    d[v] = fmaf(s0[v], f0[v], -m);
                    d[4 + v] = fmaf(s1[v], f1[v], -m);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    d[v] = fmaf(s0[v], cz, -m);
                    d[4 + v] = fmaf(s1[v], cz, -m);
                }
            }
            return max8(d) > kJump;
        };
        // Softmax of tile `it`, in eight steps that the P.V of the previous
        // tile interleaves with its MFMAs.  Steps 0-3: two probabilities
        // 2^(d - shift) each; step 4: their sum (and the e4m3 row scales);
        // steps 4-7: one packed pair each of P = hi + lo in bf16 (hi is P
        // rounded, lo the rounding error).  In the stream (MASK false) no
        // entry is dropped and the shift is 0: tiles that hold padding
        // entries, or in which some head passes the lazy threshold, are
        // redone afterwards with MASK true.
        struct Soft {
            float pr[8];
            float psum;
            uint32_t phi[4], plo[4];
        };
        auto soft_step = [&](int j, int it, const float (&d)[8], float shift, Soft& s, auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            if (j < 4) {
                if constexpr (MASK) {
                    const int lim = nvalid - it * kTile;  // entries of this tile that are real
                    s.pr[j] = (4 * g + j < lim) ? __builtin_amdgcn_exp2f(d[j] - shift) : 0.f;
                    s.pr[4 + j] = (16 + 4 * g + j < lim) ? __builtin_amdgcn_exp2f(d[4 + j] - shift) : 0.f;
                } else {
                    s.pr[j] = __builtin_amdgcn_exp2f(d[j]);
                    s.pr[4 + j] = __builtin_amdgcn_exp2f(d[4 + j]);
                }
                // computed here, in the MFMA shadow: the results are only read
                // after the loop's branch, past which the compiler would sink them
                asm volatile("" : "+v"(s.pr[j]), "+v"(s.pr[4 + j]));
                return;
            }
            if (j == 4) {
                s.psum = ((s.pr[0] + s.pr[1]) + (s.pr[2] + s.pr[3])) + ((s.pr[4] + s.pr[5]) + (s.pr[6] + s.pr[7]));
                if constexpr (KVDT != DT_BF16) {
                    const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sh.epf[it * kTile + 4 * g]);
                    const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sh.epf[it * kTile + 16 + 4 * g]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        s.pr[v] *= f0[v];
                        s.pr[4 + v] *= f1[v];
                    }
                }
            }
            const int i = j - 4;
            const uint32_t hi = cvt_bf16x2(s.pr[2 * i], s.pr[2 * i + 1]);
            s.phi[i] = hi;
            s.plo[i] = cvt_bf16x2(s.pr[2 * i] - __uint_as_float(hi << 16),
                                  s.pr[2 * i + 1] - __uint_as_float(hi & 0xFFFF0000u));
            asm volatile("" : "+v"(s.phi[i]), "+v"(s.plo[i]));
            if (j == 4) asm volatile("" : "+v"(s.psum));
        };
        // The exact softmax of tile `it` (first tile of an item, padded
        // tiles, threshold passes): heads whose tile maximum exceeds the
        // reference by more than kJump move their reference to it, rescaling
        // O and l; padding entries are dropped.
        auto soft_exact = [&](int it, const float (&d)[8], Soft& s) {
            const float hm = max4_rows(max8(d));  // head's tile max relative to m_run
            const bool jump = hm > kJump;
            const float shift = jump ? hm : 0.f;
            if (__any(jump)) {
                const float sc = __builtin_amdgcn_exp2f(-shift);
#pragma unroll
                for (int u = 0; u < kU; ++u) acc[u] *= sc;
                l_run *= sc;
            }
            m_run += shift;
#pragma unroll
            for (int j = 0; j < 8; ++j) soft_step(j, it, d, shift, s, std::true_type{});
        };
        auto packed = [](const uint32_t (&w)[4]) { return as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}); };
        // O^T += X^T P^T for tile `it`: channels ch0 + 16*u + 4g + v, head h.
        // The transposing read: lane s of group g -> row 4g + s/4 (and 16 +
        // ...), channels d0 + 4(s%4) .. +3; the operands of channel group
        // k+1 are read before the MFMAs of group k.  side(step) runs between
        // the MFMAs of each of the eight channel groups (kUG blocks each).
        auto tile_pv = [&](int it, const bf16x8& bhi, const bf16x8& blo, auto&& side) {
            const uint8_t* xb = sh.xb[it % NB];
            const uint8_t* tr0 = xb + (4 * g + (l16 >> 2)) * kXPitch + 8 * (l16 & 3) + 2 * ch0;
            const uint8_t* tr1 = tr0 + 16 * kXPitch;
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            // operands two channel groups ahead (bf16; e4m3 has no registers
            // to spare and reads one group ahead)
            constexpr int kVA = (KVDT == DT_BF16 || kDec) ? 3 : 2;
            bf16x8 va[kVA][kUG];
            auto vload = [&](int uh, bf16x8* d) {
#pragma unroll
                for (int u = 0; u < kUG; ++u) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(tr0 + 32 * (uh + u)));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(tr1 + 32 * (uh + u)));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    d[u] = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
                }
            };
            vload(0, va[0]);
            if constexpr (kVA == 3) vload(kUG, va[1]);
#pragma unroll
            for (int uh = 0; uh < kU; uh += kUG) {
                const int k = (uh / kUG) % kVA;
                if (uh + kUG * (kVA - 1) < kU) vload(uh + kUG * (kVA - 1), va[(k + kVA - 1) % kVA]);
                __builtin_amdgcn_sched_barrier(0);  // the reads above stay ahead
#pragma unroll
                for (int u = 0; u < kUG; ++u) acc[uh + u] = mfma16x16x32(va[k][u], bhi, acc[uh + u]);
                side(uh / kUG);
#pragma unroll
                for (int u = 0; u < kUG; ++u) acc[uh + u] = mfma16x16x32(va[k][u], blo, acc[uh + u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

#pragma unroll
        for (int i = 0; i < kQS; ++i) qf[i] = nx.q[i];
        bf16x8 bhi, blo;  // P of the tile whose P.V comes next
        if (ntile > 0) {
            float z[8];
            Soft s;
            Qk q;
            tile_ready(0);
            qk_begin(0, q);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                qk_step(q, j);
            }
            if constexpr (kDec) {
                qk_share(q);
                lds_sync();
                qk_gather(q);
            }
            qk_end(0, q, 0.f, z);
            // the first tile sets the reference: the head's maximum
            const float hm = max4_rows(max8(z));
            m_run = hm;
#pragma unroll
            for (int v = 0; v < 8; ++v) z[v] -= hm;
#pragma unroll
            for (int j = 0; j < 8; ++j) soft_step(j, 0, z, 0.f, s, std::true_type{});
            l_run = s.psum;
            bhi = packed(s.phi);
            blo = packed(s.plo);
        }
        // Every path into the tile loop has now waited for the query loads
        // (the first tile did, after its copies landed; an item without
        // tiles does so here).  Otherwise the compiler, unable to tell the
        // paths apart, waits for them inside the loop, before the S^T
        // MFMAs, with counts that also cover the row copies just issued
        // by the same step.
        settle_q(qf);
        // Iteration `it`: one stream of MFMAs -- the P.V of tile it, with the
        // S^T of tile it+1 in its first half and that tile's softmax in its
        // second half.
        // One iteration.  With CP (bf16, tile it+3 exists) the copies of tile
        // it+3 (into tile it-1's buffer, free since the barrier) go out one
        // row per channel group of the MFMA stream instead of stalling the
        // barrier phase; the two variants keep the stream branch-free.
        auto step = [&](int it, auto cp_tag) {
            constexpr bool CP = decltype(cp_tag)::value;
            // row addresses of the copies (wave-uniform, scalar registers),
            // read before the barrier so the reads land during its wait
            const uint8_t* rp[kRowsPerWave];
            uint32_t cdst = 0;
            if constexpr (CP) {
                const u32x4* ep = reinterpret_cast<const u32x4*>(&sh.eptr[(it + 3) * kTile + kRowsPerWave * wave]);
                u32x4 pa[kRowsPerWave / 2];
#pragma unroll
                for (int i = 0; i < kRowsPerWave / 2; ++i) pa[i] = ep[i];
#pragma unroll
                for (int i = 0; i < kRowsPerWave / 2; ++i) {
                    rp[2 * i] = uniform_ptr(pa[i][0], pa[i][1]);
                    rp[2 * i + 1] = uniform_ptr(pa[i][2], pa[i][3]);
                }
                cdst = lds_addr(sh.xb[(it + 3) % NB]) + kRowsPerWave * wave * kXPitch;
            }
            tile_ready(it + 1);
            Qk q;
            qk_begin(it + 1, q);
            float dn[8];
            bool over = false;
            Soft s;
            tile_pv(it, bhi, blo, [&](int j) {
                if constexpr (CP) row_copy16(rp[j], voff, cdst + j * kXPitch);
                if (j < 4) {
                    qk_step(q, j);
                    if (kDec && j == 3) qk_share(q);
                    return;
                }
                if constexpr (kDec) {
                    // the partials: published in step 3, complete past this
                    // barrier, summed in step 5; the softmax in steps 5-7
                    if (j == 4) {
                        lds_sync();
                        qk_gather(q);
                        return;
                    }
                    if (j == 5) over = qk_end(it + 1, q, m_run, dn);
                    constexpr int kFirst[5] = {0, 0, 3, 6, 8};  // softmax steps of stream steps 5, 6, 7
#pragma unroll
                    for (int k = kFirst[j - 4]; k < kFirst[j - 3]; ++k)
                        soft_step(k, it + 1, dn, 0.f, s, std::false_type{});
                    return;
                }
                if (j == 4) over = qk_end(it + 1, q, m_run, dn);
                soft_step(2 * (j - 4), it + 1, dn, 0.f, s, std::false_type{});
                soft_step(2 * (j - 4) + 1, it + 1, dn, 0.f, s, std::false_type{});
            });
            // rare: a head passes the threshold, or the tile holds padding
            if (__any(over) || nvalid - (it + 1) * kTile < kTile) soft_exact(it + 1, dn, s);
            l_run += s.psum;
            // O stays in the accumulation registers across iterations (else
            // the compiler keeps it in VGPRs and copies it in and out of the
            // MFMA accumulators every tile)
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if constexpr (kDec) asm volatile("" : "+v"(acc[u]));
                else asm volatile("" : "+a"(acc[u]));
            }
            bhi = packed(s.phi);
            blo = packed(s.plo);
        };
        int it = 0;
        if constexpr (KVDT == DT_BF16)
            for (; it + 3 < ntile; ++it) step(it, std::true_type{});
        for (; it + 1 < ntile; ++it) step(it, std::false_type{});
        if (ntile > 0) tile_pv(ntile - 1, bhi, blo, [](int) {});
        if (ntile == 0 && nxt < n_items) fetch(nxt, nx);
        settle_fetch(nx);
        if (nxt < n_items) fetch_q(nxt, nx);
        l_run = sum4_rows(l_run);  // the head's sum over the four lane groups
        prev_qr = qr;
        prev_split = split;
        prev_h = hh;
        prev_sink = sink;
        item = nxt;
    }
    if (prev_qr >= 0) {
        lds_sync();  // the last item's tiles are no longer read
        finish(prev_qr, prev_split, prev_h);
    }
}

}  // namespace
}  // namespace csa2
