// Sparse shared-latent attention with a sliding window and a sink: host
// launch, split merging and the generic kernel.  The MFMA kernel and its
// description are in attn_kernel.h.
#include <mutex>

#include "attn_kernel.h"

namespace csa2 {
namespace {

// Merges split partials: one workgroup per (query, pair of heads).  The
// split weights w_s = 2^(m_s - a) / den (a the largest of the partial maxima
// and the sink, den = 2^(sink - a) + sum_s l_s 2^(m_s - a)) are formed by one
// half-wave per head, one lane per split; then each thread sums four
// channels of one head over the splits, four splits' loads in flight at a
// time, and applies the inverse rotation.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnP p) {
    __shared__ float rope_cs[kMaxRope][2];
    __shared__ float wts[2][kMaxSplits];
    const int qr = blockIdx.x;
    const int h0 = 2 * blockIdx.y;
    const int tid = threadIdx.x;
    const int ns = p.nsplit;
    // this thread's channels of the first kPre splits load first: their
    // latency then overlaps the split weights and the rotary table
    const int hl = tid >> 7;  // 128 threads per head
    const int h = h0 + hl;
    const int d = 4 * (tid & 127);
    const float* pb = p.part_o + (static_cast<size_t>(qr) * ns * kH + h) * kD + d;
    constexpr int kPre = 16;
    f32x4 v0[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (i < ns) v0[i] = *reinterpret_cast<const f32x4*>(pb + static_cast<size_t>(i) * kH * kD);
    const int64_t t = p.q_pos[qr];
    const int rd = p.rope_dims;
    for (int i = tid; i < rd / 2; i += 256) rope_angle(t, i, rd, p.rope_base, rope_cs[i][0], rope_cs[i][1]);
    if (tid < 64) {
        const int hw = tid >> 5, s = tid & 31;
        const int h = h0 + hw;
        const float* ml = p.part_ml + ((static_cast<size_t>(qr) * ns + min(s, ns - 1)) * kH + h) * 2;
        const float m = s < ns ? ml[0] : -__builtin_huge_valf();  // log2 units
        const float l = s < ns ? ml[1] : 0.f;
        const float sk = p.sink[h] * kLog2e;
        float a = m;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
        a = fmaxf(a, sk);
        const float e = (m != -__builtin_huge_valf() && a != -__builtin_huge_valf()) ? __builtin_amdgcn_exp2f(m - a) : 0.f;
        float den = l * e;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) den += __shfl_xor(den, o);
        if (a != -__builtin_huge_valf()) den += __builtin_amdgcn_exp2f(sk - a);
        if (s < ns) wts[hw][s] = den > 0.f ? e / den : 0.f;
    }
    __syncthreads();
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (i < ns) x += wts[hl][i] * v0[i];
    for (int s0 = kPre; s0 < ns; s0 += 4) {
        f32x4 v[4];
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sc = min(s0 + i, ns - 1);  // past the last split: reread it with weight 0
            v[i] = *reinterpret_cast<const f32x4*>(pb + static_cast<size_t>(sc) * kH * kD);
            w[i] = s0 + i < ns ? wts[hl][sc] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) x += w[i] * v[i];
    }
    const int r0 = kD - rd;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        const int dd = d + i;
        if (dd >= r0) {
            const int jp = (dd - r0) >> 1;
            const float cs = rope_cs[jp][0], sn = rope_cs[jp][1];
            const float xa = x[i], ya = x[i + 1];
            x[i] = xa * cs + ya * sn;
            x[i + 1] = -xa * sn + ya * cs;
        }
    }
    store_out4(p.out, (static_cast<size_t>(qr) * kH + h) * kD + d, x, p.out_bf16);
}

// ---------------------------------------------------------------- generic

struct AttnG {
    int B, Tq, H, D, N, K, S, W, qdt, kvdt, swadt;
    int dense_m;            // > 0: dense mode (K = N, entry j < visible count is record j)
    const int32_t* n_rec;
    const void* q;
    const void* kv;
    const float* kv_scale;
    const int32_t* idx;
    const void* swa;
    const float* swa_scale;
    const int64_t* q_pos;
    const float* sink;
    float sm;
    int rope_dims;
    float rope_base;
    void* out;
    int out_bf16;
};

__device__ float block_reduce(float v, float* red, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        const float u = shfl_xor_f(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

__global__ __launch_bounds__(256) void attn_generic_kernel(AttnG p) {
    extern __shared__ float gsh[];  // q[D], ctx[D], z[E]
    __shared__ float red[4];
    const int qr = blockIdx.x;
    const int h = blockIdx.y;
    const int b = qr / p.Tq;
    const int64_t t = p.q_pos[qr];
    const int D = p.D;
    float* sq = gsh;
    float* ctx = gsh + D;
    float* z = gsh + 2 * D;
    const size_t qoff = (static_cast<size_t>(qr) * p.H + h) * D;
    for (int i = threadIdx.x; i < D; i += blockDim.x) sq[i] = load_elem(p.q, qoff + i, p.qdt);
    const int nwin = t < 0 ? 0 : static_cast<int>(t + 1 < p.W ? t + 1 : p.W);
    const int64_t win0 = t - nwin + 1;
    const int E = p.K + nwin;
    __syncthreads();
    int nvis = 0;  // dense mode: visible records
    if (p.dense_m) {
        const int nrec = p.n_rec ? min(p.n_rec[b], p.N) : p.N;
        const int64_t v = t < 0 ? 0 : (t + 1) / p.dense_m;
        nvis = static_cast<int>(v < nrec ? v : nrec);
    }
    auto entry = [&](int j, const void*& base, size_t& off, float& sc, int& dt) -> bool {
        if (j < p.K) {
            const int rec = p.dense_m ? (j < nvis ? j : -1) : p.idx[static_cast<size_t>(qr) * p.K + j];
            if (rec < 0 || rec >= p.N) return false;
            const size_t r = static_cast<size_t>(b) * p.N + rec;
            base = p.kv; off = r * D; dt = p.kvdt;
            sc = p.kvdt == DT_E4M3 ? p.kv_scale[r] : 1.f;
            return true;
        }
        const int64_t pos = win0 + (j - p.K);
        const size_t r = static_cast<size_t>(b) * p.S + static_cast<size_t>(pos % p.S);
        base = p.swa; off = r * D; dt = p.swadt;
        sc = p.swadt == DT_E4M3 ? p.swa_scale[r] : 1.f;
        return true;
    };
    float lmax = -__builtin_huge_valf();
    for (int j = threadIdx.x; j < E; j += blockDim.x) {
        const void* base; size_t off; float sc; int dt;
        float zz = -__builtin_huge_valf();
        if (entry(j, base, off, sc, dt)) {
            float dot = 0.f;
            for (int i = 0; i < D; ++i) dot = fmaf(sq[i], load_elem(base, off + i, dt), dot);
            zz = dot * sc * p.sm;
        }
        z[j] = zz;
        lmax = fmaxf(lmax, zz);
    }
    const float sk = p.sink[h];
    const float a = fmaxf(block_reduce(lmax, red, true), sk);
    float lsum = 0.f;
    for (int j = threadIdx.x; j < E; j += blockDim.x) {
        const float e = (z[j] == -__builtin_huge_valf() || a == -__builtin_huge_valf()) ? 0.f : __expf(z[j] - a);
        z[j] = e;
        lsum += e;
    }
    float den = block_reduce(lsum, red, false);
    if (a != -__builtin_huge_valf() && sk != -__builtin_huge_valf()) den += __expf(sk - a);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        float s = 0.f;
        for (int j = 0; j < E; ++j) {
            if (z[j] == 0.f) continue;
            const void* base; size_t off; float sc; int dt;
            entry(j, base, off, sc, dt);
            s = fmaf(z[j] * sc, load_elem(base, off + i, dt), s);
        }
        ctx[i] = s * inv;
    }
    __syncthreads();
    const int rd = p.rope_dims, r0 = D - rd;
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        float o = ctx[i];
        if (i >= r0) {
            const int jp = (i - r0) >> 1;
            float cs, sn;
            rope_angle(t, jp, rd, p.rope_base, cs, sn);
            const float x = ctx[r0 + 2 * jp], y = ctx[r0 + 2 * jp + 1];
            o = ((i - r0) & 1) ? (-x * sn + y * cs) : (x * cs + y * sn);
        }
        if (p.out_bf16)
            static_cast<uint16_t*>(p.out)[qoff + i] = static_cast<uint16_t>(f32_to_bf16_rne(o));
        else
            static_cast<float*>(p.out)[qoff + i] = o;
    }
}

int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// MI355X compute units.  The layout and split choices below depend only on
// the shapes (so the workspace size does too); the grid uses the count the
// device reports.
constexpr int kCUs = 256;

// Decode layout (one 16-head group per item) when the queries' four head
// groups fit on the chip at once and a query's list fits one item's entry
// table (emax entries); otherwise 64 heads per item.  Long lists (dense
// mode) thus take 64-head items split across the chip: their tiles are
// computed once for all heads (the decode layout's four head groups would
// each copy and multiply every tile), at twice the decode layout's matrix
// work per wave and tile.
bool decode_layout(int Q, int emax) { return 4 * Q <= kCUs && emax <= kMaxEnt; }

// Bytes of split partials (fp32 O, then (max, sum) per head) for Q
// queries in ns splits.
size_t part_bytes(int Q, int ns) {
    if (ns <= 1) return 0;
    const size_t o = static_cast<size_t>(Q) * ns * kH * kD * sizeof(float);
    const size_t ml = static_cast<size_t>(Q) * ns * kH * 2 * sizeof(float);
    return ((o + 255) & ~static_cast<size_t>(255)) + ((ml + 255) & ~static_cast<size_t>(255));
}

// Entry splits per query.  Every split writes an fp32 partial O of its
// heads that attn_combine_kernel reads back, so splits are used only while
// the items would otherwise leave most compute units idle, and wherever a
// split would hold more entries than the entry table (kMaxEnt):
//  * decode layout: at most 256 items in all, one per compute unit (four
//    per split; measured against 128 and 512: C4's 16 queries in four
//    splits run 8% faster than in two, and 21% faster than in eight), so at
//    most 64 partials (8 MiB);
//  * 64-head items of lists longer than the entry table (dense mode): one
//    item per compute unit as well (C6's 8 queries in 29 splits: 37 us;
//    half as many splits: 42 us);
//  * other 64-head items are not split for parallelism: the partials'
//    round trip (128 KiB per split and query, written and read back) costs
//    as much as it gains (80 queries in three splits: 37.3 against 35.7 us
//    unsplit).
// The splits taken only for parallelism are reduced until the partials fit
// part_cap bytes.  K is the longest list of records (dense mode: N).
int choose_splits(int Q, int K, int W, int& per, size_t part_cap) {
    const int emax = K + W;
    const int ntiles = (emax + kTile - 1) / kTile;
    const int need = (ntiles * kTile + kMaxEnt - 1) / kMaxEnt;  // splits the entry table needs
    int ns = need;
    // rounded down: never more items than compute units
    const int want = decode_layout(Q, emax) ? kCUs / (4 * Q) : (emax > kMaxEnt ? kCUs / Q : 0);
    if (want > ns) ns = want;
    if (ns > ntiles) ns = ntiles;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    auto fit = [&](int n) {  // n splits as equal tile counts
        const int tps = (ntiles + n - 1) / n;
        return (ntiles + tps - 1) / tps;
    };
    ns = fit(ns);
    while (ns > need && ns > 1 && part_bytes(Q, ns) > part_cap) ns = fit(ns - 1);
    const int tps = (ntiles + ns - 1) / ns;  // tiles per split
    per = tps * kTile;
    return ns;
}

}  // namespace

// Device-resident scratch of the allocation-free attention entry point: the
// split partials (fp32 O, then (max, sum) per head) of one call.  Each GPU
// holds its own copy for the life of the process; calls on one GPU share
// it, so they must not overlap.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per
// device (sparse_attn_scratch below), and only that address is ever passed
// to a kernel.
constexpr size_t kScratchBytes = size_t(6) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t sparse_attn_scratch_bytes() { return kScratchBytes; }

void* sparse_attn_scratch(int& err) {
    static std::mutex mu;
    static void* ptr[kMaxDevices];
    int dev = 0;
    err = static_cast<int>(hipGetDevice(&dev));
    if (err) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        err = static_cast<int>(hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        err = static_cast<int>(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (err) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

bool sparse_attn_mfma_ok(const AttnArgs& a) {
    const int klist = a.dense_m ? a.N : a.K;  // longest list of records
    return a.H == kH && a.D == kD && a.q_dtype == DT_BF16 && (a.dense_m ? 1 : a.K <= kMaxKList) &&
           a.W <= kMaxWin && static_cast<long long>(klist) + a.W <= static_cast<long long>(kMaxSplits) * kMaxEnt &&
           (((a.kv_dtype == DT_BF16 || a.kv_dtype == DT_E4M3) && a.swa_dtype == a.kv_dtype) ||
            (a.kv_dtype == DT_FP4 && a.swa_dtype == DT_E4M3)) &&
           a.rope_dims <= kD;
}

size_t dense_attn_ws_bytes(int B, int Tq, int H, int D, int N, int W) {
    if (H != kH || D != kD) return 0;
    int per;
    const int Q = B * Tq;
    return part_bytes(Q, choose_splits(Q, N, W, per, SIZE_MAX));
}

size_t sparse_attn_ws_bytes(int B, int Tq, int H, int D, int K, int W, size_t part_cap) {
    if (H != kH || D != kD) return 0;
    int per;
    const int Q = B * Tq;
    return part_bytes(Q, choose_splits(Q, K, W, per, part_cap));
}

int launch_sparse_attn(const AttnArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const float sm = a.sm_scale != 0.f ? a.sm_scale : 1.f / sqrtf(static_cast<float>(a.D));
    const int Q = a.B * a.Tq;
    if (sparse_attn_mfma_ok(a)) {
        AttnP p;
        p.B = a.B; p.Tq = a.Tq; p.N = a.N; p.K = a.K; p.S = a.S; p.W = a.W;
        p.q = static_cast<const uint16_t*>(a.q);
        p.kv = static_cast<const uint8_t*>(a.kv);
        p.kv_scale = a.kv_scale;
        p.idx = a.idx;
        p.swa = static_cast<const uint8_t*>(a.swa);
        p.swa_scale = a.swa_scale;
        p.q_pos = a.q_pos;
        p.sink = a.sink;
        p.sm = sm;
        p.rope_dims = a.rope_dims;
        p.rope_base = a.rope_base;
        p.out = a.out;
        p.out_bf16 = a.out_dtype == DT_BF16;
        const bool dec = decode_layout(Q, (a.dense_m ? a.N : a.K) + a.W);
        p.dense_m = a.dense_m;
        p.n_rec = a.n_rec;
        p.nsplit = choose_splits(Q, a.dense_m ? a.N : a.K, a.W, p.per_split, a.part_cap);
        p.part_o = nullptr;
        p.part_ml = nullptr;
        if (p.nsplit > 1) {
            const size_t o = static_cast<size_t>(Q) * p.nsplit * kH * kD * sizeof(float);
            p.part_o = static_cast<float*>(a.ws);
            p.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(a.ws) +
                                                 ((o + 255) & ~static_cast<size_t>(255)));
        }
        // persistent: one workgroup per compute unit (the LDS footprint
        // allows one), each walking its share of the work items.  Decode
        // items come in blocks of 32 (8 XCDs x 4 head groups) and the grid
        // is a multiple of 8, so every workgroup keeps to one XCD's items.
        const int qs = Q * p.nsplit;
        p.n_items = dec ? 32 * ((qs + 7) / 8) : qs;
        const int cus = dec ? (num_cus() / 8) * 8 : num_cus();
        const dim3 grid(p.n_items < cus ? p.n_items : cus);
        if (dec) {
            const int e = launch_attn_decode(p, grid.x, a.kv_dtype, st);
            if (e) return e;
        } else {
            if (a.kv_dtype == DT_BF16)
                hipLaunchKernelGGL((attn_mfma_kernel<DT_BF16, 64>), grid, dim3(kThreads), 0, st, p);
            else if (a.kv_dtype == DT_E4M3)
                hipLaunchKernelGGL((attn_mfma_kernel<DT_E4M3, 64>), grid, dim3(kThreads), 0, st, p);
            else
                hipLaunchKernelGGL((attn_mfma_kernel<DT_FP4, 64>), grid, dim3(kThreads), 0, st, p);
        }
        int e = static_cast<int>(hipGetLastError());
        if (e || p.nsplit == 1) return e;
        hipLaunchKernelGGL(attn_combine_kernel, dim3(Q, kH / 2), dim3(256), 0, st, p);
        return static_cast<int>(hipGetLastError());
    }
    AttnG p;
    p.B = a.B; p.Tq = a.Tq; p.H = a.H; p.D = a.D; p.N = a.N; p.K = a.K; p.S = a.S; p.W = a.W;
    p.qdt = a.q_dtype; p.kvdt = a.kv_dtype; p.swadt = a.swa_dtype;
    p.q = a.q; p.kv = a.kv; p.kv_scale = a.kv_scale; p.idx = a.idx; p.swa = a.swa;
    p.swa_scale = a.swa_scale; p.q_pos = a.q_pos; p.sink = a.sink; p.sm = sm;
    p.rope_dims = a.rope_dims; p.rope_base = a.rope_base; p.out = a.out;
    p.out_bf16 = a.out_dtype == DT_BF16;
    p.dense_m = a.dense_m; p.n_rec = a.n_rec;
    if (a.dense_m) p.K = a.N;  // entry j < N is record j when visible
    const size_t lds = (2 * static_cast<size_t>(a.D) + p.K + a.W) * sizeof(float);
    hipLaunchKernelGGL(attn_generic_kernel, dim3(Q, a.H), dim3(256), lds, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
