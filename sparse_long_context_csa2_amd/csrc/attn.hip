// Sparse shared-latent attention with a sliding window and a sink.
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
//  * one workgroup = 4 waves per (query, split of the entry list); wave w
//    owns heads 16w .. 16w+15;
//  * the valid selected records are first compacted into an LDS list, so
//    -1 padding costs nothing;
//  * entries are processed in tiles of 32 rows (32 KiB of bf16).  A tile is
//    fetched with fully used 256-byte segments into registers one tile
//    ahead, then written to LDS twice: row-major (padded to 1040 B per row)
//    for S^T = X Q^T, and transposed in a group-major, XOR-swizzled layout
//    for O^T += X^T P^T.  Both the transposing writes and the MFMA operand
//    reads then touch each 16-byte bank slot exactly as often as the data
//    volume requires;
//  * S^T is computed with 16x16x32 bf16 MFMAs (entries on M, heads on N),
//    so each lane holds 8 logits of ONE head: the online-softmax max and
//    sum need only two cross-lane steps, and those 8 probabilities are
//    exactly the B operand of the P.V MFMA (heads on N again), so P never
//    leaves registers.  P is split into bf16 hi + lo parts (two MFMAs) so
//    that rounding P to bf16 costs no accuracy;
//  * e4m3 rows are converted exactly to bf16 while staging; their per-row
//    scale multiplies the logit and the probability instead;
//  * with one split the workgroup finishes (sink, normalisation, inverse
//    RoPE) itself; otherwise it writes (max, sum, unnormalised O) and
//    attn_combine_kernel merges the splits.
// attn_generic_kernel: any head count and dim (one workgroup per query and
// head, fp32 throughout); used for small shapes such as the toy.
#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kH = 64;
constexpr int kD = 512;
constexpr int kTile = 32;
constexpr int kXrPitch = kD * 2 + 16;  // bytes per row-major LDS row
constexpr int kMaxKList = 2048;
constexpr int kMaxRope = kD / 2;
constexpr int kMaxSplits = 32;

struct AttnP {
    int B, Tq, N, K, S, W, nsplit, per_split;
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
    float* out;               // [B][Tq][64][512]
    float* part_o;            // [Q][nsplit][64][512]
    float* part_ml;           // [Q][nsplit][64][2]
};

struct __align__(16) AttnShared {
    uint8_t xr[kTile * kXrPitch];         // row-major tile
    uint8_t xt[4 * kD * 16];              // [entry group][d (swizzled)][8 entries]
    int32_t list[kMaxKList];              // compacted valid record ids
    float esc[kTile];                     // per-entry scale
    int evalid[kTile];
    float rope_cs[kMaxRope][2];
    int wave_cnt[4];
    int nsel;
};

// Physical d slot of (entry group grp, channel d) in the transposed tile:
// an XOR inside each aligned block of 16 channels.
__device__ __forceinline__ int xt_slot(int grp, int d) {
    return grp * kD + ((d & ~15) | ((d ^ (d >> 4) ^ (grp << 2)) & 15));
}

template <int KVDT>
__device__ __forceinline__ u32x4 load_row_chunk(const uint8_t* row, int c, bool ok) {
    if (!ok) return u32x4{0, 0, 0, 0};
    if (KVDT == DT_BF16) return *reinterpret_cast<const u32x4*>(row + 16 * c);
    const u32x2 v = *reinterpret_cast<const u32x2*>(row + 8 * c);
    return e4m3x8_to_bf16x8(v);
}

__device__ __forceinline__ uint32_t pick_half(uint32_t a, uint32_t b, int k) {
    // element k of two bf16x8 dwords -> packed pair (a's, b's)
    return (k & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
}

template <int KVDT>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnP p) {
    __shared__ AttnShared sh;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int split = blockIdx.x;
    const int qr = blockIdx.y;
    const int b = qr / p.Tq;
    const int64_t t = p.q_pos[qr];
    constexpr int kRowBytes = (KVDT == DT_BF16) ? kD * 2 : kD;

    // ---- compact the valid selected records (in order) ----
    const int32_t* irow = p.idx + static_cast<size_t>(qr) * p.K;
    int nsel = 0;
    for (int base = 0; base < p.K; base += 256) {
        const int j = base + threadIdx.x;
        int rec = -1;
        if (j < p.K) rec = irow[j];
        const bool ok = rec >= 0 && rec < p.N;
        const unsigned long long bal = __ballot(ok);
        if (lane == 0) sh.wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = nsel;
        for (int i = 0; i < wave; ++i) off += sh.wave_cnt[i];
        if (ok) sh.list[off + __popcll(bal & ((1ull << lane) - 1ull))] = rec;
        for (int i = 0; i < 4; ++i) nsel += sh.wave_cnt[i];
        __syncthreads();
    }
    const int nwin = t < 0 ? 0 : static_cast<int>(t + 1 < p.W ? t + 1 : p.W);
    const int64_t win0 = t - nwin + 1;
    const int E = nsel + nwin;
    const int j0 = split * p.per_split;
    const int j1 = min(E, j0 + p.per_split);

    // rotary angles of this query (double precision: t reaches 2^20)
    const int rd = p.rope_dims;
    for (int i = threadIdx.x; i < rd / 2; i += 256) {
        const double inv = pow(static_cast<double>(p.rope_base), -2.0 * i / rd);
        double s, c;
        sincos(static_cast<double>(t) * inv, &s, &c);
        sh.rope_cs[i][0] = static_cast<float>(c);
        sh.rope_cs[i][1] = static_cast<float>(s);
    }

    // ---- query fragments: head 16*wave + l16, 16 k-steps of 8 channels ----
    const int h = 16 * wave + l16;
    bf16x8 qf[16];
    {
        const uint16_t* qh = p.q + (static_cast<size_t>(qr) * kH + h) * kD;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
            qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 8 * (g + 4 * ks)));
    }

    // ---- staging geometry: rows 8*g .. 8*g+7 of the tile, chunk c ----
    const int c = 16 * wave + l16;  // 8-channel chunk owned by this lane
    auto row_ptr = [&](int e, bool& ok, float& scale) -> const uint8_t* {
        ok = e < j1;
        scale = 0.f;
        if (!ok) return nullptr;
        if (e < nsel) {
            const int rec = sh.list[e];
            const size_t r = static_cast<size_t>(b) * p.N + rec;
            scale = KVDT == DT_E4M3 ? p.kv_scale[r] : 1.f;
            return p.kv + r * kRowBytes;
        }
        const int64_t pos = win0 + (e - nsel);
        const size_t r = static_cast<size_t>(b) * p.S + static_cast<size_t>(pos % p.S);
        scale = KVDT == DT_E4M3 ? p.swa_scale[r] : 1.f;
        return p.swa + r * kRowBytes;
    };

    u32x4 stg[8];
    auto fetch = [&](int tb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bool ok;
            float sc;
            const uint8_t* rp = row_ptr(tb + 8 * g + i, ok, sc);
            stg[i] = load_row_chunk<KVDT>(rp, c, ok);
        }
    };

    float m_run = -__builtin_huge_valf();
    float l_run = 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // list, rope table visible
    if (j0 < j1) fetch(j0);

    for (int tb = j0; tb < j1; tb += kTile) {
        __syncthreads();  // previous tile fully consumed
        // ---- write the staged tile: row-major and transposed ----
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4*>(sh.xr + (8 * g + i) * kXrPitch + 16 * c) = stg[i];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            u32x4 v;
#pragma unroll
            for (int m = 0; m < 4; ++m) v[m] = pick_half(stg[2 * m][k >> 1], stg[2 * m + 1][k >> 1], k);
            *reinterpret_cast<u32x4*>(sh.xt + 16 * xt_slot(g, 8 * c + k)) = v;
        }
        if (threadIdx.x < kTile) {
            bool ok;
            float sc;
            row_ptr(tb + threadIdx.x, ok, sc);
            sh.esc[threadIdx.x] = sc;
            sh.evalid[threadIdx.x] = ok ? 1 : 0;
        }
        // prefetch the next tile while this one is computed
        if (tb + kTile < j1) fetch(tb + kTile);
        __syncthreads();

        // ---- S^T = X Q^T : entries 16*mt + 4g + v, head h ----
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int ch = g + 4 * ks;
            const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4*>(sh.xr + l16 * kXrPitch + 16 * ch));
            const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4*>(sh.xr + (16 + l16) * kXrPitch + 16 * ch));
            s0 = mfma16x16x32(a0, qf[ks], s0);
            s1 = mfma16x16x32(a1, qf[ks], s1);
        }
        // ---- online softmax over this tile ----
        float z[8];
        float tmax = -__builtin_huge_valf();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int e0 = 4 * g + v, e1 = 16 + 4 * g + v;
            z[v] = sh.evalid[e0] ? s0[v] * p.sm * sh.esc[e0] : -__builtin_huge_valf();
            z[4 + v] = sh.evalid[e1] ? s1[v] * p.sm * sh.esc[e1] : -__builtin_huge_valf();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_new == -__builtin_huge_valf()) ? 1.f : __expf(m_run - m_new);
        float psum = 0.f;
        uint32_t phi[4], plo[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            float pp[2], pw[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ii = i + u;
                const int e = (ii < 4) ? 4 * g + ii : 16 + 4 * g + (ii - 4);
                pp[u] = (z[ii] == -__builtin_huge_valf()) ? 0.f : __expf(z[ii] - m_new);
                pw[u] = pp[u] * sh.esc[e];
                psum += pp[u];
            }
            const uint32_t hi = pack_bf16x2(pw[0], pw[1]);
            const float r0 = pw[0] - __uint_as_float(hi << 16);
            const float r1 = pw[1] - __uint_as_float(hi & 0xFFFF0000u);
            phi[i >> 1] = hi;
            plo[i >> 1] = pack_bf16x2(r0, r1);
        }
        psum += shfl_xor_f(psum, 16);
        psum += shfl_xor_f(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const bf16x8 bhi = as_bf16x8(u32x4{phi[0], phi[1], phi[2], phi[3]});
        const bf16x8 blo = as_bf16x8(u32x4{plo[0], plo[1], plo[2], plo[3]});

        // ---- O^T += X^T P^T : channels 16*dt + 4g + v, head h ----
        const int half = 8 * (g & 1);
        const int ga = g >> 1, gb = 2 + (g >> 1);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            const int d = 16 * dt + l16;
            const u32x2 xa = *reinterpret_cast<const u32x2*>(sh.xt + 16 * xt_slot(ga, d) + half);
            const u32x2 xb = *reinterpret_cast<const u32x2*>(sh.xt + 16 * xt_slot(gb, d) + half);
            const bf16x8 a = as_bf16x8(u32x4{xa[0], xa[1], xb[0], xb[1]});
            f32x4 o = acc[dt] * alpha;
            o = mfma16x16x32(a, bhi, o);
            acc[dt] = mfma16x16x32(a, blo, o);
        }
    }

    // ---- finish ----
    if (p.nsplit == 1) {
        const float sk = p.sink[h];
        const float a = fmaxf(m_run, sk);
        float f = 0.f;
        if (a != -__builtin_huge_valf()) {
            const float em = (m_run == -__builtin_huge_valf()) ? 0.f : __expf(m_run - a);
            const float es = (sk == -__builtin_huge_valf()) ? 0.f : __expf(sk - a);
            const float den = l_run * em + es;
            f = den > 0.f ? em / den : 0.f;
        }
        float* orow = p.out + (static_cast<size_t>(qr) * kH + h) * kD;
        const int r0 = kD - rd;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            const int d = 16 * dt + 4 * g;
            f32x4 o = acc[dt] * f;
            if (d + 3 >= r0) {
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    const int dd = d + v;
                    if (dd >= r0) {
                        const int jp = (dd - r0) >> 1;
                        const float cs = sh.rope_cs[jp][0], sn = sh.rope_cs[jp][1];
                        const float x = o[v], y = o[v + 1];
                        o[v] = x * cs + y * sn;
                        o[v + 1] = -x * sn + y * cs;
                    }
                }
            }
            *reinterpret_cast<f32x4*>(orow + d) = o;
        }
    } else {
        const size_t slot = (static_cast<size_t>(qr) * p.nsplit + split) * kH + h;
        float* po = p.part_o + slot * kD;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = acc[dt];
        if (g == 0) {
            p.part_ml[2 * slot] = m_run;
            p.part_ml[2 * slot + 1] = l_run;
        }
    }
}

// Merges split partials: one workgroup per query, each thread one channel
// pair of every head.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnP p) {
    __shared__ float rope_cs[kMaxRope][2];
    __shared__ float wts[kH][kMaxSplits + 1];
    const int qr = blockIdx.x;
    const int64_t t = p.q_pos[qr];
    const int rd = p.rope_dims;
    for (int i = threadIdx.x; i < rd / 2; i += 256) {
        const double inv = pow(static_cast<double>(p.rope_base), -2.0 * i / rd);
        double s, c;
        sincos(static_cast<double>(t) * inv, &s, &c);
        rope_cs[i][0] = static_cast<float>(c);
        rope_cs[i][1] = static_cast<float>(s);
    }
    const int ns = p.nsplit;
    // per-head split weights: w_s = e^{m_s - a} / den
    if (threadIdx.x < kH) {
        const int h = threadIdx.x;
        const float* ml = p.part_ml + (static_cast<size_t>(qr) * ns * kH + h) * 2;
        float a = p.sink[h];
        for (int s = 0; s < ns; ++s) a = fmaxf(a, ml[static_cast<size_t>(s) * kH * 2]);
        float den = 0.f;
        if (a != -__builtin_huge_valf()) {
            den = (p.sink[h] == -__builtin_huge_valf()) ? 0.f : __expf(p.sink[h] - a);
            for (int s = 0; s < ns; ++s) {
                const float m = ml[static_cast<size_t>(s) * kH * 2];
                if (m != -__builtin_huge_valf()) den += ml[static_cast<size_t>(s) * kH * 2 + 1] * __expf(m - a);
            }
        }
        for (int s = 0; s < ns; ++s) {
            const float m = ml[static_cast<size_t>(s) * kH * 2];
            wts[h][s] = (den > 0.f && m != -__builtin_huge_valf()) ? __expf(m - a) / den : 0.f;
        }
    }
    __syncthreads();
    const int d = 2 * threadIdx.x;
    const int r0 = kD - rd;
    for (int h = 0; h < kH; ++h) {
        float x = 0.f, y = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float* po = p.part_o + ((static_cast<size_t>(qr) * ns + s) * kH + h) * kD;
            const float2 v = *reinterpret_cast<const float2*>(po + d);
            x += wts[h][s] * v.x;
            y += wts[h][s] * v.y;
        }
        if (d >= r0) {
            const int jp = (d - r0) >> 1;
            const float cs = rope_cs[jp][0], sn = rope_cs[jp][1];
            const float nx = x * cs + y * sn;
            y = -x * sn + y * cs;
            x = nx;
        }
        *reinterpret_cast<float2*>(p.out + (static_cast<size_t>(qr) * kH + h) * kD + d) = make_float2(x, y);
    }
}

// ---------------------------------------------------------------- generic

struct AttnG {
    int B, Tq, H, D, N, K, S, W, qdt, kvdt, swadt;
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
    float* out;
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
    auto entry = [&](int j, const void*& base, size_t& off, float& sc, int& dt) -> bool {
        if (j < p.K) {
            const int rec = p.idx[static_cast<size_t>(qr) * p.K + j];
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
    float* orow = p.out + qoff;
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        if (i < r0) {
            orow[i] = ctx[i];
        } else {
            const int jp = (i - r0) >> 1;
            const double th = static_cast<double>(t) * pow(static_cast<double>(p.rope_base), -2.0 * jp / rd);
            double s, cth;
            sincos(th, &s, &cth);
            const float cs = static_cast<float>(cth), sn = static_cast<float>(s);
            const float x = ctx[r0 + 2 * jp], y = ctx[r0 + 2 * jp + 1];
            orow[i] = ((i - r0) & 1) ? (-x * sn + y * cs) : (x * cs + y * sn);
        }
    }
}

int choose_splits(int Q, int K, int W, int& per) {
    const int emax = K + W;
    const int ntiles = (emax + kTile - 1) / kTile;
    int ns = (256 + Q - 1) / Q;
    if (ns > ntiles) ns = ntiles;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    const int tps = (ntiles + ns - 1) / ns;  // tiles per split
    ns = (ntiles + tps - 1) / tps;
    per = tps * kTile;
    return ns;
}

}  // namespace

bool sparse_attn_mfma_ok(const AttnArgs& a) {
    return a.H == kH && a.D == kD && a.q_dtype == DT_BF16 && a.K <= kMaxKList &&
           (a.kv_dtype == DT_BF16 || a.kv_dtype == DT_E4M3) && a.swa_dtype == a.kv_dtype &&
           a.rope_dims <= kD;
}

size_t sparse_attn_ws_bytes(int B, int Tq, int H, int D, int K, int W) {
    if (H != kH || D != kD) return 0;
    int per;
    const int Q = B * Tq;
    const int ns = choose_splits(Q, K, W, per);
    if (ns == 1) return 0;
    const size_t o = static_cast<size_t>(Q) * ns * kH * kD * sizeof(float);
    const size_t ml = static_cast<size_t>(Q) * ns * kH * 2 * sizeof(float);
    return ((o + 255) & ~static_cast<size_t>(255)) + ((ml + 255) & ~static_cast<size_t>(255));
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
        p.nsplit = choose_splits(Q, a.K, a.W, p.per_split);
        p.part_o = nullptr;
        p.part_ml = nullptr;
        if (p.nsplit > 1) {
            const size_t o = static_cast<size_t>(Q) * p.nsplit * kH * kD * sizeof(float);
            p.part_o = static_cast<float*>(a.ws);
            p.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(a.ws) +
                                                 ((o + 255) & ~static_cast<size_t>(255)));
        }
        dim3 grid(p.nsplit, Q);
        if (a.kv_dtype == DT_BF16)
            hipLaunchKernelGGL(attn_mfma_kernel<DT_BF16>, grid, dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL(attn_mfma_kernel<DT_E4M3>, grid, dim3(256), 0, st, p);
        int e = static_cast<int>(hipGetLastError());
        if (e || p.nsplit == 1) return e;
        hipLaunchKernelGGL(attn_combine_kernel, dim3(Q), dim3(256), 0, st, p);
        return static_cast<int>(hipGetLastError());
    }
    AttnG p;
    p.B = a.B; p.Tq = a.Tq; p.H = a.H; p.D = a.D; p.N = a.N; p.K = a.K; p.S = a.S; p.W = a.W;
    p.qdt = a.q_dtype; p.kvdt = a.kv_dtype; p.swadt = a.swa_dtype;
    p.q = a.q; p.kv = a.kv; p.kv_scale = a.kv_scale; p.idx = a.idx; p.swa = a.swa;
    p.swa_scale = a.swa_scale; p.q_pos = a.q_pos; p.sink = a.sink; p.sm = sm;
    p.rope_dims = a.rope_dims; p.rope_base = a.rope_base; p.out = a.out;
    const size_t lds = (2 * static_cast<size_t>(a.D) + a.K + a.W) * sizeof(float);
    hipLaunchKernelGGL(attn_generic_kernel, dim3(Q, a.H), dim3(256), lds, st, p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
