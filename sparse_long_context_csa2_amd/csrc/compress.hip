// Record construction: the CSA2 compressor and the cache write.
//
// Record s of a sequence pools its block of m consecutive token rows
// (groups do not overlap, "DeepSeek-V4.1-Flash explained", section 2): each
// channel is a softmax-weighted sum over the block's tokens with weights
// from that channel's gate logits ("Create DeepSeek from scratch", "How
// CSA2 compresses, shares, and selects attention memory": learned,
// channel-wise softmax gates; at ratio 1 no pooling, a normalized
// projection).  The pooled row is RMS-normalized with a gain, its last r
// channels are rotated to the position of the block's last token, and only
// then is it quantized into the cache ("Quantize after RoPE", the FP4
// lesson of the same course).  Indexer keys are derived from the stored
// (dequantized) row: k = x_stored W_ik ("explained", section 2: CSA2
// derives indexer keys from main KV), then quantized into the key cache.
//
// Two kernels on the caller's stream:
//
// pool_kernel streams the token rows (the HBM-bound part).  A wave builds
// one record at a time, four per wave: lane l owns channels CPL*l ..
// CPL*l+CPL-1 and loads them with 16-byte loads, four tokens at once; the
// softmax runs over each group of four tokens with one exponential per
// token and channel; the row's mean square is a wave reduction; the
// cosines and sines of all the workgroup's records are tabulated in LDS at
// the start (angle in double precision, every thread a few), so a rotation
// is a table read by the lanes that own the pair; the quantized row is
// written with one packed store per lane.  Each record's first token group
// is loaded while the previous record is finished.
//
// keys_kernel forms the keys as a matrix product on the matrix cores: 64
// records (rows, read back from the cache just written, dequantized
// exactly to bf16) times W_ik.  W_ik is split into bf16 high and low parts
// (w = hi + lo to 2^-16 relative), float32 record rows likewise, so the
// bf16 products accumulate in float32 to about float32 accuracy.  W_ik is
// staged transposed in LDS 64 input channels at a time; the keys go
// through LDS once more to be quantized, four threads per record.
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kPoolWaves = 4;
constexpr int kPoolRecPerWave = 4;
constexpr int kPoolRecPerWG = kPoolWaves * kPoolRecPerWave;
constexpr int kMaxRopePairs = 512;  // rope_dims <= D <= 1024
constexpr int kKeyRows = 64;        // records per keys workgroup (4 waves x 16 rows)
constexpr int kWPitch = 72;         // bf16 per staged W_ik^T row: 64 channels + 8 (bank spread)

struct CompP {
    int B, T, D, m, Di, N_out;
    const uint8_t* c;      // [B][T][D] candidate latents (f32 or bf16)
    const uint8_t* z;      // [B][T][D] gate logits
    int in_dt;
    const int64_t* t0;     // [B] absolute position of token row 0
    const float* gain;     // [D]
    float eps;
    int rope_dims;
    float rope_base;
    const uint8_t* w;      // [D][Di] W_ik (f32 or bf16)
    int w_dt;
    uint8_t* kv;           // [B][N_out][kv row bytes]
    float* kv_scale;       // e4m3: [B][N_out]
    int kv_dt;
    uint8_t* k;            // [B][N_out][key row bytes]
    uint8_t* k_scale;      // e4m3: float [B][N_out]; MXFP4: E8M0 [B][N_out][Di/32]
    int k_dt;
};

// Nearest e4m3fn code of v (ties to even, saturating at +-448).  gfx950's
// conversion rounds to nearest even but turns magnitudes from 464 up into
// NaN, so the input is clamped to the largest finite value first; with
// that it agrees with a comparison encoder on every e4m3 midpoint, its
// float neighbours and the saturation range.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const float c = fminf(fmaxf(v, -448.f), 448.f);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Two e4m3 codes (a in the low byte).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.f), 448.f), fminf(fmaxf(b, -448.f), 448.f), 0,
                                           false) & 0xFFFFu;
}

// Nearest E2M1 codes of a, b (ties to even, saturating at 6; a in the low
// nibble) in byte `sel` of `old`: gfx950's conversion with unit scale,
// which matches a comparison encoder on every midpoint of the E2M1 levels,
// their float neighbours and the saturation range.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_encode2(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Reductions over aligned groups of N neighbouring lanes (N a power of
// two up to 64), with xor shuffles.
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v = fmaxf(v, shfl_xor_f(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return warp_sum(v); }

// ---------------------------------------------------------------- loads / stores

// CPL channels of one token row, raw (bf16 pairs or float32 words).
template <int CPL, bool BF>
struct RawCh {
    uint32_t w[BF ? CPL / 2 : CPL];
};

template <int CPL, bool BF>
__device__ __forceinline__ void load_raw(const uint8_t* base, size_t elem, RawCh<CPL, BF>& r) {
    constexpr int NW = BF ? CPL / 2 : CPL;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(base + elem * (BF ? 2 : 4));
    if constexpr (NW >= 4) {
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const u32x4 v = reinterpret_cast<const u32x4*>(q)[k];
            r.w[4 * k] = v[0];
            r.w[4 * k + 1] = v[1];
            r.w[4 * k + 2] = v[2];
            r.w[4 * k + 3] = v[3];
        }
    } else if constexpr (NW == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(q);
        r.w[0] = v[0];
        r.w[1] = v[1];
    } else {
        r.w[0] = q[0];
    }
}

template <int CPL, bool BF>
__device__ __forceinline__ float raw_at(const RawCh<CPL, BF>& r, int j) {
    if constexpr (BF) return __uint_as_float((j & 1) ? (r.w[j >> 1] & 0xFFFF0000u) : (r.w[j >> 1] << 16));
    else return __uint_as_float(r.w[j]);
}

// NB bytes (1, 2, 4, 8 or a multiple of 16; the packed words w) to an
// address aligned to min(NB, 16).
template <int NB>
__device__ __forceinline__ void st_bytes(uint8_t* dst, const uint32_t* w) {
    if constexpr (NB == 1) {
        *dst = static_cast<uint8_t>(w[0]);
    } else if constexpr (NB == 2) {
        *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(w[0]);
    } else if constexpr (NB == 4) {
        *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else if constexpr (NB == 8) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
        for (int k = 0; k < NB / 16; ++k)
            reinterpret_cast<u32x4*>(dst)[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    }
}

// ---------------------------------------------------------------- records

template <int CPL, bool BF, bool G4>
__global__ __launch_bounds__(kPoolWaves * 64) void pool_kernel(CompP p) {
    __shared__ double inv_sh[kMaxRopePairs];  // inverse frequencies
    extern __shared__ float2 rot_sh[];  // [kPoolRecPerWG][rope_dims / 2] cos, sin per record and pair
    constexpr int D = CPL * 64;
    constexpr int kG = G4 ? 4 : 1;  // tokens of a record's first group (m >= 4: four)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.y;
    const int n_rec = p.T / p.m;
    const int d0 = CPL * lane;
    auto rec_of = [&](int k) { return blockIdx.x * kPoolRecPerWG + k * kPoolWaves + wave; };
    auto row_of = [&](int s) {  // element of this lane's first channel in the record's first token row
        return (static_cast<size_t>(b) * p.T + static_cast<size_t>(min(s, n_rec - 1)) * p.m) * D + d0;
    };
    // A record's first token group is requested while the previous record
    // is normalized, rotated and stored (the first record's before the
    // set-up below).
    RawCh<CPL, BF> gc[kG], gz[kG];
    auto load_group = [&](size_t row0) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            load_raw(p.c, row0 + static_cast<size_t>(u) * D, gc[u]);
            load_raw(p.z, row0 + static_cast<size_t>(u) * D, gz[u]);
        }
    };
    const int64_t t0 = p.t0[b];
    const int npairs = p.rope_dims / 2;
    const int r0 = D - p.rope_dims;
    for (int j = tid; j < npairs; j += kPoolWaves * 64) inv_sh[j] = rope_inv_freq(j, p.rope_dims, p.rope_base);
    load_group(row_of(rec_of(0)));
    if (t0 < 0) return;  // nothing of this sequence is written (workgroup-uniform)
    const int64_t s0 = t0 / p.m;
    __syncthreads();
    // cosines and sines of the workgroup's records (record kr = k * kPoolWaves
    // + wave is rotated to position t0 + s m + m - 1), all threads at once
    for (int e = tid; e < kPoolRecPerWG * npairs; e += kPoolWaves * 64) {
        const int kr = e / npairs, j = e - kr * npairs;
        const int64_t pos = t0 + static_cast<int64_t>(blockIdx.x * kPoolRecPerWG + kr) * p.m + p.m - 1;
        float cs, sn;
        rope_cos_sin(pos, inv_sh[j], cs, sn);
        rot_sh[e] = make_float2(cs, sn);
    }
    __syncthreads();
    float gain[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) gain[j] = p.gain[d0 + j];

    for (int k = 0; k < kPoolRecPerWave; ++k) {
        const int s = rec_of(k);
        if (s >= n_rec || s0 + s >= p.N_out) break;  // wave-uniform; s grows with k
        // ---- channel-wise softmax pooling over the block's m tokens, four at a time
        float mx[CPL], sm[CPL], ac[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            mx[j] = -__builtin_huge_valf();
            sm[j] = 0.f;
            ac[j] = 0.f;
        }
        const size_t row0 = row_of(s);
        // weights 2^(z log2(e) - max log2(e)); the running sums are rescaled
        // when a later group of tokens raises the maximum
        constexpr float kL2E = 1.4426950408889634f;
        auto fold = [&](const auto& cr, const auto& zr, auto first_c) {
            constexpr int NT = sizeof(cr) / sizeof(cr[0]);
            constexpr bool kFirst = decltype(first_c)::value;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                float nm = mx[j];
#pragma unroll
                for (int u = 0; u < NT; ++u) nm = fmaxf(nm, raw_at(zr[u], j));
                const float nml = nm * kL2E;
                float sa = 0.f, aa = 0.f;
                if constexpr (!kFirst) {
                    const float sc = __builtin_amdgcn_exp2f(fmaf(mx[j], kL2E, -nml));
                    sa = sm[j] * sc;
                    aa = ac[j] * sc;
                }
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(raw_at(zr[u], j), kL2E, -nml));
                    sa += e;
                    aa = fmaf(e, raw_at(cr[u], j), aa);
                }
                mx[j] = nm;
                sm[j] = sa;
                ac[j] = aa;
            }
        };
        auto tokens = [&](int i0, auto nt_c) {
            constexpr int NT = decltype(nt_c)::value;
            RawCh<CPL, BF> cr[NT], zr[NT];
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                load_raw(p.c, row0 + static_cast<size_t>(i0 + u) * D, cr[u]);
                load_raw(p.z, row0 + static_cast<size_t>(i0 + u) * D, zr[u]);
            }
            fold(cr, zr, std::false_type{});
        };
        fold(gc, gz, std::true_type{});
        using One = std::integral_constant<int, 1>;
        int i0 = kG;
        if constexpr (G4) {  // further groups of four go through the same registers
            for (; i0 + 4 <= p.m; i0 += 4) {
                load_group(row0 + static_cast<size_t>(i0) * D);
                fold(gc, gz, std::false_type{});
            }
        }
        for (; i0 < p.m; ++i0) tokens(i0, One{});
        if (k + 1 < kPoolRecPerWave) load_group(row_of(rec_of(k + 1)));
        // ---- RMSNorm
        float x[CPL];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            x[j] = ac[j] * __builtin_amdgcn_rcpf(sm[j]);
            ss = fmaf(x[j], x[j], ss);
        }
        ss = wave_sum(ss);
        const float rn = rsqrtf(ss / static_cast<float>(D) + p.eps);
#pragma unroll
        for (int j = 0; j < CPL; ++j) x[j] *= rn * gain[j];
        // ---- RoPE at the block's last token (pairs never straddle lanes: CPL
        // and r0 are even)
        if (d0 + CPL > r0) {
            const float2* rot = rot_sh + (k * kPoolWaves + wave) * npairs;
#pragma unroll
            for (int j = 0; j < CPL; j += 2) {
                if (d0 + j >= r0) {
                    const float2 cs = rot[(d0 + j - r0) >> 1];
                    const float a = x[j], bb = x[j + 1];
                    x[j] = a * cs.x - bb * cs.y;
                    x[j + 1] = a * cs.y + bb * cs.x;
                }
            }
        }
        // ---- quantize and store the cache row
        const size_t ci = static_cast<size_t>(b) * p.N_out + static_cast<size_t>(s0 + s);
        if (p.kv_dt == DT_F32) {
            uint32_t w[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) w[j] = __float_as_uint(x[j]);
            st_bytes<4 * CPL>(p.kv + (ci * D + d0) * 4, w);
        } else if (p.kv_dt == DT_BF16) {
            uint32_t w[CPL / 2];
#pragma unroll
            for (int j = 0; j < CPL; j += 2) w[j / 2] = pack_bf16x2(x[j], x[j + 1]);
            st_bytes<2 * CPL>(p.kv + (ci * D + d0) * 2, w);
        } else if (p.kv_dt == DT_E4M3) {  // one scale per row: max|x| / 448
            float am = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) am = fmaxf(am, fabsf(x[j]));
            am = lanes_max<64>(am);
            const float scl = am / 448.f;
            const float inv = scl > 0.f ? 1.f / scl : 0.f;
            uint32_t w[(CPL + 3) / 4] = {};
#pragma unroll
            for (int j = 0; j < CPL; j += 2) w[j / 4] |= e4m3_encode2(x[j] * inv, x[j + 1] * inv) << (8 * (j % 4));
            st_bytes<CPL>(p.kv + ci * D + d0, w);
            if (lane == 0) p.kv_scale[ci] = scl;
        } else {  // FP4 row: E2M1 codes, one E4M3 scale (nearest max|x| / 6) per 16 channels
            uint8_t* row = p.kv + ci * (D / 2 + D / 16);
            uint32_t w[(CPL + 7) / 8] = {};
#pragma unroll
            for (int gi = 0; gi < (CPL >= 16 ? CPL / 16 : 1); ++gi) {
                constexpr int kGN = CPL >= 16 ? 16 : CPL;  // channels of the group in this lane
                float ga = 0.f;
#pragma unroll
                for (int j = 0; j < kGN; ++j) ga = fmaxf(ga, fabsf(x[kGN * gi + j]));
                if constexpr (CPL < 16) ga = lanes_max<16 / CPL>(ga);
                const uint32_t scode = e4m3_encode(ga / 6.f);
                const float scl = e4m3_to_f32(static_cast<uint8_t>(scode));
                const float inv = scl > 0.f ? 1.f / scl : 0.f;
#pragma unroll
                for (int j = 0; j < kGN; j += 8) {  // up to 8 codes per word, 2 per conversion
                    const int jj = kGN * gi + j;
                    uint32_t wd = 0u;
                    wd = e2m1_encode2<0>(wd, x[jj] * inv, x[jj + 1] * inv);
                    if constexpr (kGN >= 4) wd = e2m1_encode2<1>(wd, x[jj + 2] * inv, x[jj + 3] * inv);
                    if constexpr (kGN >= 8) {
                        wd = e2m1_encode2<2>(wd, x[jj + 4] * inv, x[jj + 5] * inv);
                        wd = e2m1_encode2<3>(wd, x[jj + 6] * inv, x[jj + 7] * inv);
                    }
                    w[jj / 8] = wd;
                }
                const int ch = d0 + kGN * gi;
                if (ch % 16 == 0) row[D / 2 + ch / 16] = static_cast<uint8_t>(scode);
            }
            st_bytes<CPL / 2>(row + d0 / 2, w);
        }
    }
}

// ---------------------------------------------------------------- keys

// Raw A-operand data of one lane for one 64-channel chunk: its record's
// channels gw*g + 16c .. +15 in the stored format.
template <int RDT>
struct RawA {
    uint32_t w[RDT == DT_F32 ? 16 : (RDT == DT_BF16 ? 8 : (RDT == DT_E4M3 ? 4 : 3))];
};

template <int RDT>
__device__ __forceinline__ void load_a(const CompP& p, size_t ci, int ch, bool rv, RawA<RDT>& a) {
    constexpr int NW = sizeof(a.w) / 4;
#pragma unroll
    for (int i = 0; i < NW; ++i) a.w[i] = 0u;
    if (!rv) return;
    const int D = p.D;
    if constexpr (RDT == DT_FP4) {
        const uint8_t* row = p.kv + ci * (D / 2 + D / 16);
        const u32x2 codes = *reinterpret_cast<const u32x2*>(row + ch / 2);
        a.w[0] = codes[0];
        a.w[1] = codes[1];
        a.w[2] = row[D / 2 + ch / 16];
    } else {
        constexpr int EB = RDT == DT_F32 ? 4 : (RDT == DT_BF16 ? 2 : 1);
        const u32x4* q = reinterpret_cast<const u32x4*>(p.kv + (ci * D + ch) * EB);
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const u32x4 v = q[k];
            a.w[4 * k] = v[0];
            a.w[4 * k + 1] = v[1];
            a.w[4 * k + 2] = v[2];
            a.w[4 * k + 3] = v[3];
        }
    }
}

// The chunk's two k-steps as bf16 operands (hi; lo only for float32 rows).
template <int RDT>
__device__ __forceinline__ void a_operands(const RawA<RDT>& a, bf16x8 (&ah)[2], bf16x8 (&al)[2]) {
    if constexpr (RDT == DT_FP4) {
        const float scl = e4m3_to_f32(static_cast<uint8_t>(a.w[2]));
        ah[0] = as_bf16x8(fp4x8_to_bf16x8(a.w[0], scl));
        ah[1] = as_bf16x8(fp4x8_to_bf16x8(a.w[1], scl));
    } else if constexpr (RDT == DT_E4M3) {  // codes; the row scale multiplies the keys
        ah[0] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{a.w[0], a.w[1]}));
        ah[1] = as_bf16x8(e4m3x8_to_bf16x8(u32x2{a.w[2], a.w[3]}));
    } else if constexpr (RDT == DT_BF16) {
        ah[0] = as_bf16x8(u32x4{a.w[0], a.w[1], a.w[2], a.w[3]});
        ah[1] = as_bf16x8(u32x4{a.w[4], a.w[5], a.w[6], a.w[7]});
    } else {  // float32 rows: x = hi + lo
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = __uint_as_float(a.w[8 * h + 2 * e]), x1 = __uint_as_float(a.w[8 * h + 2 * e + 1]);
                hi[e] = cvt_bf16x2(x0, x1);
                lo[e] = cvt_bf16x2(x0 - __uint_as_float(hi[e] << 16), x1 - __uint_as_float(hi[e] & 0xFFFF0000u));
            }
            ah[h] = as_bf16x8(hi);
            al[h] = as_bf16x8(lo);
        }
    }
}

// Records written for sequence b: local ids 0 .. n_w-1 (cache rows s0 + s).
// One workgroup: 64 records x all Di keys; wave w takes records
// 32*(w & 1) .. +31 (two 16-row operand tiles) and key columns of half
// (w >> 1), so each B operand read from LDS feeds two products.  Per
// 64-channel chunk c, W_ik rows gw*g' + 16c + i (g' = 0..3, i = 0..15) sit
// transposed in LDS column 16g' + i, high and low bf16 parts,
// double-buffered: the next chunk's W_ik and record data are loaded into
// registers before this chunk's products, so one barrier per chunk
// separates a buffer's writes from its reads.
template <int RDT, int NT, bool WF32>
__global__ __launch_bounds__(256) void keys_kernel(CompP p) {
    extern __shared__ __align__(16) uint8_t ksh[];
    constexpr int Di = NT * 16;
    constexpr int NH = NT / 2;                            // column tiles per wave
    constexpr int kBuf = 2 * Di * kWPitch;                // bf16 per buffer: hi then lo
    uint16_t* wsh = reinterpret_cast<uint16_t*>(ksh);      // [2 buffers][hi, lo][Di][kWPitch]
    float* kout = reinterpret_cast<float*>(ksh);           // [64][Di + 4] keys, after the last chunk
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.y;
    const int D = p.D;
    const int64_t t0 = p.t0[b];
    if (t0 < 0) return;
    const int64_t s0 = t0 / p.m;
    const int n_rec = p.T / p.m;
    const int n_w = static_cast<int>(min(static_cast<int64_t>(n_rec), static_cast<int64_t>(p.N_out) - s0));
    const int s_base = blockIdx.x * kKeyRows;
    if (s_base >= n_w) return;  // workgroup-uniform
    const int r = lane & 15;
    const int g = lane >> 4;
    const int rbase = 32 * (wave & 1);  // first of this wave's rows within the workgroup
    const int t_lo = NH * (wave >> 1);  // first of this wave's column tiles
    bool rv[2];
    size_t ci[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int s = s_base + rbase + 16 * a + r;  // this lane's record in operand tile a
        rv[a] = s < n_w;
        ci[a] = static_cast<size_t>(b) * p.N_out + static_cast<size_t>(s0 + (rv[a] ? s : 0));
    }
    const int gw = D / 4;  // channels of each lane group
    const int nch = D / 64;

    // W_ik staging: item (dq, jq) = 4 consecutive staged columns 4dq .. 4dq+3
    // (one 16-row run of W_ik) x keys 4jq .. 4jq+3; Di / 64 items per thread
    constexpr int kWI = Di / 64;
    f32x4 wr[kWI][4];
    auto load_w = [&](int c) {
#pragma unroll
        for (int it = 0; it < kWI; ++it) {
            const int idx = tid + 256 * it;
            const int dq = idx & 15, jq = idx >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dl = 4 * dq + i;
                const size_t d = static_cast<size_t>(gw * (dl >> 4) + 16 * c + (dl & 15));
                if constexpr (WF32) {
                    wr[it][i] = *reinterpret_cast<const f32x4*>(p.w + (d * Di + 4 * jq) * 4);
                } else {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(p.w + (d * Di + 4 * jq) * 2);
                    wr[it][i] = f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                                      __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
                }
            }
        }
    };
    auto store_w = [&](int buf) {
        uint16_t* hi = wsh + buf * kBuf;
        uint16_t* lo = hi + Di * kWPitch;
#pragma unroll
        for (int it = 0; it < kWI; ++it) {
            const int idx = tid + 256 * it;
            const int dq = idx & 15, jq = idx >> 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int off = (4 * jq + e) * kWPitch + 4 * dq;
                uint32_t h[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) h[i] = cvt_bf16x2(wr[it][2 * i][e], wr[it][2 * i + 1][e]);
                *reinterpret_cast<u32x2*>(hi + off) = u32x2{h[0], h[1]};
                if constexpr (WF32) {  // low parts: w - hi, exact in float32, rounded to bf16
                    uint32_t l[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        l[i] = cvt_bf16x2(wr[it][2 * i][e] - __uint_as_float(h[i] << 16),
                                          wr[it][2 * i + 1][e] - __uint_as_float(h[i] & 0xFFFF0000u));
                    *reinterpret_cast<u32x2*>(lo + off) = u32x2{l[0], l[1]};
                }
            }
        }
    };

    f32x4 acc[2][NH];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < NH; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    RawA<RDT> araw[2];
    load_w(0);
#pragma unroll
    for (int a = 0; a < 2; ++a) load_a<RDT>(p, ci[a], gw * g, rv[a], araw[a]);
    store_w(0);
    for (int c = 0; c < nch; ++c) {
        bf16x8 ah[2][2], al[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a) a_operands<RDT>(araw[a], ah[a], al[a]);
        if (c + 1 < nch) {
            load_w(c + 1);
#pragma unroll
            for (int a = 0; a < 2; ++a) load_a<RDT>(p, ci[a], gw * g + 16 * (c + 1), rv[a], araw[a]);
        }
        __syncthreads();  // buffer c % 2 written by every wave; buffer (c + 1) % 2 no longer read
        const uint16_t* hi = wsh + (c & 1) * kBuf;
        const uint16_t* lo = hi + Di * kWPitch;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                const int off = (16 * (t_lo + t) + r) * kWPitch + 16 * g + 8 * q;
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(hi + off);
                bf16x8 bl;
                if constexpr (WF32) bl = *reinterpret_cast<const bf16x8*>(lo + off);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    acc[a][t] = mfma16x16x32(ah[a][q], bh, acc[a][t]);
                    if constexpr (WF32) acc[a][t] = mfma16x16x32(ah[a][q], bl, acc[a][t]);
                    if constexpr (RDT == DT_F32) acc[a][t] = mfma16x16x32(al[a][q], bh, acc[a][t]);
                }
            }
        }
        if (c + 1 < nch) store_w((c + 1) & 1);
    }
    // keys of rows rbase + 16a + 4g + v, columns 16(t_lo + t) + r -> LDS
    constexpr int kp = Di + 4;
    float rs[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            rs[a][v] = 1.f;
            if constexpr (RDT == DT_E4M3) {
                const int sv = s_base + rbase + 16 * a + 4 * g + v;
                rs[a][v] = sv < n_w ? p.kv_scale[static_cast<size_t>(b) * p.N_out + static_cast<size_t>(s0 + sv)]
                                    : 0.f;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < NH; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                kout[(rbase + 16 * a + 4 * g + v) * kp + 16 * (t_lo + t) + r] = acc[a][t][v] * rs[a][v];
    __syncthreads();

    // ---- quantize the keys: thread t takes record t / 4, key columns
    // kq*(t % 4) .. +kq (whole MXFP4 blocks: kq is 32 or 64 there); a
    // record's maximum for its E4M3 scale is a reduction over its four
    // neighbouring lanes
    constexpr int kq = Di / 4;
    const int rr = tid >> 2, qd = tid & 3, kd = kq * qd;
    const int sr = s_base + rr;
    const bool ok = sr < n_w;
    const size_t cr = static_cast<size_t>(b) * p.N_out + static_cast<size_t>(s0 + (ok ? sr : 0));
    float v[kq];
#pragma unroll
    for (int j = 0; j < kq / 4; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(kout + rr * kp + kd + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = x[e];
    }
    if (p.k_dt == DT_F32) {
        f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.k) + cr * Di + kd);
#pragma unroll
        for (int j = 0; j < kq / 4; ++j)
            if (ok) dst[j] = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
    } else if (p.k_dt == DT_BF16) {
        uint32_t w[kq / 2];
#pragma unroll
        for (int j = 0; j < kq / 2; ++j) w[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        if (ok) st_bytes<2 * kq>(p.k + (cr * Di + kd) * 2, w);
    } else if (p.k_dt == DT_E4M3) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < kq; ++j) am = fmaxf(am, fabsf(v[j]));
        am = lanes_max<4>(am);
        const float scl = am / 448.f;
        const float inv = scl > 0.f ? 1.f / scl : 0.f;
        uint32_t w[kq / 4];
#pragma unroll
        for (int j = 0; j < kq / 4; ++j)
            w[j] = e4m3_encode2(v[4 * j] * inv, v[4 * j + 1] * inv) |
                   (e4m3_encode2(v[4 * j + 2] * inv, v[4 * j + 3] * inv) << 16);
        if (ok) {
            st_bytes<kq>(p.k + cr * Di + kd, w);
            if (qd == 0) reinterpret_cast<float*>(p.k_scale)[cr] = scl;
        }
    } else if constexpr (kq % 32 == 0) {  // MXFP4: blocks of 32 dims share 2^e, e = floor(log2 max|x|) - 2
        uint32_t w[kq / 8], sc = 0u;
#pragma unroll
        for (int blk = 0; blk < kq / 32; ++blk) {
            float am = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(v[32 * blk + j]));
            int e = -127;
            if (am > 0.f) {
                const int be = static_cast<int>((__float_as_uint(am) >> 23) & 0xFFu);
                e = (be == 0 ? -127 : be - 127) - 2;
                e = e < -127 ? -127 : (e > 127 ? 127 : e);
            }
            const float inv = __builtin_amdgcn_ldexpf(1.f, -e);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float* x = v + 32 * blk + 8 * j;
                uint32_t wd = e2m1_encode2<0>(0u, x[0] * inv, x[1] * inv);
                wd = e2m1_encode2<1>(wd, x[2] * inv, x[3] * inv);
                wd = e2m1_encode2<2>(wd, x[4] * inv, x[5] * inv);
                w[4 * blk + j] = e2m1_encode2<3>(wd, x[6] * inv, x[7] * inv);
            }
            sc |= static_cast<uint32_t>(e + 127) << (8 * blk);
        }
        if (ok) {
            st_bytes<kq / 2>(p.k + cr * (Di / 2) + kd / 2, w);
            st_bytes<kq / 32>(p.k_scale + cr * (Di / 32) + kd / 32, &sc);
        }
    }
}

}  // namespace

int launch_compress(const CompressArgs& a, void* stream) {
    CompP p;
    p.B = a.B; p.T = a.T; p.D = a.D; p.m = a.m; p.Di = a.Di; p.N_out = a.N_out;
    p.c = static_cast<const uint8_t*>(a.c);
    p.z = static_cast<const uint8_t*>(a.z);
    p.in_dt = a.in_dtype;
    p.t0 = a.t0;
    p.gain = a.gain;
    p.eps = a.eps;
    p.rope_dims = a.rope_dims;
    p.rope_base = a.rope_base;
    p.w = static_cast<const uint8_t*>(a.w_ik);
    p.w_dt = a.w_dtype;
    p.kv = static_cast<uint8_t*>(a.kv);
    p.kv_scale = a.kv_scale;
    p.kv_dt = a.kv_dtype;
    p.k = static_cast<uint8_t*>(a.k_idx);
    p.k_scale = static_cast<uint8_t*>(a.k_scale);
    p.k_dt = a.k_dtype;
    const int n_rec = a.T / a.m;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 pgrid((n_rec + kPoolRecPerWG - 1) / kPoolRecPerWG, a.B);
    const dim3 pblk(kPoolWaves * 64);
    const bool bf = a.in_dtype == DT_BF16;
    const bool g4 = a.m >= 4;
    const size_t rot = static_cast<size_t>(kPoolRecPerWG) * (a.rope_dims / 2) * sizeof(float2);
#define CSA2_POOL(C)                                                                          \
    if (bf && g4) hipLaunchKernelGGL((pool_kernel<C, true, true>), pgrid, pblk, rot, st, p);      \
    else if (bf) hipLaunchKernelGGL((pool_kernel<C, true, false>), pgrid, pblk, rot, st, p);      \
    else if (g4) hipLaunchKernelGGL((pool_kernel<C, false, true>), pgrid, pblk, rot, st, p);      \
    else hipLaunchKernelGGL((pool_kernel<C, false, false>), pgrid, pblk, rot, st, p);
    switch (a.D / 64) {
        case 2: CSA2_POOL(2) break;
        case 4: CSA2_POOL(4) break;
        case 8: CSA2_POOL(8) break;
        default: CSA2_POOL(16) break;
    }
#undef CSA2_POOL
    if (int e = static_cast<int>(hipGetLastError())) return e;
    const dim3 kgrid((n_rec + kKeyRows - 1) / kKeyRows, a.B);
    const size_t wbytes = static_cast<size_t>(4) * a.Di * kWPitch * sizeof(uint16_t);
    const size_t obytes = static_cast<size_t>(kKeyRows) * (a.Di + 4) * sizeof(float);
    const size_t lds = wbytes > obytes ? wbytes : obytes;
#define CSA2_KEYS_W(R, W)                                                                             \
    switch (a.Di / 16) {                                                                              \
        case 4: hipLaunchKernelGGL((keys_kernel<R, 4, W>), kgrid, dim3(256), lds, st, p); break;      \
        case 8: hipLaunchKernelGGL((keys_kernel<R, 8, W>), kgrid, dim3(256), lds, st, p); break;      \
        case 12: hipLaunchKernelGGL((keys_kernel<R, 12, W>), kgrid, dim3(256), lds, st, p); break;    \
        default: hipLaunchKernelGGL((keys_kernel<R, 16, W>), kgrid, dim3(256), lds, st, p); break;    \
    }
#define CSA2_KEYS(R)                  \
    if (a.w_dtype == DT_F32) {        \
        CSA2_KEYS_W(R, true)          \
    } else {                          \
        CSA2_KEYS_W(R, false)         \
    }
    switch (a.kv_dtype) {
        case DT_F32: CSA2_KEYS(DT_F32) break;
        case DT_BF16: CSA2_KEYS(DT_BF16) break;
        case DT_E4M3: CSA2_KEYS(DT_E4M3) break;
        default: CSA2_KEYS(DT_FP4) break;
    }
#undef CSA2_KEYS
#undef CSA2_KEYS_W
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
