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
// compress_kernel: one workgroup of 4 waves per 16 records of one
// sequence.  A wave builds one record at a time: lane l owns channels
// CPL*l .. CPL*l+CPL-1 (so rotary pairs and FP4 groups of 16 channels stay
// within one lane or a few neighbouring lanes), runs an online softmax over
// the block's tokens, reduces the row's mean square across the wave,
// rotates, quantizes and stores the row, and keeps the stored row's values
// in LDS.  The 16 rows' keys are then formed in float32 (each thread owns
// one key dimension of 8 records; W_ik is read once per workgroup) and
// quantized per record.
#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kRecPerWG = 16;
constexpr int kCThreads = 256;

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

__device__ __forceinline__ float ld_in(const uint8_t* base, size_t i, int dt) {
    return dt == DT_F32 ? reinterpret_cast<const float*>(base)[i]
                        : bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
}

// Nearest e4m3fn code of v (ties to even, saturating at +-448).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fminf(fabsf(v), 448.f);
    uint32_t mag;
    if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (rintf rounds ties to even)
        mag = static_cast<uint32_t>(rintf(a * 512.f));
    } else {               // keep 3 mantissa bits of the float, ties to even
        uint32_t u = __float_as_uint(a);
        u += 0x7FFFFu + ((u >> 20) & 1u);
        mag = ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);
    }
    return sign | (mag < 0x7Eu ? mag : 0x7Eu);
}

// Nearest E2M1 code of v (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; ties to
// the even code; saturating at 6).  A tie at a midpoint goes up exactly
// when the lower code is odd.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    const float a = fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_value(uint32_t code) {
    const float lv[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    const float x = lv[code & 7u];
    return (code & 8u) ? -x : x;
}

// Largest |x| over aligned groups of `lanes` neighbouring lanes (a power of 2).
__device__ __forceinline__ float group_max(float a, int lanes) {
    for (int o = 1; o < lanes; o <<= 1) a = fmaxf(a, shfl_xor_f(a, o));
    return a;
}

template <int CPL>
__global__ __launch_bounds__(kCThreads) void compress_kernel(CompP p) {
    extern __shared__ __align__(16) float csh[];
    float* xs = csh;                               // [16][D] stored rows' values
    float* ks = csh + kRecPerWG * p.D;             // [16][Di] keys before quantization
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.y;
    const int D = p.D;
    const int n_rec = p.T / p.m;
    const int s_begin = blockIdx.x * kRecPerWG;
    const int64_t t0 = p.t0[b];
    const int64_t s0 = t0 >= 0 ? t0 / p.m : -1;    // cache row of the first record
    const int r0 = D - p.rope_dims;
    const int d0 = CPL * lane;

    // ---- records: pool, normalize, rotate, quantize, store ----
    for (int rr = wave; rr < kRecPerWG; rr += 4) {
        const int s = s_begin + rr;
        if (s >= n_rec) break;  // wave-uniform
        float mx[CPL], sum[CPL], acc[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            mx[j] = -__builtin_huge_valf();
            sum[j] = 0.f;
            acc[j] = 0.f;
        }
#pragma unroll 4
        for (int i = 0; i < p.m; ++i) {  // online softmax over the block's tokens
            const size_t row = (static_cast<size_t>(b) * p.T + static_cast<size_t>(s) * p.m + i) * D + d0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float cv = ld_in(p.c, row + j, p.in_dt);
                const float zv = ld_in(p.z, row + j, p.in_dt);
                const float nm = fmaxf(mx[j], zv);
                const float sc = __expf(mx[j] - nm);
                const float e = __expf(zv - nm);
                sum[j] = sum[j] * sc + e;
                acc[j] = acc[j] * sc + e * cv;
                mx[j] = nm;
            }
        }
        float x[CPL];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            x[j] = acc[j] / sum[j];
            ss += x[j] * x[j];
        }
        ss = warp_sum(ss);
        const float inv = rsqrtf(ss / static_cast<float>(D) + p.eps);
#pragma unroll
        for (int j = 0; j < CPL; ++j) x[j] *= inv * p.gain[d0 + j];
        // forward rotation of the rotary pairs to the record's position
        const int64_t pos = t0 + static_cast<int64_t>(s) * p.m + p.m - 1;
#pragma unroll
        for (int j = 0; j < CPL; j += 2) {
            const int d = d0 + j;
            if (d >= r0) {
                float cs, sn;
                rope_angle(pos, (d - r0) >> 1, p.rope_dims, p.rope_base, cs, sn);
                const float a = x[j], bb = x[j + 1];
                x[j] = a * cs - bb * sn;
                x[j + 1] = a * sn + bb * cs;
            }
        }
        // quantize into the cache row; xs keeps the stored values
        const int64_t crow = s0 + s;
        const bool in_cache = s0 >= 0 && crow < p.N_out;
        const size_t ci = static_cast<size_t>(b) * p.N_out + static_cast<size_t>(crow);
        float xq[CPL];
        if (p.kv_dt == DT_F32 || p.kv_dt == DT_BF16) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                if (p.kv_dt == DT_BF16) {
                    const uint32_t hb = f32_to_bf16_rne(x[j]);
                    xq[j] = __uint_as_float(hb << 16);
                    if (in_cache) reinterpret_cast<uint16_t*>(p.kv)[ci * D + d0 + j] = static_cast<uint16_t>(hb);
                } else {
                    xq[j] = x[j];
                    if (in_cache) reinterpret_cast<float*>(p.kv)[ci * D + d0 + j] = x[j];
                }
            }
        } else if (p.kv_dt == DT_E4M3) {  // one scale per row: max|x| / 448
            float am = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) am = fmaxf(am, fabsf(x[j]));
            am = warp_max(am);
            const float scl = am / 448.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const uint32_t code = scl > 0.f ? e4m3_encode(x[j] / scl) : 0u;
                xq[j] = e4m3_to_f32(static_cast<uint8_t>(code)) * scl;
                if (in_cache) p.kv[ci * D + d0 + j] = static_cast<uint8_t>(code);
            }
            if (in_cache && lane == 0) p.kv_scale[ci] = scl;
        } else {  // FP4 row: E2M1 codes, one E4M3 scale (max|x| / 6) per 16 channels
            constexpr int kGL = CPL >= 16 ? 1 : 16 / CPL;  // lanes per group
            float am = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) am = fmaxf(am, fabsf(x[j]));
            const size_t rb = static_cast<size_t>(D) / 2 + D / 16;  // row bytes
            uint8_t* row = p.kv + ci * rb;
#pragma unroll
            for (int gsub = 0; gsub < (CPL >= 16 ? CPL / 16 : 1); ++gsub) {
                float ga = 0.f;
                if constexpr (CPL >= 16) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) ga = fmaxf(ga, fabsf(x[16 * gsub + j]));
                } else {
                    ga = group_max(am, kGL);
                }
                const uint32_t scode = e4m3_encode(ga / 6.f);
                const float scl = e4m3_to_f32(static_cast<uint8_t>(scode));
                const int jb = CPL >= 16 ? 16 * gsub : 0;
                const int je = CPL >= 16 ? jb + 16 : CPL;
                for (int j = jb; j < je; j += 2) {
                    const uint32_t c0 = scl > 0.f ? e2m1_encode(x[j] / scl) : 0u;
                    const uint32_t c1 = scl > 0.f ? e2m1_encode(x[j + 1] / scl) : 0u;
                    xq[j] = e2m1_value(c0) * scl;
                    xq[j + 1] = e2m1_value(c1) * scl;
                    if (in_cache) row[(d0 + j) / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
                }
                const int grp = (d0 + jb) / 16;
                if (in_cache && (d0 + jb) % 16 == 0) row[D / 2 + grp] = static_cast<uint8_t>(scode);
            }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) xs[rr * D + d0 + j] = xq[j];
    }
    __syncthreads();

    // ---- keys: k = x_stored W_ik, float32 ----
    const int nr = min(kRecPerWG, n_rec - s_begin);
    for (int j = tid % p.Di, half = tid / p.Di; half * 8 < kRecPerWG; half += kCThreads / p.Di) {
        if (tid >= (kCThreads / p.Di) * p.Di) break;
        float a[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) a[r] = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) {
            const float w = ld_in(p.w, static_cast<size_t>(d) * p.Di + j, p.w_dt);
#pragma unroll
            for (int r = 0; r < 8; ++r) a[r] = fmaf(xs[(half * 8 + r) * D + d], w, a[r]);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) ks[(half * 8 + r) * p.Di + j] = a[r];
    }
    __syncthreads();

    // ---- quantize the keys: one wave per record ----
    const int kpl = p.Di / 64;  // key dims per lane (Di is a multiple of 64, <= 256)
    for (int rr = wave; rr < nr; rr += 4) {
        const int64_t crow = s0 + s_begin + rr;
        if (s0 < 0 || crow >= p.N_out) continue;
        const size_t ci = static_cast<size_t>(b) * p.N_out + static_cast<size_t>(crow);
        float v[4];
        for (int j = 0; j < kpl; ++j) v[j] = ks[rr * p.Di + kpl * lane + j];
        const int kd = kpl * lane;
        if (p.k_dt == DT_F32) {
            for (int j = 0; j < kpl; ++j) reinterpret_cast<float*>(p.k)[ci * p.Di + kd + j] = v[j];
        } else if (p.k_dt == DT_BF16) {
            for (int j = 0; j < kpl; ++j)
                reinterpret_cast<uint16_t*>(p.k)[ci * p.Di + kd + j] = static_cast<uint16_t>(f32_to_bf16_rne(v[j]));
        } else if (p.k_dt == DT_E4M3) {
            float am = 0.f;
            for (int j = 0; j < kpl; ++j) am = fmaxf(am, fabsf(v[j]));
            am = warp_max(am);
            const float scl = am / 448.f;
            for (int j = 0; j < kpl; ++j)
                p.k[ci * p.Di + kd + j] = static_cast<uint8_t>(scl > 0.f ? e4m3_encode(v[j] / scl) : 0u);
            if (lane == 0) reinterpret_cast<float*>(p.k_scale)[ci] = scl;
        } else {  // MXFP4: blocks of 32 dims share 2^e, e = floor(log2 max|x|) - 2
            float am = 0.f;
            for (int j = 0; j < kpl; ++j) am = fmaxf(am, fabsf(v[j]));
            am = group_max(am, 32 / kpl);
            int e = -127;
            if (am > 0.f) {
                const int be = static_cast<int>((__float_as_uint(am) >> 23) & 0xFFu);
                e = (be == 0 ? -127 : be - 127) - 2;
                e = e < -127 ? -127 : (e > 127 ? 127 : e);
            }
            const float inv = ldexpf(1.f, -e);
            uint8_t* krow = p.k + ci * (p.Di / 2);
            for (int j = 0; j < kpl; j += 2) {
                const uint32_t c0 = e2m1_encode(v[j] * inv);
                const uint32_t c1 = e2m1_encode(v[j + 1] * inv);
                krow[(kd + j) / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
            }
            if (kd % 32 == 0) p.k_scale[ci * (p.Di / 32) + kd / 32] = static_cast<uint8_t>(e + 127);
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
    const dim3 grid((n_rec + kRecPerWG - 1) / kRecPerWG, a.B);
    const size_t lds = static_cast<size_t>(kRecPerWG) * (a.D + a.Di) * sizeof(float);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (a.D / 64) {
        case 2: hipLaunchKernelGGL(compress_kernel<2>, grid, dim3(kCThreads), lds, st, p); break;
        case 4: hipLaunchKernelGGL(compress_kernel<4>, grid, dim3(kCThreads), lds, st, p); break;
        case 8: hipLaunchKernelGGL(compress_kernel<8>, grid, dim3(kCThreads), lds, st, p); break;
        default: hipLaunchKernelGGL(compress_kernel<16>, grid, dim3(kCThreads), lds, st, p); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace csa2
