// Bandwidth-bound quantized GEMV core shared by the dense linear and the MoE kernels.
//
// A row of a group-affine quantized matrix is covered by a segment of `lpr` lanes; lane
// `sl` of the segment owns the 32-input chunks sl, sl + lpr, ...  Per chunk it issues
// 128-bit loads of the packed words (16 bytes for 4-bit, 32 bytes for 8-bit), one fp16
// scale and bias, builds exact fp16 codes (device.hpp) and dots them with the staged x
// pairs of each token by v_dot2 into fp32.  The group's affine terms enter once per
// chunk: s*sum(q x) + b*sum(x) = (C s) * dot + (b - C s) * sum(x), where C = 16 (4-bit)
// or 256 (8-bit) and dot = sum((1 + q/C) x).
#pragma once

#include "device.hpp"

namespace qmoe {

constexpr int GEMV_MT = 8;  // most tokens per pass over a weight row

// Stage `mt` token rows of an fp16 source into LDS: `xs` gets the inputs as pairs in the
// order the unpacking produces (K/2 pairs per token), `xsum` the per-chunk (32-input)
// sums in fp32.  Token i of the batch is source row `rows[i]`.  All threads of the block
// take part; the caller synchronises.
template <int BITS>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ src, const int* rows,
                                             int mt, int K, f16x2* xs, float* xsum) {
    const int units = K / 8;
    for (int u = threadIdx.x; u < mt * units; u += blockDim.x) {
        const int t = u / units, c = u % units;
        const uint4 raw = *reinterpret_cast<const uint4*>(src + (long)rows[t] * K + c * 8);
        const f16* h = reinterpret_cast<const f16*>(&raw);
        f16x2* dst = xs + (long)t * (K / 2) + c * 4;
        if constexpr (BITS == 4) {
            pair_perm8(h, dst);
        } else {
            pair_perm4(h, dst);
            pair_perm4(h + 4, dst + 2);
        }
    }
    const int chunks = K / 32;
    for (int u = threadIdx.x; u < mt * chunks; u += blockDim.x) {
        const int t = u / chunks, c = u % chunks;
        const uint4* p = reinterpret_cast<const uint4*>(src + (long)rows[t] * K + c * 32);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 raw = p[i];
            const f16* h = reinterpret_cast<const f16*>(&raw);
#pragma unroll
            for (int j = 0; j < 8; ++j) s += (float)h[j];
        }
        xsum[t * chunks + c] = s;
    }
}

// acc[t] += this lane's share of row `row` . x_t for t < mt (segment-partial sums).
template <int BITS>
__device__ __forceinline__ void qdot_row(const uint32_t* __restrict__ packed,
                                         const uint16_t* __restrict__ scales,
                                         const uint16_t* __restrict__ biases, int K, long row,
                                         int lpr, int sl, const f16x2* xs, const float* xsum,
                                         int mt, float (&acc)[GEMV_MT]) {
    constexpr int WPC = BITS == 4 ? 4 : 8;  // words per chunk
    constexpr float C = code_div<BITS>();
    const int chunks = K / 32;
    const long wpr = (long)K * BITS / 32;
    for (int c = sl; c < chunks; c += lpr) {
        uint32_t wd[WPC];
        const uint4* src = reinterpret_cast<const uint4*>(packed + row * wpr + c * WPC);
#pragma unroll
        for (int i = 0; i < WPC / 4; ++i) {
            const uint4 v = src[i];
            wd[4 * i] = v.x; wd[4 * i + 1] = v.y; wd[4 * i + 2] = v.z; wd[4 * i + 3] = v.w;
        }
        const long gi = row * (K / 64) + c / 2;
        const float s = h2f(scales[gi]), b = h2f(biases[gi]);
        const float sC = s * C, bb = b - sC;
#pragma unroll
        for (int t = 0; t < GEMV_MT; ++t) {
            if (t < mt) {
                const f16x2* xp = xs + (long)t * (K / 2) + c * 16;
                float d = 0.0f;
#pragma unroll
                for (int j = 0; j < WPC; ++j) {
                    if constexpr (BITS == 4) d = dot_word4(wd[j], xp + 4 * j, d);
                    else d = dot_word8(wd[j], xp + 2 * j, d);
                }
                acc[t] = fmaf(sC, d, fmaf(bb, xsum[t * chunks + c], acc[t]));
            }
        }
    }
}

// Sum over the `lpr`-lane segment (butterfly; every lane of the segment gets the total).
__device__ __forceinline__ float segment_sum(float v, int lpr) {
    for (int off = lpr / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Largest power of two <= 64 dividing K/32: lanes per row segment.
__host__ __device__ inline int lanes_per_row(int K) {
    int g = 64;
    while (g > 1 && ((K / 32) % g) != 0) g >>= 1;
    return g;
}

}  // namespace qmoe
