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

constexpr int NT = 256;   // threads per block of every kernel that stages rows

// Stage `mt` token rows of an fp16 source into LDS: `xs` gets the inputs as pairs in the
// order the unpacking produces (K/2 pairs per token), `xsum` the per-chunk (32-input)
// sums in fp32.  Token i of the batch is source row `rows[i]`.  All threads of the block
// take part; the caller synchronises.
template <int BITS>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ src, const int* rows,
                                             int mt, int K, f16x2* xs, float* xsum) {
    const int units = K / 8;
    for (int u = threadIdx.x; u < mt * units; u += NT) {
        const int t = u / units, c = u % units;
        const uint4 raw = *reinterpret_cast<const uint4*>(src + (long)rows[t] * K + c * 8);
        reinterpret_cast<uint4*>(xs + (long)t * (K / 2))[c] = BITS == 4 ? pair_perm8_w(raw) : pair_perm4x2_w(raw);
    }
    const int chunks = K / 32;
    for (int u = threadIdx.x; u < mt * chunks; u += NT) {
        const int t = u / chunks, c = u % chunks;
        const uint4* p = reinterpret_cast<const uint4*>(src + (long)rows[t] * K + c * 32);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s += sum8_w(p[i]);
        xsum[t * chunks + c] = s;
    }
}



// Write one staged 8-input unit to LDS (pair order of the unpacking) and, from the quad
// of lanes that holds a 32-input chunk, its fp32 sum.  All lanes must call (DPP).
template <int BITS>
__device__ __forceinline__ void commit_unit(const uint4& raw, int u, bool valid, f16x2* xs,
                                            float* xsum) {
    float s = valid ? sum8_w(raw) : 0.0f;
    s += dpp<DPP_XOR1>(s);
    s += dpp<DPP_XOR2>(s);
    if (valid) {
        reinterpret_cast<uint4*>(xs)[u] = BITS == 4 ? pair_perm8_w(raw) : pair_perm4x2_w(raw);   // one 16-byte LDS store
        if ((threadIdx.x & 3) == 0) xsum[u / 4] = s;
    }
}

// Stage n_rows fp16 rows of K inputs (row i starts at rowp(i), a 16-byte aligned uint4
// pointer) into LDS in the pair order of the unpacking, plus the fp32 sum of every
// 32-input chunk.  Every load of a pass is issued before any is used (MAXP 16-byte loads
// per thread per pass).  The whole block (NT threads) must call this; the caller
// synchronises afterwards.
template <int BITS, int MAXP, class RowPtr>
__device__ __forceinline__ void stage_rows(RowPtr rowp, int n_rows, int K, f16x2* xs,
                                           float* xsum) {
    const int units = K / 8, total = n_rows * units;
    const int q_step = NT / units, r_step = NT % units;   // one division per call
    for (int base = 0; base < total; base += NT * MAXP) {
        uint4 raw[MAXP];
        int r = (base + (int)threadIdx.x) / units, c = (base + (int)threadIdx.x) % units;
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {   // unconditional loads (clamped row): no branch
            raw[p] = rowp(min(r, n_rows - 1))[c];
            c += r_step;
            r += q_step;
            if (c >= units) { c -= units; ++r; }
        }
        __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any use
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int u = base + p * NT + threadIdx.x;
            commit_unit<BITS>(raw[p], u, u < total, xs, xsum);
        }
    }
}

// Two-phase form of stage_rows for one pass (n_rows * K/8 <= NT * MAXP): load() issues the
// loads into registers, commit() writes LDS.  Whatever a kernel issues between the two
// stays in flight together with these loads.
template <int BITS, int MAXP>
struct StageRegs {
    uint4 raw[MAXP];
    template <class RowPtr>
    __device__ __forceinline__ void load(RowPtr rowp, int n_rows, int K) {
        const int units = K / 8, total = n_rows * units;
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int u = min(p * NT + (int)threadIdx.x, total - 1);
            raw[p] = rowp(u / units)[u % units];
        }
    }
    __device__ __forceinline__ void commit(int n_rows, int K, f16x2* xs, float* xsum) const {
        const int total = n_rows * (K / 8);
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int u = p * NT + threadIdx.x;
            commit_unit<BITS>(raw[p], u, u < total, xs, xsum);
        }
    }
};

// A stored group parameter as fp32: fp16 bits, or bf16 bits when BF.
template <bool BF>
__device__ __forceinline__ float param_f32(uint16_t v) { return BF ? bf2f(v) : h2f(v); }

// acc[t] += this lane's share of row `row` . x_t for t < mt (segment-partial sums).  G is
// the group size (64, or 32: then every 32-input chunk has its own parameters), BF selects
// bf16 parameters.
template <int BITS, int G = 64, bool BF = false>
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
        const long gi = row * (K / G) + c / (G / 32);
        const float s = param_f32<BF>(scales[gi]), b = param_f32<BF>(biases[gi]);
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

// One row's chunks for this lane (the chunk set of qdot_row, at most MAXC of them), loaded
// into registers by load() so that every load of a wave is in flight before any dot.
template <int BITS, int MAXC, int G = 64, bool BF = false>
struct RowRegs {
    static constexpr int WPC = BITS == 4 ? 4 : 8;
    uint32_t w[MAXC][WPC];
    uint16_t s[MAXC], b[MAXC];   // raw parameter bits: converted only when used
    int n;
    // Loads are unconditional (chunk index clamped into the row, `valid == false` reads the
    // same row and marks nothing usable) so the compiler issues them without branches and
    // does not wait on them until dot().
    __device__ __forceinline__ void load(const uint32_t* __restrict__ packed,
                                         const uint16_t* __restrict__ scales,
                                         const uint16_t* __restrict__ biases, int K, long row,
                                         int lpr, int sl, bool valid = true) {
        const int chunks = K / 32;
        const long wpr = (long)K * BITS / 32;
        n = 0;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int c = min(sl + i * lpr, chunks - 1);
            const uint4* src = reinterpret_cast<const uint4*>(packed + row * wpr + c * WPC);
#pragma unroll
            for (int j = 0; j < WPC / 4; ++j) {
                const uint4 v = src[j];
                w[i][4 * j] = v.x; w[i][4 * j + 1] = v.y; w[i][4 * j + 2] = v.z; w[i][4 * j + 3] = v.w;
            }
            const long gi = row * (K / G) + c / (G / 32);
            s[i] = scales[gi];
            b[i] = biases[gi];
            if (valid && sl + i * lpr < chunks) n = i + 1;
        }
    }
    // Pins the first use of every loaded register here (see hold()): called after a later
    // round trip is issued, it keeps the compiler from converting the weights (and so waiting
    // for them) ahead of it, e.g. by hoisting the conversions out of a loop.
    __device__ __forceinline__ void hold() {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
#pragma unroll
            for (int j = 0; j < WPC; ++j) asm volatile("" : "+v"(w[i][j]));
            uint32_t sb = (uint32_t)s[i] | ((uint32_t)b[i] << 16);
            asm volatile("" : "+v"(sb));
            s[i] = (uint16_t)sb;
            b[i] = (uint16_t)(sb >> 16);
        }
    }
    // acc[t] += chunk dots for tokens t < mt staged in xs/xsum
    __device__ __forceinline__ void dot(int K, int lpr, int sl, const f16x2* xs, const float* xsum,
                                        int mt, float (&acc)[GEMV_MT]) const {
        constexpr float C = code_div<BITS>();
        const int chunks = K / 32;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            if (i < n) {
                const int c = sl + i * lpr;
                const float sC = param_f32<BF>(s[i]) * C, bb = param_f32<BF>(b[i]) - sC;
#pragma unroll
                for (int t = 0; t < GEMV_MT; ++t) {
                    if (t < mt) {
                        const f16x2* xp = xs + (long)t * (K / 2) + c * 16;
                        float d = 0.0f;
#pragma unroll
                        for (int j = 0; j < WPC; ++j) {
                            if constexpr (BITS == 4) d = dot_word4(w[i][j], xp + 4 * j, d);
                            else d = dot_word8(w[i][j], xp + 2 * j, d);
                        }
                        acc[t] = fmaf(sC, d, fmaf(bb, xsum[t * chunks + c], acc[t]));
                    }
                }
            }
        }
    }
};

// Sum over the `lpr`-lane segment (every lane of the segment gets the total; see seg_sum).
__device__ __forceinline__ float segment_sum(float v, int lpr) {
    switch (lpr) {
        case 1: return v;
        case 2: return seg_sum<2>(v);
        case 4: return seg_sum<4>(v);
        case 8: return seg_sum<8>(v);
        case 16: return seg_sum<16>(v);
        case 32: return seg_sum<32>(v);
        default: return seg_sum<64>(v);
    }
}

// Largest power of two <= 64 dividing K/32: lanes per row segment.
__host__ __device__ inline int lanes_per_row(int K) {
    int g = 64;
    while (g > 1 && ((K / 32) % g) != 0) g >>= 1;
    return g;
}

}  // namespace qmoe
