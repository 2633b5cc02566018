// Weight-activation integer path of the super-group GEMM:
//   y[b][n] = fp16( s_W[n] * s_X[b] * sum_k Q(W)[n][k] * Q(X)[b][k] ).
//
// "EDGERAZOR deep dive" (zhichai.net) section 2.1, matrix-multiplication decomposition: with
// the activations quantized as well, the sum over the inputs is an integer dot product and
// the product of the two scales is applied once per output; section 3.1 (table of the
// weight-activation results) runs activations at 8 bits.  Activations: one symmetric scale
// per token, s_X = fp16(max(max|x| / 127, 1e-5)), Q(x) = clip(rint(x / s_X), -127, 127) in
// fp32 against the stored scale (as the weight quantizers take their codes).  Weights: the
// super-group format of supergroup.hip (4-bit channel rows, nibble q + 8; ternary rows, 2-bit
// field q + 1).
//
// Codes stay unsigned in the byte lanes of the integer dot (c = q + off, off = 8 or 1) and
// the offset is taken out once per output: sum_k q x = sum_k c x - off * sum_k x, all in
// int32 (exact).  Token codes are staged in LDS in the byte order in which a packed weight
// word unpacks (4-bit: w & 0x0F0F0F0F holds inputs 0, 2, 4, 6 of the word, (w >> 4) & ...
// inputs 1, 3, 5, 7; 2-bit: (w >> 2e) & 0x03030303 holds inputs e, e + 4, e + 8, e + 12).
//   * few tokens (<= 8): one wave per output channel, v_dot4_i32_i8 over 4-byte groups;
//   * more tokens, inputs a multiple of 1024: v_mfma_i32_16x16x64_i8 with 16 tokens as A
//     (from LDS) and 16 channels of one kind as B (unpacked in registers), 128 channels and
//     16 tokens per block.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace qmoe {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int A8_MT = 8;          // tokens per pass of the few-token kernel
constexpr int A8_CHUNK = 1024;    // inputs staged per pass of the MFMA kernel
constexpr int A8_PITCH = A8_CHUNK + 16;   // LDS row pitch in bytes (16-byte reads spread over the banks)
constexpr int A8_WAVES = 8;       // waves per block of the MFMA kernel (16 channels each)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// s_X of a token from its largest magnitude: fp16(max(amax / 127, 1e-5)), returned as fp32
__device__ __forceinline__ float act8_scale(float amax) {
    return h2f(f2h(fmaxf(amax / 127.0f, 1e-5f)));
}

// Q(x): the correctly rounded fp32 quotient x / s rounded to the nearest integer (ties to
// even), clipped to +-127.
__device__ __forceinline__ int act8_code(float x, float s) {
    return min(max((int)rintf(x / s), -127), 127);
}

// The largest |x| of a row of K fp16 inputs, by one wave (K a multiple of 512).
__device__ __forceinline__ float row_amax(const uint16_t* __restrict__ row, int K) {
    const int lane = threadIdx.x & 63;
    float m = 0.0f;
    for (int k = lane * 8; k < K; k += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(half_lo(w[i])), fabsf(half_hi(w[i]))));
    }
    return wave_max(m);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// Codes of 16 consecutive inputs (two 16-byte loads) and their sum.
__device__ __forceinline__ int codes16(const uint4& r0, const uint4& r1, float s, int (&q)[16]) {
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        q[2 * i] = act8_code(half_lo(w[i]), s);
        q[2 * i + 1] = act8_code(half_hi(w[i]), s);
        sum += q[2 * i] + q[2 * i + 1];
    }
    return sum;
}

// The 16 codes in the byte order of two 4-bit words (8 inputs each)
__device__ __forceinline__ uint4 order4(const int (&q)[16]) {
    return make_uint4(pack4(q[0], q[2], q[4], q[6]), pack4(q[1], q[3], q[5], q[7]),
                      pack4(q[8], q[10], q[12], q[14]), pack4(q[9], q[11], q[13], q[15]));
}

// ... and of one 2-bit word (16 inputs)
__device__ __forceinline__ uint4 order2(const int (&q)[16]) {
    return make_uint4(pack4(q[0], q[4], q[8], q[12]), pack4(q[1], q[5], q[9], q[13]),
                      pack4(q[2], q[6], q[10], q[14]), pack4(q[3], q[7], q[11], q[15]));
}

// ---- activation codes alone (the integer decisions, exported for testing and reuse) ------

__global__ void __launch_bounds__(256) k_act8_quantize(const uint16_t* __restrict__ x, int nb, int K,
                                                       int8_t* __restrict__ qx,
                                                       uint16_t* __restrict__ sx) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= nb) return;
    const uint16_t* row = x + (long)t * K;
    const float s = act8_scale(row_amax(row, K));
    if (lane == 0) sx[t] = f2h(s);
    for (int k = lane * 16; k < K; k += 1024) {
        const uint4 r0 = *reinterpret_cast<const uint4*>(row + k);
        const uint4 r1 = *reinterpret_cast<const uint4*>(row + k + 8);
        int q[16];
        codes16(r0, r1, s, q);
        *reinterpret_cast<uint4*>(qx + (long)t * K + k) =
            make_uint4(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]),
                       pack4(q[8], q[9], q[10], q[11]), pack4(q[12], q[13], q[14], q[15]));
    }
}

// ---- few tokens: one wave per output channel, v_dot4 -------------------------------------

__global__ void __launch_bounds__(256) k_sg_a8_gemv(const uint16_t* __restrict__ x, int nb, int K,
                                                    int rows, int period,
                                                    const uint32_t* __restrict__ p4,
                                                    const uint32_t* __restrict__ p2,
                                                    const uint16_t* __restrict__ scales,
                                                    uint16_t* __restrict__ y) {
    __shared__ __align__(16) int8_t x4[16384];    // [mt][K] codes in 4-bit word order
    __shared__ __align__(16) int8_t x2[16384];    // [mt][K] codes in 2-bit word order
    __shared__ float sx[A8_MT];
    __shared__ int ssum[A8_MT];
    const int mt_max = min(A8_MT, 16384 / K);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_global = blockIdx.x * 4 + wave;
    const int n_waves = gridDim.x * 4;
    for (int t0 = 0; t0 < nb; t0 += mt_max) {
        const int mt = min(mt_max, nb - t0);
        __syncthreads();
        if (threadIdx.x < A8_MT) ssum[threadIdx.x] = 0;
        for (int t = wave; t < mt; t += 4) {
            const float s = act8_scale(row_amax(x + (long)(t0 + t) * K, K));
            if (lane == 0) sx[t] = s;
        }
        __syncthreads();
        for (int u = threadIdx.x; u < mt * (K / 16); u += 256) {
            const int t = u / (K / 16), c = u % (K / 16);
            const uint4* src = reinterpret_cast<const uint4*>(x + (long)(t0 + t) * K + c * 16);
            int q[16];
            const int sum = codes16(src[0], src[1], sx[t], q);
            *reinterpret_cast<uint4*>(x4 + t * K + c * 16) = order4(q);
            *reinterpret_cast<uint4*>(x2 + t * K + c * 16) = order2(q);
            atomicAdd(&ssum[t], sum);
        }
        __syncthreads();
        for (int n = wave_global; n < rows; n += n_waves) {
            const bool four = (n % period) == 0;
            const int blk = n / period, pos = n % period;
            int acc[A8_MT];
#pragma unroll
            for (int t = 0; t < A8_MT; ++t) acc[t] = 0;
            if (four) {
                const uint4* row = reinterpret_cast<const uint4*>(p4 + (long)blk * (K / 8));
                for (int c = lane; c < K / 32; c += 64) {        // 4 words = 32 inputs
                    const uint4 v = row[c];
                    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int t = 0; t < A8_MT; ++t) {
                        if (t < mt) {
                            const int* xp = reinterpret_cast<const int*>(x4 + t * K + c * 32);
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                acc[t] = __builtin_amdgcn_sdot4((int)(wd[j] & 0x0F0F0F0Fu), xp[2 * j], acc[t], false);
                                acc[t] = __builtin_amdgcn_sdot4((int)((wd[j] >> 4) & 0x0F0F0F0Fu), xp[2 * j + 1], acc[t], false);
                            }
                        }
                    }
                }
            } else {
                const long r2 = (long)blk * (period - 1) + (pos - 1);
                const uint4* row = reinterpret_cast<const uint4*>(p2 + r2 * (K / 16));
                for (int c = lane; c < K / 64; c += 64) {        // 4 words = 64 inputs
                    const uint4 v = row[c];
                    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int t = 0; t < A8_MT; ++t) {
                        if (t < mt) {
                            const int* xp = reinterpret_cast<const int*>(x2 + t * K + c * 64);
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[t] = __builtin_amdgcn_sdot4((int)((wd[j] >> (2 * e)) & 0x03030303u),
                                                                    xp[4 * j + e], acc[t], false);
                            }
                        }
                    }
                }
            }
            const int off = four ? 8 : 1;
            const float sw = h2f(scales[n]);
#pragma unroll
            for (int t = 0; t < A8_MT; ++t) {
                if (t < mt) {
                    const int v = wave_sum_i(acc[t]) - off * ssum[t];
                    if (lane == 0) y[(long)(t0 + t) * rows + n] = f2h(((float)v * sx[t]) * sw);
                }
            }
        }
    }
}

// ---- batched: int8 MFMA --------------------------------------------------------------------

// The largest |x| of 16 inputs held as two 16-byte loads.
__device__ __forceinline__ float amax16(const uint4& r0, const uint4& r1) {
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(half_lo(w[i])), fabsf(half_hi(w[i]))));
    return m;
}

// A block: 16 * A8_WAVES channels of one kind x 16 tokens, 16 channels per wave.  Wave w
// stages tokens w, w + A8_WAVES, ... (a 1024-input chunk of a row is one 16-input unit per
// lane), so each wave holds whole rows: a row's scale is a wave maximum over values already
// in registers (one pass over the inputs when they fit one chunk) and its code sum a wave
// sum.  Every block codes its 16 tokens itself; 8 waves halve that repeated work against 4
// (7.9 -> 7.6 us at 64 tokens), 16 waves stream too many weight bytes through one CU.
template <bool FOUR>
__device__ __forceinline__ void sg_a8_mfma_block(const uint16_t* __restrict__ x, int nb, int K,
                                                 int rows, int period,
                                                 const uint32_t* __restrict__ pw,
                                                 const uint16_t* __restrict__ scales,
                                                 uint16_t* __restrict__ y, int kind_rows, int rb,
                                                 int8_t* xl, float* sx, int* ssum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, j = lane >> 4;
    const int kr = rb * (16 * A8_WAVES) + wave * 16 + col;     // this lane's row of its kind
    const int krc = min(kr, kind_rows - 1);
    const int t0 = blockIdx.y * 16;
    const int nt = min(16, nb - t0);
    constexpr int PASSES = 16 / A8_WAVES;                      // token rows per wave
    const uint16_t* xr[PASSES];                                // rows past nt repeat the last
#pragma unroll
    for (int i = 0; i < PASSES; ++i) xr[i] = x + (long)(t0 + min(A8_WAVES * i + wave, nt - 1)) * K + lane * 16;
    float srow[PASSES];
    int qsum[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) qsum[i] = 0;
    if (K > A8_CHUNK) {   // the rows' scales first, one pass over every chunk
        float m[PASSES];
#pragma unroll
        for (int i = 0; i < PASSES; ++i) m[i] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += A8_CHUNK) {
            uint4 v[PASSES][2];
#pragma unroll
            for (int i = 0; i < PASSES; ++i) {
                v[i][0] = reinterpret_cast<const uint4*>(xr[i] + k0)[0];
                v[i][1] = reinterpret_cast<const uint4*>(xr[i] + k0)[1];
            }
#pragma unroll
            for (int i = 0; i < PASSES; ++i) m[i] = fmaxf(m[i], amax16(v[i][0], v[i][1]));
        }
#pragma unroll
        for (int i = 0; i < PASSES; ++i) srow[i] = act8_scale(wave_max(m[i]));
    }
    // words of one row per 128 inputs: 16 (4-bit) or 8 (2-bit); per lane group 4 or 2
    constexpr int WPS = FOUR ? 16 : 8, LW = WPS / 4;
    const uint32_t* row = pw + (long)krc * (K / 128) * WPS + j * LW;
    i32x4 acc = {0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += A8_CHUNK) {
        // every weight load of this chunk first
        uint32_t w[8][LW];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if constexpr (FOUR) {
                const uint4 v = reinterpret_cast<const uint4*>(row + (long)(k0 / 128 + s) * WPS)[0];
                w[s][0] = v.x; w[s][1] = v.y; w[s][2] = v.z; w[s][3] = v.w;
            } else {
                const uint2 v = reinterpret_cast<const uint2*>(row + (long)(k0 / 128 + s) * WPS)[0];
                w[s][0] = v.x; w[s][1] = v.y;
            }
        }
        // this wave's rows, inputs k0 .. k0 + 1023 (one 16-input unit per lane)
        uint4 raw[PASSES][2];
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            raw[i][0] = reinterpret_cast<const uint4*>(xr[i] + k0)[0];
            raw[i][1] = reinterpret_cast<const uint4*>(xr[i] + k0)[1];
        }
        if (K == A8_CHUNK) {
#pragma unroll
            for (int i = 0; i < PASSES; ++i) srow[i] = act8_scale(wave_max(amax16(raw[i][0], raw[i][1])));
        }
        __syncthreads();   // the previous chunk's MFMAs are done with xl
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            int q[16];
            qsum[i] += codes16(raw[i][0], raw[i][1], srow[i], q);
            *reinterpret_cast<uint4*>(xl + (A8_WAVES * i + wave) * A8_PITCH + lane * 16) = FOUR ? order4(q) : order2(q);
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // inputs 128 s + 32 j + 16 h .. +15 of the chunk: 4-bit words 4j + 2h, +1;
                // 2-bit word 2j + h
                i32x4 bv;
                if constexpr (FOUR) {
                    const uint32_t a0 = w[s][2 * h], a1 = w[s][2 * h + 1];
                    bv = i32x4{(int)(a0 & 0x0F0F0F0Fu), (int)((a0 >> 4) & 0x0F0F0F0Fu),
                               (int)(a1 & 0x0F0F0F0Fu), (int)((a1 >> 4) & 0x0F0F0F0Fu)};
                } else {
                    const uint32_t a0 = w[s][h];
                    bv = i32x4{(int)(a0 & 0x03030303u), (int)((a0 >> 2) & 0x03030303u),
                               (int)((a0 >> 4) & 0x03030303u), (int)((a0 >> 6) & 0x03030303u)};
                }
                const i32x4 av = *reinterpret_cast<const i32x4*>(xl + col * A8_PITCH + 128 * s + 32 * j + 16 * h);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
            }
        }
    }
    // the rows' scales and code sums to LDS for the epilogue's lanes
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int tot = wave_sum_i(qsum[i]);
        if (lane == 0) { sx[A8_WAVES * i + wave] = srow[i]; ssum[A8_WAVES * i + wave] = tot; }
    }
    __syncthreads();
    if (kr >= kind_rows) return;
    const int n = FOUR ? kr * period : (kr / (period - 1)) * period + 1 + kr % (period - 1);
    const int off = FOUR ? 8 : 1;
    const float sw = h2f(scales[n]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * j + r;
        if (t < nt) y[(long)(t0 + t) * rows + n] = f2h(((float)(acc[r] - off * ssum[t]) * sx[t]) * sw);
    }
}

// Both channel kinds in one launch: blocks 0 .. nb4 - 1 take 4-bit rows, the rest ternary.
__global__ void __launch_bounds__(64 * A8_WAVES) k_sg_a8_mfma(const uint16_t* __restrict__ x, int nb, int K,
                                                    int rows, int period,
                                                    const uint32_t* __restrict__ p4,
                                                    const uint32_t* __restrict__ p2,
                                                    const uint16_t* __restrict__ scales,
                                                    uint16_t* __restrict__ y, int n4, int nb4) {
    __shared__ __align__(16) int8_t xl[16 * A8_PITCH];
    __shared__ float sx[16];
    __shared__ int ssum[16];
    if ((int)blockIdx.x < nb4)
        sg_a8_mfma_block<true>(x, nb, K, rows, period, p4, scales, y, n4, blockIdx.x, xl, sx, ssum);
    else
        sg_a8_mfma_block<false>(x, nb, K, rows, period, p2, scales, y, rows - n4, blockIdx.x - nb4,
                                xl, sx, ssum);
}

}  // namespace

hipError_t launch_quantize_act8(const uint16_t* x, int b, int cols, int8_t* qx, uint16_t* sx,
                                hipStream_t s) {
    k_act8_quantize<<<(unsigned)((b + 3) / 4), 256, 0, s>>>(x, b, cols, qx, sx);
    return hipGetLastError();
}

hipError_t launch_qlinear_supergroup_a8(const uint16_t* x, int b, const uint32_t* p4,
                                        const uint32_t* p2, const uint16_t* scales, int rows,
                                        int cols, int period, uint16_t* y, hipStream_t s) {
    if (b > A8_MT && cols % A8_CHUNK == 0) {   // batched: MFMA
        const int n4 = rows / period, n2 = rows - n4;
        constexpr int CPB = 16 * A8_WAVES;   // channels per block
        const int nb4 = (n4 + CPB - 1) / CPB, nb2 = (n2 + CPB - 1) / CPB;
        const dim3 g((unsigned)(nb4 + nb2), (unsigned)((b + 15) / 16));
        k_sg_a8_mfma<<<g, 64 * A8_WAVES, 0, s>>>(x, b, cols, rows, period, p4, p2, scales, y, n4, nb4);
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)std::max(1, std::min((rows + 3) / 4, 2048));
    k_sg_a8_gemv<<<blocks, 256, 0, s>>>(x, b, cols, rows, period, p4, p2, scales, y);
    return hipGetLastError();
}

}  // namespace qmoe
