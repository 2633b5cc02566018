// Affine group quantization, unpacking and dequantization; super-group quantization.
//
// Affine format ("Recover-LoRA ..." section 1; "Bit-exact MLX 4-bit port ..." section
// "4-bit group quantization"): per row and group of 64 (or 32) inputs one fp16 scale and
// one fp16 bias, codes in packed uint32 words (lowest field first); w = scale * q + bias.
// Super-group format ("EDGERAZOR deep dive" section 2.1): one 4-bit symmetric channel per
// block of `period` output channels, the others ternary.
//
// Every value that decides a code is computed with explicit IEEE float32 operations
// (__fsub_rn, __fdiv_rn, rintf = ties to even) on the stored fp16 parameters.  Offline
// work: clarity over speed, but every launch still covers the matrix with many waves.
#include "device.hpp"
#include "launch.hpp"

namespace qmoe {

// One thread per (row, group of G inputs).
template <int BITS, int G>
__global__ void __launch_bounds__(256) k_quantize_affine(const float* __restrict__ w,
                                                         long n_groups,
                                                         uint32_t* __restrict__ packed,
                                                         uint16_t* __restrict__ scales,
                                                         uint16_t* __restrict__ biases) {
    const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_groups) return;
    const float4* src = reinterpret_cast<const float4*>(w + g * G);
    float v[G];
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
        float4 t = src[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 1; i < G; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
    constexpr float top = BITS == 4 ? 15.0f : 255.0f;
    const f16 sh = (f16)__fdiv_rn(__fsub_rn(hi, lo), top);
    const f16 bh = (f16)lo;
    const float s = (float)sh, b = (float)bh;
    constexpr int PER = 32 / BITS;          // codes per word
    constexpr int NW = G / PER;             // words per group
    uint32_t words[NW];
#pragma unroll
    for (int m = 0; m < NW; ++m) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            float q = 0.0f;
            if (s != 0.0f) q = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(v[m * PER + j], b), s)), 0.0f), top);
            word |= (uint32_t)q << (BITS * j);
        }
        words[m] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(packed + g * NW);
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) dst[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    scales[g] = __builtin_bit_cast(uint16_t, sh);
    biases[g] = __builtin_bit_cast(uint16_t, bh);
}

hipError_t launch_quantize_affine(const float* w, int rows, int cols, int bits, int group,
                                  uint32_t* packed, uint16_t* scales, uint16_t* biases,
                                  hipStream_t s) {
    const long n_groups = (long)rows * (cols / group);
    const unsigned blocks = (unsigned)((n_groups + 255) / 256);
    if (group == 32) {
        if (bits == 4) k_quantize_affine<4, 32><<<blocks, 256, 0, s>>>(w, n_groups, packed, scales, biases);
        else k_quantize_affine<8, 32><<<blocks, 256, 0, s>>>(w, n_groups, packed, scales, biases);
    } else {
        if (bits == 4) k_quantize_affine<4, 64><<<blocks, 256, 0, s>>>(w, n_groups, packed, scales, biases);
        else k_quantize_affine<8, 64><<<blocks, 256, 0, s>>>(w, n_groups, packed, scales, biases);
    }
    return hipGetLastError();
}

// One thread per word: its codes as bytes.
template <int BITS>
__global__ void __launch_bounds__(256) k_unpack(const uint32_t* __restrict__ packed, long n_words,
                                                uint8_t* __restrict__ q) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_words) return;
    const uint32_t w = packed[i];
    if constexpr (BITS == 4) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= ((w >> (4 * j)) & 0xFu) << (8 * j);
            hi |= ((w >> (4 * j + 16)) & 0xFu) << (8 * j);
        }
        reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
    } else {
        reinterpret_cast<uint32_t*>(q)[i] = w;   // bytes are already the codes
    }
}

hipError_t launch_unpack(const uint32_t* packed, long n_words, int bits, uint8_t* q,
                         hipStream_t s) {
    const unsigned blocks = (unsigned)((n_words + 255) / 256);
    if (bits == 4) k_unpack<4><<<blocks, 256, 0, s>>>(packed, n_words, q);
    else k_unpack<8><<<blocks, 256, 0, s>>>(packed, n_words, q);
    return hipGetLastError();
}

// One thread per word: fp32(s * q + b) with one rounding (fmaf of an exact product); the
// parameters fp16 or bf16 (bf16 of the port page's checkpoint), the group 64 or 32.
template <int BITS>
__global__ void __launch_bounds__(256) k_dequantize(const uint32_t* __restrict__ packed,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ biases,
                                                    long n_words, int group, int bf16,
                                                    float* __restrict__ out) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_words) return;
    constexpr int PER = 32 / BITS;
    const long grp = i / (group / PER);   // words of a group are consecutive
    const float sc = bf16 ? bf2f(scales[grp]) : h2f(scales[grp]);
    const float bi = bf16 ? bf2f(biases[grp]) : h2f(biases[grp]);
    const uint32_t w = packed[i];
    float r[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) r[j] = fmaf(sc, (float)((w >> (BITS * j)) & ((1u << BITS) - 1)), bi);
    float4* dst = reinterpret_cast<float4*>(out + i * PER);
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) dst[j] = make_float4(r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]);
}

hipError_t launch_dequantize(const qmoe_qweight& w, float* out, hipStream_t s) {
    const long n_words = (long)w.n_experts * w.rows * (w.cols * w.bits / 32);
    const unsigned blocks = (unsigned)((n_words + 255) / 256);
    const int bf = w.param_dtype == QMOE_PARAM_BF16;
    if (w.bits == 4) k_dequantize<4><<<blocks, 256, 0, s>>>(w.packed, w.scales, w.biases, n_words, w.group, bf, out);
    else k_dequantize<8><<<blocks, 256, 0, s>>>(w.packed, w.scales, w.biases, n_words, w.group, bf, out);
    return hipGetLastError();
}

// Super-group quantization: one wave per output channel.  Lane l owns the 16-input units
// u = l, l + 64, ... of the channel (a unit is one ternary word or two 4-bit words).
__global__ void __launch_bounds__(256) k_quantize_supergroup(const float* __restrict__ w, int rows,
                                                             int cols, int period,
                                                             uint32_t* __restrict__ p4,
                                                             uint32_t* __restrict__ p2,
                                                             uint16_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= rows) return;
    const bool four = (n % period) == 0;
    const float* row = w + (long)n * cols;
    const int units = cols / 16;
    double asum = 0.0;
    float amax = 0.0f;
    for (int u = lane; u < units; u += 64) {
        const float4* src = reinterpret_cast<const float4*>(row + u * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 t = src[i];
            asum += (double)fabsf(t.x) + (double)fabsf(t.y) + (double)fabsf(t.z) + (double)fabsf(t.w);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        asum += __shfl_xor(asum, off, 64);
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    }
    float s32;
    float qmax;
    if (four) {
        s32 = fmaxf(__fdiv_rn(amax, 7.0f), 1e-5f);
        qmax = 7.0f;
    } else {
        const float mean = (float)(asum / (double)cols);
        s32 = fmaxf(2.0f * mean, 1e-5f);
        qmax = 1.0f;
    }
    const f16 sh = (f16)s32;
    const float sc = (float)sh;
    if (lane == 0) scales[n] = __builtin_bit_cast(uint16_t, sh);
    // row index inside its packed array (channel order within each kind)
    const int blk = n / period, pos = n % period;
    for (int u = lane; u < units; u += 64) {
        const float4* src = reinterpret_cast<const float4*>(row + u * 16);
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 t = src[i];
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
        int q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = (int)fminf(fmaxf(rintf(__fdiv_rn(v[i], sc)), -qmax), qmax);
        if (four) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                w0 |= (uint32_t)(q[j] + 8) << (4 * j);
                w1 |= (uint32_t)(q[j + 8] + 8) << (4 * j);
            }
            uint32_t* dst = p4 + (long)blk * (cols / 8) + u * 2;
            dst[0] = w0;
            dst[1] = w1;
        } else {
            uint32_t w0 = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) w0 |= (uint32_t)(q[j] + 1) << (2 * j);
            const long r2 = (long)blk * (period - 1) + (pos - 1);
            p2[r2 * (cols / 16) + u] = w0;
        }
    }
}

hipError_t launch_quantize_supergroup(const float* w, int rows, int cols, int period,
                                      uint32_t* p4, uint32_t* p2, uint16_t* scales,
                                      hipStream_t s) {
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    k_quantize_supergroup<<<blocks, 256, 0, s>>>(w, rows, cols, period, p4, p2, scales);
    return hipGetLastError();
}

}  // namespace qmoe
