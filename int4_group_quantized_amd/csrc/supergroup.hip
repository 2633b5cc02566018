// Mixed ternary / 4-bit super-group weight-only GEMM: y[b][n] = fp16(s_n * sum_k q[n][k] x[b][k]).
//
// "EDGERAZOR deep dive" (zhichai.net) section 2.1 SQMP: in every block of floor(1/rho)
// consecutive output channels exactly one is 4-bit (symmetric, q in [-7, 7]) and the others
// ternary (q in {-1, 0, 1}); the matmul factors into a scale product and an integer dot
// product, so the per-channel scale is applied once after the sum over k.
//
// Codes become exact fp16 values in registers as in the affine kernels: a 4-bit field
// c = q + 8 gives 1 + c/16, a 2-bit field c = q + 1 gives 1 + c/4; with dot = sum((1 + c/C) x)
// and X = sum(x): sum(q x) = C dot - (C + off) X, off = 8 (4-bit) or 1 (ternary).
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace qmoe {

namespace {

constexpr int SG_MT = 8;

// 2-bit word: fields c0..c15 (c_j in bits [2j, 2j+2)).  Pair j in 0..7 = (1 + c_j/4,
// 1 + c_{j+8}/4): field j moved to mantissa bits 8..9 of each half.
template <int J>
__device__ __forceinline__ uint32_t tern_pair(uint32_t w) {
    constexpr int sh = 8 - 2 * J;
    const uint32_t s = sh >= 0 ? (w << sh) : (w >> (-sh));
    return (s & 0x03000300u) | 0x3C003C00u;
}

__device__ __forceinline__ float dot_word2(uint32_t w, const f16x2* xp, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<0>(w)), xp[0], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<1>(w)), xp[1], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<2>(w)), xp[2], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<3>(w)), xp[3], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<4>(w)), xp[4], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<5>(w)), xp[5], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<6>(w)), xp[6], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(tern_pair<7>(w)), xp[7], acc, false);
    return acc;
}

// One wave per output channel.  x for up to SG_MT tokens is staged in LDS twice: in the
// pair order of 4-bit words (x4) and of 2-bit words (x2), plus sums per 32 inputs.
__global__ void __launch_bounds__(256) k_sg_gemv(const uint16_t* __restrict__ x, int nb, int K,
                                                 int rows, int period,
                                                 const uint32_t* __restrict__ p4,
                                                 const uint32_t* __restrict__ p2,
                                                 const uint16_t* __restrict__ scales,
                                                 uint16_t* __restrict__ y) {
    extern __shared__ __align__(16) char smem[];
    const int mt_max = min(SG_MT, 16384 / (K * 2));
    f16x2* x4 = reinterpret_cast<f16x2*>(smem);                  // [mt][K/2]
    f16x2* x2 = reinterpret_cast<f16x2*>(smem + 16384);          // [mt][K/2]
    float* xsum = reinterpret_cast<float*>(smem + 32768);        // [mt][K/32]
    const int lane = threadIdx.x & 63;
    const int wave_global = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n_waves = gridDim.x * 4;
    for (int t0 = 0; t0 < nb; t0 += mt_max) {
        const int mt = min(mt_max, nb - t0);
        __syncthreads();
        for (int u = threadIdx.x; u < mt * (K / 16); u += blockDim.x) {
            const int t = u / (K / 16), c = u % (K / 16);
            const uint4* src = reinterpret_cast<const uint4*>(x + (long)(t0 + t) * K + c * 16);
            const uint4 r0 = src[0], r1 = src[1];
            f16 h[16];
            *reinterpret_cast<uint4*>(h) = r0;
            *reinterpret_cast<uint4*>(h + 8) = r1;
            f16x2* d4 = x4 + (long)t * (K / 2) + c * 8;
            pair_perm8(h, d4);
            pair_perm8(h + 8, d4 + 4);
            f16x2* d2 = x2 + (long)t * (K / 2) + c * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) d2[j] = f16x2{h[j], h[j + 8]};
        }
        for (int u = threadIdx.x; u < mt * (K / 32); u += blockDim.x) {
            const int t = u / (K / 32), c = u % (K / 32);
            const uint16_t* src = x + (long)(t0 + t) * K + c * 32;
            float s = 0.0f;
            for (int i = 0; i < 32; ++i) s += h2f(src[i]);
            xsum[t * (K / 32) + c] = s;
        }
        __syncthreads();
        for (int n = wave_global; n < rows; n += n_waves) {
            const bool four = (n % period) == 0;
            const int blk = n / period, pos = n % period;
            float acc[SG_MT];
#pragma unroll
            for (int t = 0; t < SG_MT; ++t) acc[t] = 0.0f;
            if (four) {
                const uint4* row = reinterpret_cast<const uint4*>(p4 + (long)blk * (K / 8));
                for (int c = lane; c < K / 32; c += 64) {       // chunk = 4 words = 32 inputs
                    const uint4 v = row[c];
                    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int t = 0; t < SG_MT; ++t) {
                        if (t < mt) {
                            const f16x2* xp = x4 + (long)t * (K / 2) + c * 16;
                            float d = 0.0f;
#pragma unroll
                            for (int j = 0; j < 4; ++j) d = dot_word4(wd[j], xp + 4 * j, d);
                            acc[t] = fmaf(16.0f, d, fmaf(-24.0f, xsum[t * (K / 32) + c], acc[t]));
                        }
                    }
                }
            } else {
                const long r2 = (long)blk * (period - 1) + (pos - 1);
                const uint4* row = reinterpret_cast<const uint4*>(p2 + r2 * (K / 16));
                for (int c = lane; c < K / 64; c += 64) {       // chunk = 4 words = 64 inputs
                    const uint4 v = row[c];
                    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int t = 0; t < SG_MT; ++t) {
                        if (t < mt) {
                            const f16x2* xp = x2 + (long)t * (K / 2) + c * 32;
                            float d = 0.0f;
#pragma unroll
                            for (int j = 0; j < 4; ++j) d = dot_word2(wd[j], xp + 8 * j, d);
                            const float X = xsum[t * (K / 32) + 2 * c] + xsum[t * (K / 32) + 2 * c + 1];
                            acc[t] = fmaf(4.0f, d, fmaf(-5.0f, X, acc[t]));
                        }
                    }
                }
            }
            const float sc = h2f(scales[n]);
#pragma unroll
            for (int t = 0; t < SG_MT; ++t) {
                if (t < mt) {
                    const float v = seg_sum<64>(acc[t]);
                    if (lane == 0) y[(long)(t0 + t) * rows + n] = f2h(sc * v);
                }
            }
        }
    }
}

// ---- batched form: fp16 MFMA over exact integer codes ------------------------------------
//
// v_mfma_f32_16x16x32_f16 with the tokens as A (16 x 32 inputs, from LDS) and the codes as B
// (32 inputs x 16 channels, in registers).  The codes are exact signed fp16 integers (the
// field under the exponent of 1024, minus 1024 + offset), so the MFMA accumulates
// sum_k q x exactly per product in fp32 over the whole row, and the channel's scale is
// applied once at the end.  A block holds 64 channels of one kind (4-bit or ternary) and 16
// tokens; the tokens' x is staged per 1024 inputs in the pair order of that kind, and every
// weight load of a lane for those 1024 inputs is issued before the first MFMA.

constexpr int SG_CHUNK = 1024;              // inputs staged per pass
constexpr int SG_PITCH = SG_CHUNK + 8;      // LDS row pitch (halves)

template <bool FOUR>
__device__ __forceinline__ void sg_mfma_block(const uint16_t* __restrict__ x, int nb, int K,
                                              int rows, int period,
                                              const uint32_t* __restrict__ pw,
                                              const uint16_t* __restrict__ scales,
                                              uint16_t* __restrict__ y, int kind_rows, int rb,
                                              f16* xl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, j = lane >> 4;
    const int kr = rb * 64 + wave * 16 + col;                  // this lane's row of its kind
    const int krc = min(kr, kind_rows - 1);
    const int t0 = blockIdx.y * 16;
    const int nt = min(16, nb - t0);
    // words of one row per 128 inputs: 16 (4-bit) or 8 (ternary); per lane group 4 or 2
    constexpr int WPS = FOUR ? 16 : 8, LW = WPS / 4;
    const uint32_t* row = pw + (long)krc * (K / 128) * WPS + j * LW;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += SG_CHUNK) {
        // every weight load of this chunk first
        uint32_t w[8][LW];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if constexpr (FOUR) {
                const uint4 v = reinterpret_cast<const uint4*>(row + (long)(k0 / 128 + ks) * WPS)[0];
                w[ks][0] = v.x; w[ks][1] = v.y; w[ks][2] = v.z; w[ks][3] = v.w;
            } else {
                const uint2 v = reinterpret_cast<const uint2*>(row + (long)(k0 / 128 + ks) * WPS)[0];
                w[ks][0] = v.x; w[ks][1] = v.y;
            }
        }
        // stage the 16 tokens' inputs k0 .. k0 + 1023 in the pair order of this kind, every
        // load of a thread issued before its first LDS write
        constexpr int PASSES = 16 * (SG_CHUNK / 16) / 256;
        uint4 raw[PASSES][2];
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int u = i * 256 + threadIdx.x;
            const int r = u / (SG_CHUNK / 16), c = u % (SG_CHUNK / 16);
            const uint4* src = reinterpret_cast<const uint4*>(x + (long)(t0 + min(r, nt - 1)) * K + k0 + c * 16);
            raw[i][0] = src[0];
            raw[i][1] = src[1];
        }
        if (k0 > 0) __syncthreads();
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int u = i * 256 + threadIdx.x;
            const int r = u / (SG_CHUNK / 16), c = u % (SG_CHUNK / 16);
            f16 h[16];
            *reinterpret_cast<uint4*>(h) = raw[i][0];
            *reinterpret_cast<uint4*>(h + 8) = raw[i][1];
            f16x2 p[8];
            if constexpr (FOUR) {
                pair_perm8(h, p);
                pair_perm8(h + 8, p + 4);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) p[q] = f16x2{h[q], h[q + 8]};
            }
            uint4* dst = reinterpret_cast<uint4*>(xl + r * SG_PITCH + c * 16);
            dst[0] = __builtin_bit_cast(uint4, *reinterpret_cast<f16x2(*)[4]>(p));
            dst[1] = __builtin_bit_cast(uint4, *reinterpret_cast<f16x2(*)[4]>(p + 4));
        }
        __syncthreads();
        const f16x2 off = FOUR ? f16x2{(f16)1032.0f, (f16)1032.0f} : f16x2{(f16)1025.0f, (f16)1025.0f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // codes of MFMA slice m: 4-bit word m, pairs (q_p, q_p+4); ternary word m/2,
                // pairs 4 (m % 2) .. +3 of (q_p, q_p+8)
                f16x2 c[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t f;
                    if constexpr (FOUR) f = ((w[ks][m] >> (4 * q)) & 0x000F000Fu) | 0x64006400u;
                    else f = ((w[ks][m >> 1] >> (2 * (4 * (m & 1) + q))) & 0x00030003u) | 0x64006400u;
                    c[q] = as_h2(f) - off;
                }
                const f16x8 bv = f16x8{c[0][0], c[0][1], c[1][0], c[1][1], c[2][0], c[2][1], c[3][0], c[3][1]};
                const f16x8 av = *reinterpret_cast<const f16x8*>(xl + col * SG_PITCH + ks * 128 + 32 * j + 8 * m);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
            }
        }
    }
    if (kr >= kind_rows) return;
    const int n = FOUR ? kr * period : (kr / (period - 1)) * period + 1 + kr % (period - 1);
    const float sc = h2f(scales[n]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * j + r;
        if (t < nt) y[(long)(t0 + t) * rows + n] = f2h(sc * acc[r]);
    }
}

// Both channel kinds in one launch: blocks 0 .. nb4 - 1 take 4-bit rows, the rest ternary.
__global__ void __launch_bounds__(256) k_sg_mfma(const uint16_t* __restrict__ x, int nb, int K,
                                                 int rows, int period,
                                                 const uint32_t* __restrict__ p4,
                                                 const uint32_t* __restrict__ p2,
                                                 const uint16_t* __restrict__ scales,
                                                 uint16_t* __restrict__ y, int n4, int nb4) {
    __shared__ __align__(16) f16 xl[16 * SG_PITCH];
    if ((int)blockIdx.x < nb4)
        sg_mfma_block<true>(x, nb, K, rows, period, p4, scales, y, n4, blockIdx.x, xl);
    else
        sg_mfma_block<false>(x, nb, K, rows, period, p2, scales, y, rows - n4, blockIdx.x - nb4, xl);
}

}  // namespace

hipError_t launch_qlinear_supergroup(const uint16_t* x, int b, const uint32_t* p4,
                                     const uint32_t* p2, const uint16_t* scales, int rows,
                                     int cols, int period, uint16_t* y, hipStream_t s) {
    if (b > SG_MT && cols % SG_CHUNK == 0) {   // batched: MFMA
        const int n4 = rows / period, n2 = rows - n4;
        const int nb4 = (n4 + 63) / 64, nb2 = (n2 + 63) / 64;
        const dim3 g((unsigned)(nb4 + nb2), (unsigned)((b + 15) / 16));
        k_sg_mfma<<<g, 256, 0, s>>>(x, b, cols, rows, period, p4, p2, scales, y, n4, nb4);
        return hipGetLastError();
    }
    const size_t smem = 32768 + (size_t)SG_MT * (cols / 32) * 4;
    const unsigned blocks = (unsigned)std::max(1, std::min((rows + 3) / 4, 2048));
    k_sg_gemv<<<blocks, 256, smem, s>>>(x, b, cols, rows, period, p4, p2, scales, y);
    return hipGetLastError();
}

}  // namespace qmoe
