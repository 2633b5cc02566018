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

}  // namespace

hipError_t launch_qlinear_supergroup(const uint16_t* x, int b, const uint32_t* p4,
                                     const uint32_t* p2, const uint16_t* scales, int rows,
                                     int cols, int period, uint16_t* y, hipStream_t s) {
    const size_t smem = 32768 + (size_t)SG_MT * (cols / 32) * 4;
    const unsigned blocks = (unsigned)std::max(1, std::min((rows + 3) / 4, 2048));
    k_sg_gemv<<<blocks, 256, smem, s>>>(x, b, cols, rows, period, p4, p2, scales, y);
    return hipGetLastError();
}

}  // namespace qmoe
