// Quantized linear for a few tokens: y = fp16(x W^T + LoRA delta), fp32 accumulation.
//
// Every linear layer of the checkpoint is stored as packed integer words plus one fp16
// scale and one fp16 bias per group of 64 inputs (the port page's QAT checkpoint: bf16
// parameters per 32 inputs, also served here) and is dequantized on the fly
// ("Recover-LoRA ..." section 1; "Bit-exact MLX 4-bit port ..." "4-bit group
// quantization"); the recovery LoRA is added as an unmerged parallel delta ("Recover-LoRA"
// section 2; "Edge0 project review" highlight 3).
//
// Decode is bandwidth-bound: rows are streamed with 128-bit loads by lane segments
// (gemv_core.hpp), x is staged once per block in LDS in the pair order of the unpacking.
#include <algorithm>

#include "gemv_core.hpp"
#include "launch.hpp"

namespace qmoe {

namespace {

constexpr int MAX_RANK = 64;
constexpr int XS_BYTES = 32768;  // LDS for staged x: tokens per pass * K * 2 <= this

// z[t][r] = A[a_t][r] . x[t] for tokens [t0, t0+mt) (one wave per (t, r) pair).
__device__ void lora_down_block(const uint16_t* __restrict__ x, int K, int t0, int mt,
                                const uint16_t* __restrict__ A, int rank,
                                const int32_t* __restrict__ adapter_idx, int n_ad, float* zl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int p = wave; p < mt * rank; p += nw) {
        const int t = p / rank, r = p % rank;
        const int a = adapter_of(adapter_idx, t0 + t, n_ad);
        const uint16_t* arow = A + ((long)a * rank + r) * K;
        const uint16_t* xrow = x + (long)(t0 + t) * K;
        float acc = 0.0f;
        for (int k = lane * 8; k < K; k += 512) {
            const uint4 av = *reinterpret_cast<const uint4*>(arow + k);
            const uint4 xv = *reinterpret_cast<const uint4*>(xrow + k);
            const f16x2* ah = reinterpret_cast<const f16x2*>(&av);
            const f16x2* xh = reinterpret_cast<const f16x2*>(&xv);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ah[i], xh[i], acc, false);
        }
        acc = seg_sum<64>(acc);
        if (lane == 0) zl[t * MAX_RANK + r] = acc;
    }
}

template <int BITS, int G, bool BF>
__global__ void __launch_bounds__(256) k_qgemv(const uint16_t* __restrict__ x, int m, int K, int N,
                                               const uint32_t* __restrict__ packed,
                                               const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases,
                                               const uint16_t* __restrict__ loraA,
                                               const uint16_t* __restrict__ loraB, int rank, int n_ad,
                                               float lscale, const int32_t* __restrict__ adapter_idx,
                                               uint16_t* __restrict__ y, int mt_max) {
    extern __shared__ __align__(16) char smem[];
    f16x2* xs = reinterpret_cast<f16x2*>(smem);                        // [mt_max][K/2]
    float* xsum = reinterpret_cast<float*>(smem + XS_BYTES);            // [GEMV_MT][K/32]
    float* zl = xsum + GEMV_MT * (K / 32);                              // [GEMV_MT][MAX_RANK]
    __shared__ int rows[GEMV_MT];

    const int lane = threadIdx.x & 63;
    const int wave_global = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int n_waves = gridDim.x * (blockDim.x >> 6);
    const int lpr = lanes_per_row(K);
    const int rpw = 64 / lpr;
    const int seg = lane / lpr, sl = lane % lpr;

    for (int t0 = 0; t0 < m; t0 += mt_max) {
        const int mt = min(mt_max, m - t0);
        __syncthreads();
        if (threadIdx.x < GEMV_MT) rows[threadIdx.x] = t0 + threadIdx.x;
        __syncthreads();
        stage_tokens<BITS>(x, rows, mt, K, xs, xsum);
        if (loraA) lora_down_block(x, K, t0, mt, loraA, rank, adapter_idx, n_ad, zl);
        __syncthreads();

        for (int rb = wave_global * rpw; rb < N; rb += n_waves * rpw) {
            const int row = rb + seg;
            float acc[GEMV_MT];
#pragma unroll
            for (int t = 0; t < GEMV_MT; ++t) acc[t] = 0.0f;
            if (row < N) qdot_row<BITS, G, BF>(packed, scales, biases, K, row, lpr, sl, xs, xsum, mt, acc);
#pragma unroll
            for (int t = 0; t < GEMV_MT; ++t) {
                if (t < mt) {
                    float v = segment_sum(acc[t], lpr);
                    if (sl == 0 && row < N) {
                        if (loraB) {
                            const int a = adapter_of(adapter_idx, t0 + t, n_ad);
                            const uint16_t* brow = loraB + ((long)a * N + row) * rank;
                            float d = 0.0f;
                            for (int r = 0; r < rank; ++r) d = fmaf(h2f(brow[r]), zl[t * MAX_RANK + r], d);
                            v = fmaf(lscale, d, v);
                        }
                        y[(long)(t0 + t) * N + row] = f2h(v);
                    }
                }
            }
        }
    }
}

// Fast path (no LoRA, m <= 8, at most two 32-input chunks per lane): each lane segment's
// weight loads are issued first, then x is staged, so the two memory round trips overlap.
template <int BITS, int G, bool BF>
__global__ void __launch_bounds__(256) k_qgemv_fast(const uint16_t* __restrict__ x, int m, int K,
                                                    int N, const uint32_t* __restrict__ packed,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ biases,
                                                    uint16_t* __restrict__ y) {
    extern __shared__ __align__(16) char smem[];
    asm volatile("" ::"s"(x), "s"(packed), "s"(scales), "s"(biases));   // args in one batch
    asm volatile("" ::"s"(y), "s"(m), "s"(K), "s"(N));
    f16x2* xs = reinterpret_cast<f16x2*>(smem);                        // [m][K/2]
    float* xsum = reinterpret_cast<float*>(smem + XS_BYTES);            // [m][K/32]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = lanes_per_row(K), rpw = 64 / lpr, seg = lane / lpr, sl = lane % lpr;
    const int row = (blockIdx.x * 4 + wave) * rpw + seg;
    RowRegs<BITS, 2, G, BF> rr;
    rr.load(packed, scales, biases, K, row < N ? row : 0, lpr, sl, row < N);
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    stage_rows<BITS, 8>([=](int i) { return x4 + (long)i * (K / 8); }, m, K, xs, xsum);
    __syncthreads();
    float acc[GEMV_MT];
#pragma unroll
    for (int t = 0; t < GEMV_MT; ++t) acc[t] = 0.0f;
    rr.dot(K, lpr, sl, xs, xsum, m, acc);
#pragma unroll
    for (int t = 0; t < GEMV_MT; ++t) {
        if (t < m) {
            const float v = segment_sum(acc[t], lpr);
            if (sl == 0 && row < N) y[(long)t * N + row] = f2h(v);
        }
    }
}

template <int BITS, int G, bool BF>
hipError_t launch_gemv_t(const uint16_t* x, int m, const qmoe_qweight& w, const qmoe_lora* lora,
                         const int32_t* adapter_idx, uint16_t* y, hipStream_t s) {
    const int K = w.cols, N = w.rows;
    const int rpw = 64 / lanes_per_row(K);
    const int mt_max = std::min(GEMV_MT, XS_BYTES / (K * 2));
    const size_t smem = (size_t)XS_BYTES + (size_t)GEMV_MT * (K / 32) * 4 + (size_t)GEMV_MT * MAX_RANK * 4;
    const int wave_rows = (N + rpw - 1) / rpw;
    const unsigned blocks = (unsigned)std::max(1, std::min((wave_rows + 3) / 4, 2048));
    const int cpl = (K / 32) / lanes_per_row(K);
    if (!lora && m <= mt_max && cpl <= 2 && m * (K / 8) <= 256 * 8) {
        const unsigned fb = (unsigned)((N + 4 * rpw - 1) / (4 * rpw));
        k_qgemv_fast<BITS, G, BF><<<fb, 256, smem, s>>>(x, m, K, N, w.packed, w.scales, w.biases, y);
        return hipGetLastError();
    }
    const uint16_t* A = lora ? lora->A : nullptr;
    const uint16_t* B = lora ? lora->B : nullptr;
    const int rank = lora ? lora->rank : 0;
    const int n_ad = lora ? lora->n_adapters : 1;
    const float ls = lora ? lora->scale : 0.0f;
    k_qgemv<BITS, G, BF><<<blocks, 256, smem, s>>>(x, m, K, N, w.packed, w.scales, w.biases, A, B, rank,
                                                  n_ad, ls, adapter_idx, y, mt_max);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_gemv_bits(const uint16_t* x, int m, const qmoe_qweight& w, const qmoe_lora* lora,
                            const int32_t* adapter_idx, uint16_t* y, hipStream_t s) {
    const bool bf = w.param_dtype == QMOE_PARAM_BF16;
    if (w.group == 32)
        return bf ? launch_gemv_t<BITS, 32, true>(x, m, w, lora, adapter_idx, y, s)
                  : launch_gemv_t<BITS, 32, false>(x, m, w, lora, adapter_idx, y, s);
    return bf ? launch_gemv_t<BITS, 64, true>(x, m, w, lora, adapter_idx, y, s)
              : launch_gemv_t<BITS, 64, false>(x, m, w, lora, adapter_idx, y, s);
}

}  // namespace

hipError_t launch_qlinear_gemv(const uint16_t* x, int m, const qmoe_qweight& w,
                               const qmoe_lora* lora, const int32_t* adapter_idx,
                               uint16_t* y, hipStream_t s) {
    return w.bits == 4 ? launch_gemv_bits<4>(x, m, w, lora, adapter_idx, y, s)
                       : launch_gemv_bits<8>(x, m, w, lora, adapter_idx, y, s);
}

}  // namespace qmoe
