// Unmerged LoRA delta accumulated into an fp32 output: y += scale * B_a (A_a x).
//
// "Recover-LoRA ..." section 2 and "Edge0 project review" highlight 3: the adapter is a
// parallel delta on a frozen, read-only quantized base, never merged, so one base serves
// many adapter sets; each token picks its adapter by index.
#include "device.hpp"
#include "launch.hpp"

namespace qmoe {

namespace {

constexpr int MAX_RANK = 64;

// Grid (out-blocks of 256 outputs, tokens).  Each block recomputes z = A_a x for its token
// (rank dot products, one wave each, 128-bit loads), then each thread adds one output.
__global__ void __launch_bounds__(256) k_lora_apply(const uint16_t* __restrict__ x, int in_dim,
                                                    int out_dim, const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ B, int rank, int n_ad,
                                                    float scale,
                                                    const int32_t* __restrict__ adapter_idx,
                                                    float* __restrict__ y) {
    __shared__ float z[MAX_RANK];
    const int tok = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int a = adapter_of(adapter_idx, tok, n_ad);
    const uint16_t* xrow = x + (long)tok * in_dim;
    for (int r = wave; r < rank; r += 4) {
        const uint16_t* arow = A + ((long)a * rank + r) * in_dim;
        float acc = 0.0f;
        for (int k = lane * 8; k < in_dim; k += 512) {
            const uint4 av = *reinterpret_cast<const uint4*>(arow + k);
            const uint4 xv = *reinterpret_cast<const uint4*>(xrow + k);
            const f16x2* ah = reinterpret_cast<const f16x2*>(&av);
            const f16x2* xh = reinterpret_cast<const f16x2*>(&xv);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ah[i], xh[i], acc, false);
        }
        acc = seg_sum<64>(acc);
        if (lane == 0) z[r] = acc;
    }
    __syncthreads();
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= out_dim) return;
    const uint16_t* brow = B + ((long)a * out_dim + n) * rank;
    float d = 0.0f;
    for (int r = 0; r < rank; ++r) d = fmaf(h2f(brow[r]), z[r], d);
    y[(long)tok * out_dim + n] = fmaf(scale, d, y[(long)tok * out_dim + n]);
}

}  // namespace

hipError_t launch_lora_apply(const uint16_t* x, int t, const qmoe_lora& l,
                             const int32_t* adapter_idx, float* y_acc, hipStream_t s) {
    dim3 grid((unsigned)((l.out_dim + 255) / 256), (unsigned)t);
    k_lora_apply<<<grid, 256, 0, s>>>(x, l.in_dim, l.out_dim, l.A, l.B, l.rank, l.n_adapters, l.scale,
                                      adapter_idx, y_acc);
    return hipGetLastError();
}

}  // namespace qmoe
