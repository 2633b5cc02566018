// Top-K routing on given logits: the K largest (ties to the lower expert index) and the
// softmax renormalized over the selected K.
//
// Routing family SOFTMAX_TOPK ("Edge0 project review", MoE spec), K = 4 of 256 experts
// ("Recover-LoRA ..." section 1).  Softmax is strictly increasing, so the top-K of the
// probabilities is the top-K of the logits; selecting on the fp32 logits keeps rounded
// probabilities from creating ties.  Indices stay on the device ("Edge0 project review",
// highlight 2).
#include "device.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace qmoe {

namespace {

constexpr int MAX_K = 32;

// One wave per token; lane 0 writes the selection.
__global__ void __launch_bounds__(256) k_router_topk(const float* __restrict__ logits, int t, int e,
                                                     int k, const float* __restrict__ bias,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout) {
    __shared__ int sel[4][MAX_K];
    __shared__ float sw[4][MAX_K];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tok = blockIdx.x * 4 + wave;
    if (tok >= t) return;
    wave_topk(logits + (long)tok * e, bias, e, k, sel[wave], sw[wave]);
    if (lane == 0) {
        for (int r = 0; r < k; ++r) {
            idx[(long)tok * k + r] = sel[wave][r];
            wout[(long)tok * k + r] = sw[wave][r];
        }
    }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int t, int e, int k, const float* bias,
                              int32_t* idx, float* weights, hipStream_t s) {
    const unsigned blocks = (unsigned)((t + 3) / 4);
    k_router_topk<<<blocks, 256, 0, s>>>(logits, t, e, k, bias, idx, weights);
    return hipGetLastError();
}

}  // namespace qmoe
