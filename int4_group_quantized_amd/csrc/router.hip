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

namespace qmoe {

namespace {

constexpr int MAX_PER_LANE = 16;  // e <= 1024
constexpr int MAX_K = 32;

// One wave per token.  Lane l holds logits l, l+64, ...; K rounds of a wave-wide argmax
// (ties to the lower index), each removing the winner.
__global__ void __launch_bounds__(256) k_router_topk(const float* __restrict__ logits, int t, int e,
                                                     int k, const float* __restrict__ bias,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= t) return;
    float v[MAX_PER_LANE];
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < MAX_PER_LANE; ++i) {
        const int ei = lane + 64 * i;
        v[i] = 0.0f;
        if (ei < e) {
            v[i] = logits[(long)tok * e + ei] + (bias ? bias[ei] : 0.0f);
            live |= 1u << i;
        }
    }
    float sv[MAX_K];
    int si[MAX_K];
    for (int r = 0; r < k; ++r) {
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < MAX_PER_LANE; ++i)
            if (((live >> i) & 1u) && (bi < 0 || v[i] > bv)) { bv = v[i]; bi = lane + 64 * i; }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) live &= ~(1u << (bi >> 6));
        sv[r] = bv;
        si[r] = bi;
    }
    if (lane == 0) {
        const float m = sv[0];
        float sum = 0.0f;
        for (int r = 0; r < k; ++r) { sv[r] = expf(sv[r] - m); sum += sv[r]; }
        for (int r = 0; r < k; ++r) {
            idx[(long)tok * k + r] = si[r];
            wout[(long)tok * k + r] = sv[r] / sum;
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
