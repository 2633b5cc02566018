// Top-K of one token's logits inside one wave, without LDS round trips.
//
// Routing family SOFTMAX_TOPK with K experts per token ("Edge0 project review" MoE spec;
// "Recover-LoRA ..." section 1).  The K largest of (logit + bias) are chosen in K rounds of
// a wave-wide maximum over 64-bit keys (order-preserving float bits above the inverted
// expert index, so an exact tie goes to the lower index); the reduction runs on DPP lane
// moves within 16-lane rows and scalar readlanes across rows.  The weights are the softmax
// over the K chosen logits (the full softmax renormalized over the selection).
#pragma once

#include "device.hpp"

namespace qmoe {

__device__ __forceinline__ uint32_t order_bits(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits(uint32_t k) {
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool key_gt(uint32_t ah, uint32_t al, uint32_t bh, uint32_t bl) {
    return ah > bh || (ah == bh && al > bl);
}
template <int CTRL>
__device__ __forceinline__ void key_max_dpp(uint32_t& h, uint32_t& l) {
    const uint32_t oh = dpp_u<CTRL>(h), ol = dpp_u<CTRL>(l);
    if (key_gt(oh, ol, h, l)) { h = oh; l = ol; }
}

// The token's logits held by this lane: entries lane*PER .. lane*PER + PER - 1 of the row;
// entries >= e are not candidates.  VEC: the row is 16-byte aligned and padded to a
// multiple of 64 floats, so every lane reads its PER entries with vector loads; otherwise
// each entry is read on its own (index clamped into the row).
template <int PER, bool VEC = true>
struct TopkKeys {
    float raw[PER], braw[PER];   // logit and bias; combined only in select()
    bool has_bias;
    __device__ __forceinline__ void load(const float* __restrict__ v, const float* __restrict__ bias,
                                         int e) {
        const int lane = threadIdx.x & 63;
        has_bias = bias != nullptr;
        if constexpr (!VEC) {
#pragma unroll
            for (int i = 0; i < PER; ++i) raw[i] = v[min(lane * PER + i, e - 1)];
        } else if constexpr (PER >= 4) {
#pragma unroll
            for (int i = 0; i < PER; i += 4) {
                const float4 q = reinterpret_cast<const float4*>(v + lane * PER)[i / 4];
                raw[i] = q.x; raw[i + 1] = q.y; raw[i + 2] = q.z; raw[i + 3] = q.w;
            }
        } else if constexpr (PER == 2) {
            const float2 q = reinterpret_cast<const float2*>(v)[lane];
            raw[0] = q.x; raw[1] = q.y;
        } else {
            raw[0] = v[lane];
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) braw[i] = has_bias ? bias[min(lane * PER + i, e - 1)] : 0.0f;
    }
    __device__ __forceinline__ void keys(int e, uint32_t& live, uint32_t (&kh)[PER]) const {
        const int lane = threadIdx.x & 63;
        live = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            live |= (lane * PER + i < e ? 1u : 0u) << i;
            kh[i] = order_bits(has_bias ? raw[i] + braw[i] : raw[i]);
        }
    }
    // One round: the largest live key of the wave (ties to the lower index); removes it.
    __device__ __forceinline__ int round(uint32_t& live, const uint32_t (&kh)[PER], float& val) const {
        const int lane = threadIdx.x & 63;
        uint32_t h = 0, l = 0;   // key = (order bits, 0xFFFFFFFF - index); 0 = empty
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t li = 0xFFFFFFFFu - (uint32_t)(lane * PER + i);
            if (((live >> i) & 1u) && key_gt(kh[i], li, h, l)) { h = kh[i]; l = li; }
        }
        key_max_dpp<DPP_XOR1>(h, l);
        key_max_dpp<DPP_XOR2>(h, l);
        key_max_dpp<DPP_HALF_MIRROR>(h, l);
        key_max_dpp<DPP_MIRROR>(h, l);
        uint32_t bh = 0, bl = 0;
#pragma unroll
        for (int row = 0; row < 4; ++row) {
            const uint32_t rh = (uint32_t)__builtin_amdgcn_readlane((int)h, 16 * row);
            const uint32_t rl = (uint32_t)__builtin_amdgcn_readlane((int)l, 16 * row);
            if (key_gt(rh, rl, bh, bl)) { bh = rh; bl = rl; }
        }
        const int idx = (int)(0xFFFFFFFFu - bl);
        if (idx / PER == lane) live &= ~(1u << (idx % PER));
        val = from_order_bits(bh);
        return idx;
    }
    // The whole wave must call this.  Lane 0 writes sel[r] (expert of rank r) and w[r] (its
    // renormalized softmax weight), r < k.
    __device__ void select(int e, int k, int* sel, float* w) const {
        const int lane = threadIdx.x & 63;
        uint32_t live, kh[PER];
        keys(e, live, kh);
        float first = 0.0f;
        for (int r = 0; r < k; ++r) {
            float val;
            const int idx = round(live, kh, val);
            if (r == 0) first = val;
            if (lane == 0) { sel[r] = idx; w[r] = expf(val - first); }
        }
        if (lane == 0) {
            float sum = 0.0f;
            for (int r = 0; r < k; ++r) sum += w[r];
            for (int r = 0; r < k; ++r) w[r] = w[r] / sum;
        }
    }
};

// Logits per lane needed for e experts (1, 2, 4, 8 or 16).
__host__ __device__ inline int topk_per_lane(int e) {
    return e <= 64 ? 1 : e <= 128 ? 2 : e <= 256 ? 4 : e <= 512 ? 8 : 16;
}

template <int PER>
__device__ void wave_topk_impl(const float* __restrict__ v, const float* __restrict__ bias, int e,
                               int k, int* sel, float* w) {
    TopkKeys<PER, false> keys;
    keys.load(v, bias, e);
    keys.select(e, k, sel, w);
}

__device__ inline void wave_topk(const float* __restrict__ v, const float* __restrict__ bias,
                                 int e, int k, int* sel, float* w) {
    if (e <= 64) wave_topk_impl<1>(v, bias, e, k, sel, w);
    else if (e <= 128) wave_topk_impl<2>(v, bias, e, k, sel, w);
    else if (e <= 256) wave_topk_impl<4>(v, bias, e, k, sel, w);
    else if (e <= 512) wave_topk_impl<8>(v, bias, e, k, sel, w);
    else wave_topk_impl<16>(v, bias, e, k, sel, w);
}

}  // namespace qmoe
