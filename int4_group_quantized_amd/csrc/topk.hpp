// Top-K of one token's logits inside one wave, without LDS round trips.
//
// Routing family SOFTMAX_TOPK with K experts per token ("Edge0 project review" MoE spec;
// "Recover-LoRA ..." section 1).  The K largest of (logit + bias) are chosen in K rounds: a
// wave-wide maximum of the order-preserving float bits (DPP max within 16-lane rows, scalar
// readlanes across rows), then the lowest expert index holding that value (a ballot over
// the lanes), so an exact tie goes to the lower index.  The weights are the softmax over
// the K chosen logits (the full softmax renormalized over the selection).
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
    // The whole wave must call this.  Lane 0 .. k - 1 write sel[r] (expert of rank r) and w[r]
    // (its renormalized softmax weight), r < k.
    //
    // Each lane first sorts its entries by key, descending; an adjacent-swap sort that swaps
    // only on a strictly larger key keeps equal keys in index order.  A round then takes the
    // wave maximum of the lanes' head keys (DPP max within 16-lane rows, the four rows through
    // readlanes) and the lowest lane whose head holds it (ballot): that lane's head is its lowest
    // index with that key, and lane l holds indices l*PER .. l*PER + PER - 1, so the round picks
    // the lowest index of the largest key.  The winner drops its head.  Lane r keeps round r's
    // expert and key, and the k weights are taken in parallel at the end.
    // This lane's keys sorted descending (order-preserving float bits, 0: no entry) with
    // their indices.
    __device__ __forceinline__ void sorted(int e, uint32_t (&kv)[PER], int (&ki)[PER]) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool ok = lane * PER + i < e;
            kv[i] = ok ? order_bits(has_bias ? raw[i] + braw[i] : raw[i]) : 0u;
            ki[i] = lane * PER + i;
        }
#pragma unroll
        for (int pass = 0; pass < PER - 1; ++pass)
#pragma unroll
            for (int i = 0; i + 1 < PER - pass; ++i) {
                const bool sw = kv[i + 1] > kv[i];
                const uint32_t ka = kv[i], kb = kv[i + 1];
                const int ia = ki[i], ib = ki[i + 1];
                kv[i] = sw ? kb : ka; kv[i + 1] = sw ? ka : kb;
                ki[i] = sw ? ib : ia; ki[i + 1] = sw ? ia : ib;
            }
    }

    // One round: the lowest index holding the largest head key (returned in every lane, its
    // key in `best`); the winning lane drops its head.
    __device__ __forceinline__ int round(uint32_t (&kv)[PER], int (&ki)[PER], uint32_t& best) const {
        const int lane = threadIdx.x & 63;
        uint32_t m = kv[0];
        m = max(m, dpp_u<DPP_XOR1>(m));
        m = max(m, dpp_u<DPP_XOR2>(m));
        m = max(m, dpp_u<DPP_HALF_MIRROR>(m));
        m = max(m, dpp_u<DPP_MIRROR>(m));
        const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
        const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
        const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)m, 32);
        const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
        best = max(max(r0, r1), max(r2, r3));
        const int lw = __builtin_ctzll(__ballot(kv[0] == best));   // the lowest lane holding it
        const int idx = __builtin_amdgcn_readlane(ki[0], lw);
        const bool win = lane == lw;
#pragma unroll
        for (int i = 0; i + 1 < PER; ++i) {
            kv[i] = win ? kv[i + 1] : kv[i];
            ki[i] = win ? ki[i + 1] : ki[i];
        }
        kv[PER - 1] = win ? 0u : kv[PER - 1];
        return idx;
    }

    // The expert chosen in round k alone (the same in every lane): rounds 0 .. k, no weights.
    __device__ int pick(int e, int k) const {
        uint32_t kv[PER];
        int ki[PER];
        sorted(e, kv, ki);
        int idx = 0;
        uint32_t best;
        for (int r = 0; r <= k; ++r) idx = round(kv, ki, best);
        return idx;
    }

    __device__ void select(int e, int k, int* sel, float* w) const {
        const int lane = threadIdx.x & 63;
        uint32_t kv[PER];
        int ki[PER];
        sorted(e, kv, ki);
        int my_idx = 0;
        uint32_t my_key = 0u;
        for (int r = 0; r < k; ++r) {
            uint32_t best;
            const int idx = round(kv, ki, best);
            if (lane == r) { my_idx = idx; my_key = best; }
        }
        // softmax over the k chosen keys, relative to the largest (round 0's, held by lane 0)
        const float first = from_order_bits((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
        const float ex = lane < k ? expf(from_order_bits(my_key) - first) : 0.0f;
        float sum = ex;
        sum += dpp<DPP_XOR1>(sum);
        sum += dpp<DPP_XOR2>(sum);
        sum += dpp<DPP_HALF_MIRROR>(sum);
        sum += dpp<DPP_MIRROR>(sum);
        const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 0));
        const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 16));
        const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 32));
        const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 48));
        const float total = (s0 + s1) + (s2 + s3);
        if (lane < k) {
            sel[lane] = my_idx;
            w[lane] = ex / total;
        }
    }
};

// Weights of a given selection (the caller's routing, not the top-K): the softmax over its k
// logits l[0..k-1] (bias included), relative to their largest and summed in selection order,
// w[i] = exp(l_i - m) / sum_j exp(l_j - m).  Register form, one thread taking all k; the
// prefill per-token kernel takes the same operations in the same order across a wave's lanes,
// so both paths give the same bits for the same logits.
template <int MAXK>
__device__ __forceinline__ void given_softmax(int k, const float (&l)[MAXK], float (&w)[MAXK]) {
    float m = l[0];
#pragma unroll
    for (int i = 1; i < MAXK; ++i)
        if (i < k) m = fmaxf(m, l[i]);
    float total = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXK; ++i)
        if (i < k) total += expf(l[i] - m);
#pragma unroll
    for (int i = 0; i < MAXK; ++i) w[i] = i < k ? expf(l[i] - m) / total : 0.0f;
}

// Expert e of a given selection clamped into [0, n), so an out-of-range index can never
// address memory outside the expert stack.
__device__ __forceinline__ int clamp_expert(int e, int n) { return e < 0 ? 0 : (e >= n ? n - 1 : e); }

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
