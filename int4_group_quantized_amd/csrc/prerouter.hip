// Prerouter head forward: logits = linear_init(f) + fc2(gelu_erf(fc1(f))),
// f = [h, one-hot of this token's routed experts, one-hot of the previous token's].
//
// "Edge0 project review" (blog.kxstl.cn), highlight 1: layer N's head reads layer N's MoE
// input and the executed top-k of this token and of the previous token, and its top-K is
// layer N + 1's routing; exact-erf GELU; fp16 weights and arithmetic.  Every layer's output
// is rounded to fp16 as an fp16 module's is (fp32 accumulation).
//
// The one-hot parts of f are K ones among E zeros, so their products with a weight row are
// the sums of K gathered columns: each row reads its D dense inputs with 16-byte loads and
// 2K single elements, never the 2E one-hot columns.
//   P1 (fc1 and linear_init rows, one wave per row): z = fp16(W1 f + b1) ->
//      a = fp16(gelu(z)) stored; y0 = fp16(Wi f + bi) stored in `logits`.
//   P2 (fc2 rows, one wave per row): logits = fp16(y0 + fp16(W2 a + b2)).
//   Then the router's top-K on the logits when asked for.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace qmoe {

namespace {

constexpr int PR_MT = 8;   // tokens per pass

struct PrArgs {
    const uint16_t *wi, *bi, *w1, *b1, *w2, *b2;
    const uint16_t* h;
    const int32_t *now, *prev;
    int T, D, E, F, K;
    uint16_t* act;
    float* logits;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2(w.x), as_h2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.y), as_h2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.z), as_h2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.w), as_h2(x.w), acc, false);
    return acc;
}

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

constexpr int PR_U = 4;    // 16-byte weight units per lane held in registers (D <= 2048)

// P1: rows [0, F) are fc1, rows [F, F + E) linear_init.  h of up to PR_MT tokens in LDS.
// For D <= 2048 (one pass of tokens at a time) the row's weights and the first tokens'
// routing indices are loaded before h is staged, so those round trips overlap.
__global__ void __launch_bounds__(256) k_pr_fc1(PrArgs a) {
    __shared__ __align__(16) uint4 hs[1024];   // mt_max tokens x D inputs <= 8192 halves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rows = a.F + a.E, row = blockIdx.x * 4 + wave;
    const int n = a.D + 2 * a.E;               // row length
    const int units = a.D / 8;                 // 16-byte units of h
    const int mt_max = min(PR_MT, 8192 / a.D);
    const bool fc1 = row < a.F;
    const int rr = min(row, rows - 1);
    const uint16_t* wrow = fc1 ? a.w1 + (long)rr * n : a.wi + (long)(rr - a.F) * n;
    const float bias = h2f(fc1 ? a.b1[rr] : a.bi[rr - a.F]);
    const bool held = units <= 64 * PR_U;
    uint4 wr[PR_U];
#pragma unroll
    for (int i = 0; i < PR_U; ++i)   // unconditional (clamped) loads: no branch around them
        wr[i] = reinterpret_cast<const uint4*>(wrow)[min(lane + 64 * i, units - 1)];
    for (int t0 = 0; t0 < a.T; t0 += mt_max) {
        const int mt = min(mt_max, a.T - t0);
        __syncthreads();
        for (int u = threadIdx.x; u < mt * units; u += 256)
            hs[u] = reinterpret_cast<const uint4*>(a.h + (long)(t0 + u / units) * a.D)[u % units];
        __syncthreads();
        float acc[PR_MT];
#pragma unroll
        for (int t = 0; t < PR_MT; ++t) acc[t] = 0.0f;
        if (held) {
#pragma unroll
            for (int i = 0; i < PR_U; ++i) {
                const int c = lane + 64 * i;
                if (c < units) {
#pragma unroll
                    for (int t = 0; t < PR_MT; ++t)
                        if (t < mt) acc[t] = dot8(wr[i], hs[t * units + c], acc[t]);
                }
            }
        } else {
            for (int c = lane; c < units; c += 64) {
                const uint4 w = reinterpret_cast<const uint4*>(wrow)[c];
#pragma unroll
                for (int t = 0; t < PR_MT; ++t)
                    if (t < mt) acc[t] = dot8(w, hs[t * units + c], acc[t]);
            }
        }
        // the one-hot parts: lane j < K gathers this token's expert j, K <= j < 2K the
        // previous token's (indices clamped into [0, E))
#pragma unroll
        for (int t = 0; t < PR_MT; ++t) {
            if (t < mt) {
                if (lane < 2 * a.K) {
                    const bool cur = lane < a.K;
                    const int j = cur ? lane : lane - a.K;
                    const int e = (cur ? a.now : a.prev)[(long)(t0 + t) * a.K + j];
                    const int ec = min(max(e, 0), a.E - 1);
                    acc[t] += h2f(wrow[a.D + (cur ? 0 : a.E) + ec]);
                }
                const float v = wave_sum(acc[t]) + bias;
                if (lane == 0 && row < rows) {
                    const uint16_t z = f2h(v);
                    if (fc1) a.act[(long)(t0 + t) * a.F + row] = f2h(gelu_erf(h2f(z)));
                    else a.logits[(long)(t0 + t) * a.E + (row - a.F)] = h2f(z);
                }
            }
        }
    }
}

// P2: one wave per expert row of fc2 (F a multiple of 512: one 16-byte unit per lane and step).
__global__ void __launch_bounds__(256) k_pr_fc2(PrArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    if (e >= a.E) return;
    const uint4* wrow = reinterpret_cast<const uint4*>(a.w2 + (long)e * a.F);
    const float bias = h2f(a.b2[e]);
    const int units = a.F / 8;
    for (int t = 0; t < a.T; ++t) {
        const uint4* arow = reinterpret_cast<const uint4*>(a.act + (long)t * a.F);
        float acc = 0.0f;
        for (int c = lane; c < units; c += 64) acc = dot8(wrow[c], arow[c], acc);
        const float v = wave_sum(acc) + bias;
        if (lane == 0) {
            float* out = a.logits + (long)t * a.E + e;
            *out = h2f(f2h(*out + h2f(f2h(v))));
        }
    }
}

}  // namespace

hipError_t launch_prerouter(const qmoe_prerouter& P, const uint16_t* h, int t, int k,
                            const int32_t* now, const int32_t* prev, uint16_t* act,
                            float* logits, int32_t* pred_idx, float* pred_w, hipStream_t s) {
    PrArgs a{P.w_init, P.b_init, P.w1, P.b1, P.w2, P.b2, h, now, prev,
             t, P.hidden, P.n_experts, P.ffn, k, act, logits};
    k_pr_fc1<<<(unsigned)((P.ffn + P.n_experts + 3) / 4), 256, 0, s>>>(a);
    k_pr_fc2<<<(unsigned)((P.n_experts + 3) / 4), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !pred_idx) return e;
    return launch_router_topk(logits, t, P.n_experts, k, nullptr, pred_idx, pred_w, s);
}

}  // namespace qmoe
