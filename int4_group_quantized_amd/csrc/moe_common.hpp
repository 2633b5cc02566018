// Shared pieces of the two MoE layer paths (moe_decode.hip: a few tokens; moe_prefill.hip:
// any token count): kernel arguments, the x-side job grid and LoRA helpers.
#pragma once

#include "gemv_core.hpp"
#include "qmoe.h"
#include "topk.hpp"

namespace qmoe {

constexpr int MAX_RANK = 64;
constexpr int MAX_K = 32;
constexpr int MAX_DEC_T = 32;  // the decode path serves up to this many tokens per call
constexpr int MAX_DEC_K = 8;   // ... and up to this many experts per token
constexpr int DEC_ZP_BLOCKS = 32;   // decode: shared-expert row blocks of 64 per token (inter <= 2048)
constexpr int DEC_ZP_RANK = 16;     // ... each holding its share of z_down for LoRA ranks up to 16
constexpr int PF_ITEM = 128;   // most pairs per work item of the token-sorted GEMMs (slots per item)
constexpr int PF_SORT_MAXSEG = 64;   // most blocks (segments of pairs) of the multi-block sort

struct QW {
    const uint32_t* p;
    const uint16_t* s;
    const uint16_t* b;
};

struct MoeArgs {
    int T, H, I, SI, E, K, add_residual;
    int Ep;  // logits row stride: E rounded up to a multiple of 64
    const uint16_t* x;
    uint16_t* y;
    const int32_t* adapter;
    QW router, sgate, eg, eu, ed, shg, shu, shd;
    const uint16_t *Ag, *Bg, *Au, *Bu, *Ad, *Bd;
    int rg, ru, rd;
    int nag, nau, nad;  // adapters per projection
    float lsg, lsu, lsd;
    const float* rbias;
    const int32_t* route;   // given selection [T][K] (the caller's routing), or null: top-K
    int egroup, ebf;        // routed experts' group size (64 or 32) and bf16 parameters (1)
    // workspace
    float *logits, *gate, *zg, *zu, *zd, *gs, *us;
    int32_t* idx;
    int32_t* scnt;     // multi-block sort: per segment of pairs, the count of each expert
    int32_t* wrec;     // per work item of the token-sorted GEMMs: (expert, tokens, 0, 0)
    int32_t* wpairs;   // per work item: PF_ITEM slots of pair ids (the item's count used)
    float* wts;
    uint16_t *h, *hs;
    uint16_t* o;       // fp16 down outputs of the routed (token, k) pairs [T K][hidden]
    float* os;
    int32_t* idx_out;
    float* w_out;
};


struct XsideGrid {
    int nb_router, nb_gate, nb_shared, nb_z;
};

__host__ __device__ inline XsideGrid xside_grid(int T, int H, int E, int SI, int zjobs) {
    XsideGrid g;
    const int r8 = 4 * (64 / lanes_per_row(H));  // rows per block, 8-bit and 4-bit alike
    g.nb_router = (E + r8 - 1) / r8;
    g.nb_gate = 1;
    g.nb_shared = (2 * SI + r8 - 1) / r8;
    g.nb_z = (zjobs + 3) / 4;
    return g;
}


// Kernel arguments live in per-launch memory that no cache holds yet, so every scalar load
// batch of argument fields is a full memory round trip.  Consuming the fields a kernel
// needs in one empty asm at entry makes the compiler issue all those loads together (one
// round trip) instead of in dependent batches spread over the kernel.
#define QMOE_SGPR_USE2(x, y) asm volatile("" ::"s"(x), "s"(y))
#define QMOE_SGPR_USE4(x, y, z, w) asm volatile("" ::"s"(x), "s"(y), "s"(z), "s"(w))

namespace {

// scale-free LoRA up-projection of one output: sum_r B[a][n][r] * z[r].  Rank rows of a
// multiple of 8 are read with 16-byte loads, all issued before the sum.
__device__ __forceinline__ float lora_b_dot(const uint16_t* __restrict__ B, int a, int out_dim,
                                            int n, int rank, const float* z) {
    const uint16_t* brow = B + ((long)a * out_dim + n) * rank;
    float d = 0.0f;
    if ((rank & 7) == 0) {
        uint4 v[MAX_RANK / 8];
#pragma unroll
        for (int i = 0; i < MAX_RANK / 8; ++i)
            if (i < rank / 8) v[i] = *reinterpret_cast<const uint4*>(brow + i * 8);
#pragma unroll
        for (int i = 0; i < MAX_RANK / 8; ++i) {
            if (i < rank / 8) {
                const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    d = fmaf(half_lo(w4[j]), z[i * 8 + 2 * j], d);
                    d = fmaf(half_hi(w4[j]), z[i * 8 + 2 * j + 1], d);
                }
            }
        }
        return d;
    }
    for (int r = 0; r < rank; ++r) d = fmaf(h2f(brow[r]), z[r], d);
    return d;
}


// LoRA-B term of one output row from 16 rank entries held as two uint4 (entries r < rank
// count), z from LDS.
__device__ __forceinline__ float bdot16(const uint4 (&v)[2], const float* z, int rank) {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (8 * i < rank) {
            const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                d = fmaf(half_lo(w4[j]), z[8 * i + 2 * j], d);
                d = fmaf(half_hi(w4[j]), z[8 * i + 2 * j + 1], d);
            }
        }
    }
    return d;
}

// z[r] = A[r] . v for r < rank (A fp16 [rank][K] row-major, v fp16 [K]), whole block: one
// 16-lane DPP row per rank row, each lane a K/16 slice (K a multiple of 128), so all loads
// of the block are in flight together.  Writes z (LDS); the caller synchronises.
__device__ __forceinline__ void lora_rows16(const uint16_t* __restrict__ A, int rank,
                                   const uint16_t* __restrict__ v, int K, float* z) {
    const int lane16 = threadIdx.x & 15, row0 = threadIdx.x >> 4, nrows = NT >> 4;
    const int per = K / 16;                 // inputs per lane (a multiple of 8)
    constexpr int MAXI = 16;                // K <= 2048
    for (int r = row0; r < rank; r += nrows) {
        const uint16_t* arow = A + (long)r * K + lane16 * per;
        const uint16_t* vrow = v + lane16 * per;
        uint4 av[MAXI], xv[MAXI];
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            if (i * 8 < per) {
                av[i] = *reinterpret_cast<const uint4*>(arow + i * 8);
                xv[i] = *reinterpret_cast<const uint4*>(vrow + i * 8);
            }
        }
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            if (i * 8 < per) {
                const f16x2* ah = reinterpret_cast<const f16x2*>(&av[i]);
                const f16x2* xh = reinterpret_cast<const f16x2*>(&xv[i]);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_fdot2(ah[q], xh[q], acc, false);
            }
        }
        acc = seg_sum<16>(acc);
        if (lane16 == 0) z[r] = acc;
    }
}

// One LoRA down-projection dot of the x-side kernels: job j = (projection, token, rank row).
__device__ inline void xside_lora_z(const MoeArgs& a, int j, int zjobs) {
    const int lane = threadIdx.x & 63;
    if (j >= zjobs) return;
    const int H = a.H;
    const int ng = a.Ag ? a.T * a.rg : 0;
    const bool isg = j < ng;
    const int jj = isg ? j : j - ng;
    const int rank = isg ? a.rg : a.ru;
    const int t = jj / rank, r = jj % rank;
    const int ad = adapter_of(a.adapter, t, isg ? a.nag : a.nau);
    const uint16_t* arow = (isg ? a.Ag : a.Au) + ((long)ad * rank + r) * H;
    const uint16_t* xrow = a.x + (long)t * H;
    constexpr int MAXI = 8;                       // hidden <= 4096: 8 x 512 inputs
    uint4 av[MAXI], xv[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int k = lane * 8 + i * 512;
        if (k < H) {
            av[i] = *reinterpret_cast<const uint4*>(arow + k);
            xv[i] = *reinterpret_cast<const uint4*>(xrow + k);
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        if (lane * 8 + i * 512 < H) {
            const f16x2* ah = reinterpret_cast<const f16x2*>(&av[i]);
            const f16x2* xh = reinterpret_cast<const f16x2*>(&xv[i]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_fdot2(ah[q], xh[q], acc, false);
        }
    }
    acc = seg_sum<64>(acc);
    if (lane == 0) (isg ? a.zg : a.zu)[t * MAX_RANK + r] = acc;
}

}  // namespace

// moe_decode.hip
bool decode_path_fits(const qmoe_moe_layer& L, int T);
hipError_t launch_moe_decode(const MoeArgs& a, int stage, hipStream_t s);
// moe_prefill.hip
int prefill_max_items(int E, int T, int K, int H, int I, bool std_experts = true);
int prefill_item_size(int E, int T, int K, int H, int I, bool std_experts = true);
int prefill_ksplit(int hidden, int T);
hipError_t launch_moe_prefill(const MoeArgs& a, int stage, hipStream_t s);
// moe_down_fs.hip: the down projections and the combine in one launch (few routed pairs)
bool down_fs_fits(const MoeArgs& a);
hipError_t launch_down_fs(const MoeArgs& a, hipStream_t s);

}  // namespace qmoe
