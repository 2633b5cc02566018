// Prefill path of the MoE SwitchGLU layer (many tokens per call): top-K, a stable sort of
// the (token, k) pairs by expert, and grouped GEMMs on fp16 MFMA.
//
// The layer is the one of moe.hip (pages: "Edge0-35B-A3B Preview model repository guide"
// model spec; "Recover-LoRA ..." sections 1-2; "Edge0 project review" highlights 2-3).
// With hundreds of tokens an expert sees several of them, so each expert's weight rows
// are read once per call and applied to all its tokens as a small GEMM on the matrix
// cores.
//
// GEMM kernel (k_pf_gemm).  A block of 4 waves covers 64 output features (16 per wave) of
// one or two quantized matrices (gate and up together) against up to 64 activation rows
// (tokens), staged in LDS per 128-input step and double buffered.  MFMA
// v_mfma_f32_16x16x32_f16 takes the activations as A (16 tokens x 32 inputs) and the
// weights as B (32 inputs x 16 features): lane l supplies feature l % 16 and inputs
// 8 (l / 16) .. +7, and ends with tokens 4 (l / 16) .. +3 of feature l % 16.
//
// Weights.  In the grouped expert GEMMs a lane turns each packed word into the exact values
// q in fp16 (the nibbles masked in place under the exponent of 1024 or 64, the constant then
// subtracted) and dequantizes them with one fp16 fma, fp16(s q + b), one rounding per weight;
// every MFMA accumulates into the row's fp32 sum.  This costs about half the vector
// instructions of the exact form below, which matters both where the GEMM is bound by
// HBM (the vector work sits between a wave's loads) and where it is compute-bound.
// The dense x-side GEMMs keep the weights exact: the codes C + q (bits dropped into the
// mantissa of C = 16 or 256) feed the MFMAs, each MFMA pair covers exactly one 64-input
// group, so the group's sum P = sum (C + q) x is formed apart and, with the group's sum of
// inputs X (one more MFMA pair against a ones operand), the affine terms are applied per
// group in fp32:
//     acc += s P + (b - C s) X.
// The 8-bit router, whose logits decide top-K, is always exact.
// For that, a lane's 16-byte load of packed words (inputs 32 j .. 32 j + 31 of a 128-input
// step, j = lane / 16, i.e. half of group j / 2) is exchanged across the wave halves with
// v_permlane32_swap so that every register then holds words of a single group; the
// activation side reads the matching inputs from LDS.
#include <algorithm>
#include <type_traits>

#include "gemv_core.hpp"
#include "launch.hpp"
#include "moe_common.hpp"

namespace qmoe {

namespace {

constexpr int PF_TOK = 64;            // tokens per block of the dense GEMMs: 4 MFMA tiles
constexpr int PF_ROWS = 64;           // output features per block: 4 waves x 16
constexpr int PF_KS = 128;            // inputs per k step (two groups)
constexpr int PF_PITCH = PF_KS + 8;   // LDS row pitch in halves (272 bytes: no bank conflicts)
constexpr int PF_XS_K = 512;          // inputs per block of the split-K x-side GEMMs (few tokens)
constexpr int PF_XS_K_BIG = 2048;     // the same from PF_XS_BIG_T tokens up (enough blocks unsplit)
constexpr int PF_XS_BIG_T = 2048;
constexpr int PF_MANY_T = 1024;       // from this many tokens the per-token kernels favour occupancy
constexpr int PF_IB_TK = 256;         // up to this many pairs the GEMM blocks form their work items

struct PfGemm {
    const uint32_t* p[2];
    const uint16_t* s[2];
    const uint16_t* b[2];
    int N, K;                      // features per matrix (per expert), inputs
    const uint16_t* act;           // activation rows, fp16 [*][K]
    int T;                         // dense: token count
    int act_div;                   // grouped: activation row = pair / act_div (1: pair itself)
    const int32_t *wrec, *wpairs;  // grouped: work items (expert, tokens) and their pair ids
    const int32_t* ridx;           // grouped, few pairs: the pairs' experts; items formed in the block
    int rtk, risz, rE;             // ... from rtk pairs, isz pairs per item, rE experts
    int nrb, items;                // row blocks, grid items (a multiple of 8)
    int bf;                        // grouped fp16-weight GEMMs: scales and biases stored as bf16
    float* out0; float* out1;      // fp32 outputs [row][ostride]
    int ostride;
    int ksplit;                    // dense: K split over this many blocks (partial outputs)
    long pstride;                  // elements between the partial outputs of two splits
    uint16_t* hout;                // fp16 silu(out0) * out1, [pair][N]; or (F_O16) fp16 out0 [row][ostride]
    // one extra feature row N (dense, single matrix): read from (xp, xs, xb), written to
    // xout[split][t]
    const uint32_t* xp; const uint16_t* xs; const uint16_t* xb; float* xout;
};

// GEMM flavours
constexpr int F_GROUPED = 1;   // work items of the expert sort (else token groups of all tokens)
constexpr int F_HOUT = 2;      // fp16 silu(out0) * out1 (else fp32 outputs)
constexpr int F_O16 = 8;       // fp16 outputs to hout, single matrix (the experts' down outputs)
constexpr int F_EXTRA = 4;     // one extra feature row from a second matrix (single matrix)
constexpr int F_G32 = 16;      // groups of 32 inputs (four per step; grouped fp16-weight GEMMs)
constexpr int PF_RES_RBG = 2;  // row blocks per block of the resident-activation GEMM
constexpr int PF_RES_RBG64 = 4;   // ... for the dense shared down over 64-token groups (its 64 KB
                                  // activation staging per block favours fewer, longer blocks)

// LDS of one GEMM block: the activation tile (double buffer: step ks computes from ks % 2
// while step ks + 1's tile is staged into the other), and with a compile-time step count NS
// the block's scales and biases as (s | b << 16) dwords per (row, group), row pitch GPS NS + 4
// dwords (16 rows read without bank conflicts; GPS groups per 128-input step: 2, or 4 for
// groups of 32).
template <int NT, int NMAT, int NS, int GPS = 2>
struct PfSmem {
    f16 tile[2][16 * NT * PF_PITCH];
    uint32_t sb[NMAT][PF_ROWS][NS ? GPS * NS + 4 : 1];   // (s, b) per group; GPS groups a step
    int arow[16 * NT], orow[16 * NT];
};

// Stage one 8-input unit of activation row r (row-major fp16) into LDS in the pair order of
// the unpacking.
template <int BITS>
__device__ __forceinline__ void pf_commit(const uint4& raw, int r, int c, f16* tile) {
    *reinterpret_cast<uint4*>(tile + r * PF_PITCH + c * 8) = BITS == 4 ? pair_perm8_w(raw) : pair_perm4x2_w(raw);
}

// fp16 codes C + q of one 8-input unit in pair order (4-bit: one word, pairs (q_j, q_j+4);
// 8-bit: two words, pairs (b0, b2) (b1, b3)): each code shifted into mantissa bits 6..9
// (4-bit) or 2..9 (8-bit) under the exponent of C, held in `magic` (0x4C00 = 16 or 0x5C00 =
// 256 in both halves).  `magic` lives in a VGPR so each pair is one shift and one
// v_and_or_b32 (gfx9 VOP3 takes no literal operand).
template <int BITS>
__device__ __forceinline__ f16x8 pf_codes(const uint32_t* w, uint32_t magic) {
    uint32_t u[4];
    if constexpr (BITS == 4) {
        constexpr uint32_t M = 0x03C003C0u;
        u[0] = ((w[0] << 6) & M) | magic; u[1] = ((w[0] << 2) & M) | magic;
        u[2] = ((w[0] >> 2) & M) | magic; u[3] = ((w[0] >> 6) & M) | magic;
    } else {
        constexpr uint32_t M = 0x03FC03FCu;
        u[0] = ((w[0] << 2) & M) | magic; u[1] = ((w[0] >> 6) & M) | magic;
        u[2] = ((w[1] << 2) & M) | magic; u[3] = ((w[1] >> 6) & M) | magic;
    }
    return __builtin_bit_cast(f16x8, u);
}

// The 4-bit values q of one word as fp16, in the pair order of pf_codes, for the fp16-weight
// path.  Each nibble stays where it is: one at bits 0..3 of a half reads as 1024 + q under
// the exponent of 1024 (ulp 1), one at bits 4..7 as 64 + q under the exponent of 64 (ulp
// 1/16), so a word costs one shift and four v_and_or_b32; subtracting the constants is exact.
// m1024 and m64 hold fp16 1024 and 64 in both halves (in VGPRs, as `magic` of pf_codes).
__device__ __forceinline__ f16x8 pf_q4(uint32_t w, uint32_t m1024, uint32_t m64) {
    const uint32_t t = w >> 8;
    const uint32_t u[4] = {(w & 0x000F000Fu) | m1024,    // (q0, q4)
                           (w & 0x00F000F0u) | m64,      // (q1, q5)
                           (t & 0x000F000Fu) | m1024,    // (q2, q6)
                           (t & 0x00F000F0u) | m64};     // (q3, q7)
    const f16x8 off = {(f16)1024.0f, (f16)1024.0f, (f16)64.0f, (f16)64.0f,
                       (f16)1024.0f, (f16)1024.0f, (f16)64.0f, (f16)64.0f};
    return __builtin_bit_cast(f16x8, u) - off;
}

// fp16(s q + b) from the exact q: one fp16 fma, a single rounding of the dequantized weight
// (the tile fed to MFMA).
__device__ __forceinline__ f16x8 pf_dequant(f16x8 q, f16 s, f16 b) {
    const f16x8 sv = {s, s, s, s, s, s, s, s}, bv = {b, b, b, b, b, b, b, b};
    return __builtin_elementwise_fma(q, sv, bv);
}

// XCD-aware block order: blocks are handed to the 8 XCDs round-robin by linear id, so the
// id's low 3 bits pick the XCD.  Every row block of one item (expert chunk or token group)
// lands on the same XCD, and that XCD runs them back to back: the item's activations are
// fetched into one L2 once.
__device__ __forceinline__ void pf_block(int id, int nrb, int& rb, int& item) {
    const int xcd = id & 7, q = id >> 3;
    rb = q % nrb;
    item = (q / nrb) * 8 + xcd;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    return v;
}

// Work item `item` of the expert sort formed inside the block from the pairs' experts, for few
// pairs (rtk <= 256, rE <= 256, 256 threads) instead of read from the sort's records: the same
// items (experts ascending, an expert's pairs in pair order, chunks of risz) and so the same
// results, without the sort's launch.  Thread tid holds pair tid; the experts' pair counts
// are taken with LDS atomics, their item counts' prefix by a block scan, and the item's pairs
// are the pairs of its expert of rank j risz .. j risz + risz - 1 (ballots).  `lds`: IIB_LDS_INTS ints.
// Returns false past the last item; else the expert, the pair count and, after the caller's
// barrier, the pair ids in orow[0 .. ntok) (the block's TOKB slots, TOKB = risz by the host's
// choice of kernel; bounded by it regardless).  Every thread of the block calls it; the
// block has 256 threads (one per expert and per pair).
constexpr int IIB_LDS_INTS = 272;
template <int TOKB>
__device__ __forceinline__ bool item_in_block(const PfGemm& a, int item, int* lds, int* orow, int& e, int& ntok) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int* cnt = lds;          // [256] pairs per expert
    int* misc = lds + 256;   // [0, 4): waves' item sums; [4, 7): the item's expert, chunk, count; [8, 12): ballots
    const int ex = tid < a.rtk ? a.ridx[tid] : -1;
    cnt[tid] = 0;
    if (tid == 0) misc[4] = -1;
    __syncthreads();
    if (ex >= 0) atomicAdd(&cnt[ex], 1);
    __syncthreads();
    const int c = tid < a.rE ? cnt[tid] : 0;
    const int nw = (c + a.risz - 1) / a.risz;
    const int inc = wave_scan(nw);
    if (lane == 63) misc[wave] = inc;
    __syncthreads();
    int wex = inc - nw;
    for (int w = 0; w < wave; ++w) wex += misc[w];
    if (item >= wex && item < wex + nw) {
        misc[4] = tid;
        misc[5] = item - wex;
        misc[6] = c;
    }
    __syncthreads();
    e = misc[4];
    if (e < 0) return false;
    const int j = misc[5];
    ntok = min(min(a.risz, TOKB), misc[6] - j * a.risz);
    const uint64_t m = __ballot(ex == e);
    if (lane == 0) misc[8 + wave] = (int)__popcll(m);
    __syncthreads();
    int rank = (int)__popcll(m & ((1ull << lane) - 1)) - j * a.risz;
    for (int w = 0; w < wave; ++w) rank += misc[8 + w];
    if (ex == e && rank >= 0 && rank < ntok) orow[rank] = tid;
    return true;
}

// The packed words, scales and biases of one 128-input step for this lane's feature row.
template <int NMAT, int BITS>
struct PfSlot {
    static constexpr int LW = BITS;   // words per lane per step: 4 (4-bit) or 8 (8-bit)
    uint32_t w[NMAT][LW];
    uint32_t s[NMAT], b[NMAT];        // the step's two groups as fp16 pairs
};

// The block's token rows: for a work item (GROUPED) the expert and its pair ids, padded
// by repeating the last pair (activation rows of the padding are loaded, their results never
// stored); for a dense GEMM the token group and split of `item`.  False: nothing to do.
template <int NT, int FL, int NS, int SM_NMAT, int NTS, int GPS>
__device__ __forceinline__ bool pf_setup(const PfGemm& a, int item, PfSmem<NTS, SM_NMAT, NS, GPS>& sm,
                                         int& ntok, int& e, int& split) {
    constexpr bool GROUPED = FL & F_GROUPED;
    constexpr int TOKB = 16 * NT;
    e = 0;
    split = 0;
    if constexpr (GROUPED) {
        static_assert(!GROUPED || TOKB <= PF_ITEM, "one work item per block");
        if (a.ridx) {   // (the tile is free until the GEMM stages its first step)
            static_assert(sizeof(sm.tile) >= IIB_LDS_INTS * sizeof(int), "LDS for item_in_block");
            if (!item_in_block<TOKB>(a, item, reinterpret_cast<int*>(sm.tile), sm.orow, e, ntok)) return false;
            __syncthreads();
            if (threadIdx.x < TOKB) sm.arow[threadIdx.x] = sm.orow[min((int)threadIdx.x, ntok - 1)] / a.act_div;
            __syncthreads();
            return true;
        }
        // the record and the pair ids in one round trip (both indexed by the item alone)
        const int4 rec = reinterpret_cast<const int4*>(a.wrec)[item];
        const int pair = threadIdx.x < TOKB ? a.wpairs[(long)item * PF_ITEM + threadIdx.x] : 0;
        if (rec.y == 0) return false;   // past the last item
        e = rec.x;
        ntok = rec.y;
        if (threadIdx.x < TOKB) sm.orow[threadIdx.x] = pair;
        __syncthreads();
        if (threadIdx.x < TOKB) sm.arow[threadIdx.x] = sm.orow[min((int)threadIdx.x, ntok - 1)] / a.act_div;
    } else {
        const int t0 = (item / a.ksplit) * TOKB;
        split = item % a.ksplit;
        if (t0 >= a.T) return false;
        ntok = min(TOKB, a.T - t0);
        if (threadIdx.x < TOKB) {
            sm.arow[threadIdx.x] = t0 + min((int)threadIdx.x, ntok - 1);
            sm.orow[threadIdx.x] = t0 + threadIdx.x;
        }
    }
    __syncthreads();
    return true;
}

// One block of the GEMM: features rb*64 .. +63 (16 per wave) of the block's tokens, NTE
// tiles of 16 (the token rows set up by pf_setup in LDS sized for NT tiles).  Weights and
// activations are loaded D steps ahead: the weights into D register slots (the loop
// unrolled by D), the activations into registers that are staged into the LDS double
// buffer one step before their use.  The weight rows of one block share a base address (the
// expert's matrix) held in scalar registers; a lane keeps 32-bit offsets, or in the fp16
// path (registers to spare) its row pointers formed once.
template <int NMAT, int BITS, int NTE, int FL, int NS, int SM_NMAT, int NTS, int GPS>
__device__ __forceinline__ void pf_gemm_body(const PfGemm& a, int rb, int ntok, int e, int split,
                                             PfSmem<NTS, SM_NMAT, NS, GPS>& sm) {
    static_assert(SM_NMAT >= NMAT, "LDS holds the scales of every matrix");
    static_assert(NTE <= NTS, "LDS holds every tile");
    constexpr bool HOUT = FL & F_HOUT, EXTRA = FL & F_EXTRA;
    // fp16 weights for the grouped 4-bit GEMMs and the dense ones with four token tiles;
    // exact codes for the 8-bit router and for dense GEMMs of fewer tiles
    constexpr bool DQ = BITS == 4 && ((FL & F_GROUPED) || NTE >= 4);
    // groups of 32: grouped fp16-weight GEMMs with a compile-time step count (parameters
    // staged in LDS), GPS = 4 groups per step
    constexpr bool G32 = FL & F_G32;
    static_assert(!G32 || (DQ && NS > 0 && !(FL & F_EXTRA)), "groups of 32: staged fp16-weight GEMMs");
    static_assert(GPS == (G32 ? 4 : 2), "LDS sized for the group size");
    const int ntiles = (ntok + 15) >> 4;   // <= NTE
    // NS > 0: the block's step count known at compile time (the loop fully unrolled); the
    // block covers steps kofs .. kofs + nsteps - 1 of the row (split-K for dense GEMMs)
    const int K = a.K, G = K / (G32 ? 32 : 64), nsteps = NS ? NS : K / PF_KS;   // even
    const int kofs = split * nsteps;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, j = lane >> 4;
    const int n = rb * PF_ROWS + wave * 16 + col;              // this lane's feature
    constexpr int WPU = BITS / 4;                              // words per 8-input unit
    const int wpr = K * BITS / 32;
    // uniform bases (this expert's matrices) and per-lane offsets; rows past the matrix are
    // clamped (their results are never stored)
    const uint32_t* wb[NMAT];
    const uint16_t* sb[NMAT];
    const uint16_t* bb_[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        wb[m] = a.p[m] + (long)e * a.N * wpr;
        sb[m] = a.s[m] + (long)e * a.N * G;
        bb_[m] = a.b[m] + (long)e * a.N * G;
    }
    const uint32_t woff = (uint32_t)min(n, a.N - 1) * wpr + j * 4 * WPU;
    const uint32_t goff = (uint32_t)min(n, a.N - 1) * G;
    // EXTRA: lanes past the last row read row 0 of the extra matrix through per-lane pointers
    const bool xrow = EXTRA && n >= a.N;
    const uint32_t* xw = xrow ? a.xp + j * 4 * WPU : wb[0] + woff;
    const uint16_t* xs = xrow ? a.xs : sb[0] + goff;
    const uint16_t* xb = xrow ? a.xb : bb_[0] + goff;
    // with NS known: the block's scales and biases into LDS with 16-byte loads, 8 groups a unit
    constexpr int UPR = NS * GPS / 8;                        // units of 8 groups per row
    constexpr int SBI = NS ? (PF_ROWS * UPR + 255) / 256 : 1;   // units per thread
    uint4 sbr[NMAT][2][SBI];
    auto load_sb = [&] {
        if constexpr (NS > 0) {
#pragma unroll
            for (int i = 0; i < SBI; ++i) {
                const int u = min(i * 256 + (int)threadIdx.x, PF_ROWS * UPR - 1);
                const int r = u / UPR, c8 = u % UPR, rowg = rb * PF_ROWS + r;
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const uint16_t* ss = sb[m] + (long)min(rowg, a.N - 1) * G;
                    const uint16_t* bs = bb_[m] + (long)min(rowg, a.N - 1) * G;
                    if (EXTRA && rowg >= a.N) { ss = a.xs; bs = a.xb; }
                    sbr[m][0][i] = reinterpret_cast<const uint4*>(ss + GPS * kofs)[c8];
                    sbr[m][1][i] = reinterpret_cast<const uint4*>(bs + GPS * kofs)[c8];
                }
            }
        }
    };
    auto commit_sb = [&] {
        if constexpr (NS > 0) {
#pragma unroll
            for (int i = 0; i < SBI; ++i) {
                const int u = i * 256 + (int)threadIdx.x;
                if (u < PF_ROWS * UPR) {
                    const int r = u / UPR, c8 = u % UPR;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) {
                        uint32_t sv[4], bv[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            sv[k] = reinterpret_cast<const uint32_t*>(&sbr[m][0][i])[k];
                            bv[k] = reinterpret_cast<const uint32_t*>(&sbr[m][1][i])[k];
                            if constexpr (DQ) {   // bf16 parameters: fp16 pairs (exact in fp16's normal range)
                                sv[k] = a.bf ? bf2_to_h2(sv[k]) : sv[k];
                                bv[k] = a.bf ? bf2_to_h2(bv[k]) : bv[k];
                            }
                        }
                        uint32_t o[8];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            o[2 * k] = __builtin_amdgcn_perm(bv[k], sv[k], 0x05040100u);       // (s, b) of group 2k
                            o[2 * k + 1] = __builtin_amdgcn_perm(bv[k], sv[k], 0x07060302u);   // group 2k + 1
                        }
                        uint4* dst = reinterpret_cast<uint4*>(&sm.sb[m][r][c8 * 8]);
                        dst[0] = uint4{o[0], o[1], o[2], o[3]};
                        dst[1] = uint4{o[4], o[5], o[6], o[7]};
                    }
                }
            }
        }
    };

    // staging: thread handles unit (r = u / 16, c = u % 16), u = tid + 256 q, q < ntiles
    const int sr = threadIdx.x >> 4, sc = threadIdx.x & 15;
    // Loads are unconditional (rows past the item repeat its last row; a step past the end
    // repeats the last step): a load inside a branch gets its wait placed right after it,
    // which would also drain every weight load in flight.
    // D steps of activations and weights in flight: step ks issues the loads of step ks + D,
    // activations before weights, so the wait for the activations of step ks + 1 leaves the
    // weights of steps ks + 1 .. ks + D - 1 in flight
    constexpr int D = NTE >= 4 ? 2 : 4;
    uint4 xr[D][NTE];
    // fp16-weight path (LDS holds it to three waves per SIMD, so registers are to spare): the
    // activation rows this thread stages and the weight rows of its feature as pointers formed
    // once, a step's load then pointer + step offset (an immediate when NS > 0).  Elsewhere
    // (four waves, at most 128 registers) the addresses are formed per load.
    constexpr bool HOIST = DQ;
    const uint16_t* xrp[HOIST ? NTE : 1];
    const uint32_t* wrp[HOIST ? NMAT : 1];
    if constexpr (HOIST) {
#pragma unroll
        for (int q = 0; q < NTE; ++q) xrp[q] = a.act + (long)sm.arow[q * 16 + sr] * K + kofs * PF_KS + sc * 8;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) wrp[m] = (EXTRA ? xw : wb[m] + woff) + (long)kofs * (PF_KS * BITS / 32);
    }
    auto load_x = [&](uint4 (&x)[NTE], int ks) {
        ks = min(ks, nsteps - 1);
#pragma unroll
        for (int q = 0; q < NTE; ++q) {
            if constexpr (HOIST)
                x[q] = *reinterpret_cast<const uint4*>(xrp[q] + ks * PF_KS);
            else
                x[q] = reinterpret_cast<const uint4*>(a.act + (long)sm.arow[q * 16 + sr] * K + (kofs + ks) * PF_KS)[sc];
        }
    };
    auto commit_x = [&](const uint4 (&x)[NTE], int buf) {
#pragma unroll
        for (int q = 0; q < NTE; ++q)
            if (q < ntiles) pf_commit<BITS>(x[q], q * 16 + sr, sc, sm.tile[buf]);
    };
    using Slot = PfSlot<NMAT, BITS>;
    auto load_w = [&](Slot& sl, int ks) {
        ks = min(ks, nsteps - 1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const int kg = kofs + ks;
            const uint4* src;
            if constexpr (HOIST)
                src = reinterpret_cast<const uint4*>(wrp[m] + ks * (PF_KS * BITS / 32));
            else
                src = EXTRA ? reinterpret_cast<const uint4*>(xw + kg * (PF_KS * BITS / 32))
                            : reinterpret_cast<const uint4*>(wb[m] + (woff + (uint32_t)kg * (PF_KS * BITS / 32)));
#pragma unroll
            for (int v = 0; v < WPU; ++v) {
                const uint4 x = src[v];
                sl.w[m][4 * v] = x.x; sl.w[m][4 * v + 1] = x.y; sl.w[m][4 * v + 2] = x.z; sl.w[m][4 * v + 3] = x.w;
            }
            if constexpr (NS > 0) {
                // scales come from LDS
            } else if constexpr (EXTRA) {
                sl.s[m] = reinterpret_cast<const uint32_t*>(xs)[kg];
                sl.b[m] = reinterpret_cast<const uint32_t*>(xb)[kg];
            } else {
                sl.s[m] = reinterpret_cast<const uint32_t*>(sb[m] + goff)[kg];
                sl.b[m] = reinterpret_cast<const uint32_t*>(bb_[m] + goff)[kg];
            }
        }
    };

    f32x4 acc[NMAT][NTE];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < NTE; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr float C = code_div<BITS>();
    uint32_t magic = BITS == 4 ? 0x4C004C00u : 0x5C005C00u;   // fp16 C in both halves
    asm volatile("" : "+v"(magic));
    uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;            // fp16 1024 and 64 (pf_q4)
    if constexpr (DQ) asm volatile("" : "+v"(m1024), "+v"(m64));
    const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
    // input unit (8 inputs) of the step that this lane's register slot (g, mm) holds after the
    // exchange: unit = 8 g + 2 mm + 4 (j & 1) + (j >> 1)
    const int ubase = 4 * (j & 1) + (j >> 1);

    // One step.  Every loop-carried register (the slot, the staged activations) is consumed
    // before its reload is issued, so old and new values never live together: the register
    // allocator keeps them in place and the loop back-edge needs no copy of a loaded register
    // (such a copy would wait for every load in flight).
    auto step = [&](Slot& sl, uint4 (&xnext)[NTE], uint4 (&xfree)[NTE], int ks) {
        const int buf = ks & 1;
        // stage the activations of step ks + 1 into the other buffer, which every wave
        // finished reading before the barrier that ended step ks - 1
        if (ks + 1 < nsteps) commit_x(xnext, buf ^ 1);
        // exchange halves: afterwards units 0 and 2 of the lane hold group 0, 1 and 3 group 1
        uint32_t cw[NMAT][Slot::LW];
        float sv[NMAT][2], bv[NMAT][2];   // 8-bit: s and b - C s of the step's two groups
        f16 sh[NMAT][2], bh[NMAT][2];     // 4-bit: s and b as stored
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int v = 0; v < WPU; ++v) {
                    const auto r = __builtin_amdgcn_permlane32_swap(sl.w[m][(2 * h) * WPU + v],
                                                                    sl.w[m][(2 * h + 1) * WPU + v], false, false);
                    cw[m][(2 * h) * WPU + v] = r[0];
                    cw[m][(2 * h + 1) * WPU + v] = r[1];
                }
            }
            if constexpr (NS > 0 && G32) {
                // groups of 32: register slot g of lane group j covers group 2 g + (j & 1)
                const uint4 p = *reinterpret_cast<const uint4*>(&sm.sb[m][wave * 16 + col][4 * ks]);
                const f16x2 g0 = as_h2((j & 1) ? p.y : p.x), g1 = as_h2((j & 1) ? p.w : p.z);
                sh[m][0] = g0[0]; bh[m][0] = g0[1];
                sh[m][1] = g1[0]; bh[m][1] = g1[1];
            } else if constexpr (NS > 0) {
                const uint2 p = *reinterpret_cast<const uint2*>(&sm.sb[m][wave * 16 + col][2 * ks]);
                const f16x2 g0 = as_h2(p.x), g1 = as_h2(p.y);   // (s, b) of the step's groups
                sh[m][0] = g0[0]; bh[m][0] = g0[1];
                sh[m][1] = g1[0]; bh[m][1] = g1[1];
            } else {
                const f16x2 s2 = as_h2(sl.s[m]), b2 = as_h2(sl.b[m]);
#pragma unroll
                for (int g = 0; g < 2; ++g) { sh[m][g] = s2[g]; bh[m][g] = b2[g]; }
            }
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                sv[m][g] = (float)sh[m][g];
                bv[m][g] = fmaf(-C, sv[m][g], (float)bh[m][g]);
            }
        }
        // then the loads of step ks + D (into the slot and the activation registers just
        // consumed): activations first, since they are needed a step earlier than the weights
        if (NS == 0 || ks + D < nsteps) {
            load_x(xfree, ks + D);
            load_w(sl, ks + D);
        }
        const f16* tb = sm.tile[buf];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            f16x8 bw[NMAT][2];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    if constexpr (DQ)
                        bw[m][mm] = pf_dequant(pf_q4(cw[m][2 * mm + g], m1024, m64), sh[m][g], bh[m][g]);
                    else
                        bw[m][mm] = pf_codes<BITS>(&cw[m][(2 * mm + g) * WPU], magic);
                }
#pragma unroll
            for (int c = 0; c < NTE; ++c) {
                if constexpr (DQ) {
                    // fp16 weights: accumulate over the whole row.  Every tile is computed
                    // (tiles past the item's tokens read padding rows; their results are never
                    // stored): with no branch between the MFMAs the compiler places no
                    // accumulator writes next to an MFMA still reading them.
                    const f16* trow = tb + (c * 16 + col) * PF_PITCH;
                    const f16x8 a0 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + ubase));
                    const f16x8 a1 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + 2 + ubase));
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) {
                        acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bw[m][0], acc[m][c], 0, 0, 0);
                        acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bw[m][1], acc[m][c], 0, 0, 0);
                    }
                    continue;
                }
                if (c < ntiles) {
                    const f16* trow = tb + (c * 16 + col) * PF_PITCH;
                    const f16x8 a0 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + ubase));
                    const f16x8 a1 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + 2 + ubase));
                    f32x4 X = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, ones, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    X = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, ones, X, 0, 0, 0);
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) {
                        f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bw[m][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bw[m][1], P, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[m][c][r] = fmaf(sv[m][g], P[r], fmaf(bv[m][g], X[r], acc[m][c][r]));
                    }
                }
            }
        }
        __syncthreads();
    };

    Slot sl[D];
    load_sb();
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_x(xr[d], d);
        load_w(sl[d], d);
    }
    commit_sb();
    commit_x(xr[0], 0);
    __syncthreads();
    static_assert(NS % D == 0, "whole rounds of D steps");
#pragma unroll
    for (int ks = 0; ks < (NS ? NS : nsteps); ks += D) {   // nsteps is a multiple of 4
#pragma unroll
        for (int d = 0; d < D; ++d) step(sl[d], xr[(d + 1) % D], xr[d], ks + d);
    }

    // epilogue: tokens 16 c + 4 j + r of feature n
    const bool extra = EXTRA && n == a.N;
    if (n >= a.N && !extra) return;
#pragma unroll
    for (int c = 0; c < NTE; ++c) {
        if (c >= ntiles) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = c * 16 + 4 * j + r;
            if (t < ntok) {
                const int orow = sm.orow[t];
                if constexpr (HOUT) {
                    a.hout[(long)orow * a.N + n] = f2h(silu(acc[0][c][r]) * acc[NMAT - 1][c][r]);
                } else if constexpr ((FL & F_O16) != 0) {
                    a.hout[(long)orow * a.ostride + n] = f2h(acc[0][c][r]);
                } else if (extra) {
                    a.xout[(long)split * a.T + orow] = acc[0][c][r];
                } else {
                    const long o = (long)split * a.pstride + (long)orow * a.ostride + n;
                    a.out0[o] = acc[0][c][r];
                    if (NMAT == 2) a.out1[o] = acc[NMAT - 1][c][r];
                }
            }
        }
    }
}

// One block: the token rows of `item` (NT tiles of 16), then the GEMM over them.  LDS is
// sized for NTS >= NT tiles, so kernels that run GEMMs of two tile counts share one layout.
// (One body per kernel: with two inlined bodies the register allocation spills.)
template <int NMAT, int BITS, int NT, int FL, int NS, int SM_NMAT, int NTS = NT, int GPS = 2>
__device__ __forceinline__ void pf_gemm_block(const PfGemm& a, int rb, int item,
                                              PfSmem<NTS, SM_NMAT, NS, GPS>& sm) {
    int ntok, e, split;
    if (!pf_setup<NT, FL, NS, SM_NMAT, NTS, GPS>(a, item, sm, ntok, e, split)) return;
    pf_gemm_body<NMAT, BITS, NT, FL, NS, SM_NMAT, NTS, GPS>(a, rb, ntok, e, split, sm);
}

template <int NMAT, int BITS, int NT, int FL, int NS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) k_pf_gemm(PfGemm a) {
    __shared__ __align__(16) PfSmem<NT, NMAT, NS, (FL & F_G32) ? 4 : 2> sm;
    int rb, item;
    pf_block(blockIdx.x, a.nrb, rb, item);
    pf_gemm_block<NMAT, BITS, NT, FL, NS, NMAT, NT, (FL & F_G32) ? 4 : 2>(a, rb, item, sm);
}

// The grouped down GEMM and the shared expert's dense down GEMM in one launch (they are
// independent; equal inner sizes, so one step count): blocks below nbd take the dense
// GEMM's (token group, row block), the rest work items.
template <int NS, int NTG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
k_pf_down(PfGemm g, PfGemm d, int nbd) {
    constexpr int NTS = NTG > 2 ? NTG : 2;   // LDS for both tile counts
    __shared__ __align__(16) PfSmem<NTS, 1, NS> sm;
    int rb, item;
    // the shared expert's dense blocks first (nbd of them, a multiple of 8 so the grouped
    // blocks keep their XCD placement)
    if ((int)blockIdx.x >= nbd) {
        pf_block(blockIdx.x - nbd, g.nrb, rb, item);
        pf_gemm_block<1, 4, NTG, F_GROUPED | F_O16, NS, 1, NTS>(g, rb, item, sm);
    } else {
        pf_block(blockIdx.x, d.nrb, rb, item);
        pf_gemm_block<1, 4, 2, 0, NS, 1, NTS>(d, rb, item, sm);
    }
}

// LDS of the resident-activation GEMM: the block's 16 NT token rows over all K inputs (pair
// order, 16-byte row pad against bank conflicts) and their sums over each group of 64.
template <int NT, int NS>
struct PfResSmem {
    static constexpr int PITCH = NS * PF_KS + 8;
    f16 tile[16 * NT * PITCH];
    float xsum[2 * NS][16 * NT];   // [group][token]
    int arow[16 * NT], orow[16 * NT];
};

// GEMM block for a short reduction (K = 128 NS <= 1024), one 4-bit matrix: the block's
// activations stay in LDS for all of K, so the block then runs RBG row blocks of 64 features
// back to back with no barrier: the weights stream through D register slots across row-block
// boundaries, each row block's scales and biases (one 16-byte load per 8 groups) come in
// with them, and the b term uses the group sums taken once per block (acc += s P + (b - C s)
// X with X from LDS), so each step is two MFMAs per group and tile.
template <int NT, int NS, int RBG, int FL>
__device__ __forceinline__ void pf_res_block(const PfGemm& a, int rbg, int item, PfResSmem<NT, NS>& sm) {
    constexpr int PITCH = PfResSmem<NT, NS>::PITCH, K = NS * PF_KS, G = K / 64, SBV = G / 8;
    constexpr int NSTEP = RBG * NS, D = 4;
    int ntok, e, split;
    {   // the token rows (pf_setup's rules)
        constexpr int TOKB = 16 * NT;
        e = 0; split = 0;
        if constexpr (FL & F_GROUPED) {
            if (a.ridx) {
                static_assert(sizeof(sm.tile) >= IIB_LDS_INTS * sizeof(int), "LDS for item_in_block");
                if (!item_in_block<TOKB>(a, item, reinterpret_cast<int*>(sm.tile), sm.orow, e, ntok)) return;
            } else {
                const int4 rec = reinterpret_cast<const int4*>(a.wrec)[item];
                const int pair = threadIdx.x < TOKB ? a.wpairs[(long)item * PF_ITEM + threadIdx.x] : 0;
                if (rec.y == 0) return;
                e = rec.x;
                ntok = rec.y;
                if (threadIdx.x < TOKB) sm.orow[threadIdx.x] = pair;
            }
            __syncthreads();
            if (threadIdx.x < TOKB) sm.arow[threadIdx.x] = sm.orow[min((int)threadIdx.x, ntok - 1)] / a.act_div;
        } else {
            const int t0 = item * TOKB;
            if (t0 >= a.T) return;
            ntok = min(TOKB, a.T - t0);
            if (threadIdx.x < TOKB) {
                sm.arow[threadIdx.x] = t0 + min((int)threadIdx.x, ntok - 1);
                sm.orow[threadIdx.x] = t0 + threadIdx.x;
            }
        }
        __syncthreads();
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, j = lane >> 4;
    constexpr int UPR = K / 8;                      // 8-input units per row
    const int wpr = K / 8;                          // packed words per row
    const uint32_t* wb = a.p[0] + (long)e * a.N * wpr;
    const uint16_t* sbase = a.s[0] + (long)e * a.N * G;
    const uint16_t* bbase = a.b[0] + (long)e * a.N * G;
    // weights of flattened step f (row block f / NS, step f % NS); rows past N clamped
    auto row_of = [&](int rbl) { return min((rbg * RBG + rbl) * PF_ROWS + wave * 16 + col, a.N - 1); };
    uint32_t sl[D][4];
    auto load_w = [&](int f) {
        const uint4 v = reinterpret_cast<const uint4*>(wb + (uint32_t)row_of(f / NS) * wpr + (f % NS) * (PF_KS / 8))[j];
        uint32_t* d = sl[f % D];
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    };
    uint4 sv[2][SBV], bvv[2][SBV];   // scales and biases of a row block: current and next
    auto load_sb = [&](int rbl) {
        const long o = (long)row_of(rbl) * G;
#pragma unroll
        for (int i = 0; i < SBV; ++i) {
            sv[rbl & 1][i] = reinterpret_cast<const uint4*>(sbase + o)[i];
            bvv[rbl & 1][i] = reinterpret_cast<const uint4*>(bbase + o)[i];
        }
    };
    // the activations: 16 NT rows x K, one 16-byte unit per thread per pass, all loads first
    {
        constexpr int NU = 16 * NT * UPR / 256;
        uint4 xr[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = i * 256 + threadIdx.x, r = u / UPR, c = u % UPR;
            xr[i] = reinterpret_cast<const uint4*>(a.act + (long)sm.arow[r] * a.K)[c];
        }
        load_sb(0);
#pragma unroll
        for (int f = 0; f < D; ++f) load_w(f);
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = i * 256 + threadIdx.x, r = u / UPR, c = u % UPR;
            *reinterpret_cast<uint4*>(sm.tile + r * PITCH + c * 8) = pair_perm8_w(xr[i]);
        }
    }
    __syncthreads();
    // fp16 weights for blocks of four token tiles, as in pf_gemm_body.  With fewer
    // tiles the exact form stays: the group sums X come from LDS here, so its per-group terms
    // cost no more vector work than the fp16 dequantization would.
    constexpr bool DQ = NT >= 4;
    // group sums of the activation rows (fp32; the pair order stays inside a unit)
    if constexpr (!DQ)
    for (int q = threadIdx.x; q < 16 * NT * G; q += 256) {
        const int r = q % (16 * NT), g = q / (16 * NT);
        const uint4* row = reinterpret_cast<const uint4*>(sm.tile + r * PITCH + g * 64);
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += sum8_w(row[u]);
        sm.xsum[g][r] = acc;
    }
    __syncthreads();

    constexpr float C = code_div<4>();
    uint32_t magic = 0x4C004C00u;
    asm volatile("" : "+v"(magic));
    uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;   // fp16 1024 and 64 (pf_q4)
    if constexpr (DQ) asm volatile("" : "+v"(m1024), "+v"(m64));
    const int ubase = 4 * (j & 1) + (j >> 1);
    const int ntiles = (ntok + 15) >> 4;
    int toff = 0;
    f32x4 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < NSTEP; ++f) {
        const int rbl = f / NS, ks = f % NS;
        uint32_t cw[4];
        {
            const uint32_t* w = sl[f % D];
            const auto r0 = __builtin_amdgcn_permlane32_swap(w[0], w[1], false, false);
            const auto r1 = __builtin_amdgcn_permlane32_swap(w[2], w[3], false, false);
            cw[0] = r0[0]; cw[1] = r0[1]; cw[2] = r1[0]; cw[3] = r1[1];
        }
        // the loads D steps ahead (the slot just consumed), and the next row block's scales
        if (f + D < NSTEP) load_w(f + D);
        if (ks == 0 && rbl + 1 < RBG) load_sb(rbl + 1);
        const uint32_t* svw = reinterpret_cast<const uint32_t*>(&sv[rbl & 1][0]);
        const uint32_t* bvw = reinterpret_cast<const uint32_t*>(&bvv[rbl & 1][0]);
        const uint32_t s2 = svw[ks], b2 = bvw[ks];   // groups 2 ks, 2 ks + 1 as fp16 pairs
        if constexpr (DQ) {
            // fp16(s q + b) weights, every tile computed (padding rows of the tile included,
            // never stored); a row block's first MFMA starts from zero, so no instruction
            // rewrites an accumulator between MFMAs.  The tile offset is made opaque per row
            // block: the activation fragments are the same in every row block, and the
            // compiler would otherwise keep all of them live in registers across row blocks.
            if (ks == 0) asm volatile("" : "+v"(toff));
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const f16 sh = as_h2(s2)[g], bh = as_h2(b2)[g];
                const f16x8 bw0 = pf_dequant(pf_q4(cw[g], m1024, m64), sh, bh);
                const f16x8 bw1 = pf_dequant(pf_q4(cw[2 + g], m1024, m64), sh, bh);
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const f16* trow = sm.tile + toff + (c * 16 + col) * PITCH + ks * PF_KS;
                    const f16x8 a0 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + ubase));
                    const f16x8 a1 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + 2 + ubase));
                    const f32x4 c0 = ks == 0 && g == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[c];
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bw0, c0, 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bw1, acc[c], 0, 0, 0);
                }
            }
        } else
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float s = g ? half_hi(s2) : half_lo(s2);
            const float bb = fmaf(-C, s, g ? half_hi(b2) : half_lo(b2));
            const f16x8 bw0 = pf_codes<4>(&cw[g], magic), bw1 = pf_codes<4>(&cw[2 + g], magic);
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                if (c < ntiles) {
                    const f16* trow = sm.tile + (c * 16 + col) * PITCH + ks * PF_KS;
                    const f16x8 a0 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + ubase));
                    const f16x8 a1 = *reinterpret_cast<const f16x8*>(trow + 8 * (8 * g + 2 + ubase));
                    f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bw0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bw1, P, 0, 0, 0);
                    const float4 X = *reinterpret_cast<const float4*>(&sm.xsum[2 * ks + g][c * 16 + 4 * j]);
                    acc[c][0] = fmaf(s, P[0], fmaf(bb, X.x, acc[c][0]));
                    acc[c][1] = fmaf(s, P[1], fmaf(bb, X.y, acc[c][1]));
                    acc[c][2] = fmaf(s, P[2], fmaf(bb, X.z, acc[c][2]));
                    acc[c][3] = fmaf(s, P[3], fmaf(bb, X.w, acc[c][3]));
                }
            }
        }
        if (ks == NS - 1) {   // row block done: tokens 16 c + 4 j + r of feature n
            const int n = (rbg * RBG + rbl) * PF_ROWS + wave * 16 + col;
            if (n < a.N) {
#pragma unroll
                for (int c = 0; c < NT; ++c) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = c * 16 + 4 * j + r;
                        if (c < ntiles && t < ntok) {
                            if constexpr ((FL & F_O16) != 0)
                                a.hout[(long)sm.orow[t] * a.ostride + n] = f2h(acc[c][r]);
                            else
                                a.out0[(long)sm.orow[t] * a.ostride + n] = acc[c][r];
                        }
                    }
                }
            }
            if constexpr (!DQ)
#pragma unroll
                for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// The grouped down GEMM and the shared expert's dense down GEMM in one launch, both with
// resident activations: blocks below nbd take the dense GEMM's (token group, row group), the
// rest (work item, row group).  With nbd = the grid, a launch of the dense GEMM alone.
template <int NS, int NT, int RBG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
k_pf_down_res(PfGemm g, PfGemm d, int nbd) {
    __shared__ __align__(16) PfResSmem<NT, NS> sm;
    int rbg, item;
    // the shared expert's dense blocks first: dispatched last they formed the launch's tail
    // (512 tokens: down stage 56.8 -> 53.4 us); nbd is a multiple of 8, so the grouped blocks
    // keep their XCD placement
    if ((int)blockIdx.x >= nbd) {
        pf_block(blockIdx.x - nbd, g.nrb, rbg, item);
        pf_res_block<NT, NS, RBG, F_GROUPED | F_O16>(g, rbg, item, sm);
    } else {
        pf_block(blockIdx.x, d.nrb, rbg, item);
        pf_res_block<NT, NS, RBG, 0>(d, rbg, item, sm);
    }
}

// v . A-row over K inputs in one wave (fp16 x fp16 into fp32), every load of a 4096-input
// chunk issued before its sum.
__device__ __forceinline__ float wave_dot16(const uint16_t* __restrict__ arow,
                                            const uint16_t* __restrict__ vrow, int K) {
    const int lane = threadIdx.x & 63;
    float acc = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 4096) {
        uint4 av[8], xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + lane * 8 + i * 512;
            if (k < K) {
                av[i] = *reinterpret_cast<const uint4*>(arow + k);
                xv[i] = *reinterpret_cast<const uint4*>(vrow + k);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (k0 + lane * 8 + i * 512 < K) {
                const f16x2* ah = reinterpret_cast<const f16x2*>(&av[i]);
                const f16x2* xh = reinterpret_cast<const f16x2*>(&xv[i]);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_fdot2(ah[q], xh[q], acc, false);
            }
        }
    }
    return seg_sum<64>(acc);
}

// Partial LoRA z over inputs k0 .. k0 + 255 for adapter ad: zpart[t][r] = A[ad][r][k0..] .
// v[t][k0..] for those of the 16 tokens t0.. that use adapter ad and 16 rank rows r0.. of one
// projection.  One wave, 8 MFMAs with every load issued first: the tokens' v as A and the fp16
// LoRA rows as B, both straight from memory in the same k order; fp16 products are exact in
// fp32.  A wave whose adapter no token of the tile uses returns at once.
__device__ void lora_z_chunk(const uint16_t* __restrict__ v, int T, int K,
                             const uint16_t* __restrict__ A, int rank, int nad, int ad,
                             const int32_t* __restrict__ adapter, float* __restrict__ zpart,
                             int t0, int r0, int k0) {
    const int lane = threadIdx.x & 63, col = lane & 15, j = lane >> 4;
    const int tok = min(t0 + col, T - 1);
    if (!__any(lane < 16 && t0 + col < T && adapter_of(adapter, tok, nad) == ad)) return;
    const int rrow = min(r0 + col, rank - 1);
    const uint16_t* vrow = v + (long)tok * K + k0 + 8 * j;
    const uint16_t* arow = A + ((long)ad * rank + rrow) * K + k0 + 8 * j;
    uint4 xa[8], wb[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        xa[m] = *reinterpret_cast<const uint4*>(vrow + 32 * m);
        wb[m] = *reinterpret_cast<const uint4*>(arow + 32 * m);
    }
    int tad[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) tad[q] = adapter_of(adapter, min(t0 + 4 * j + q, T - 1), nad);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 8; ++m)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, xa[m]),
                                                     __builtin_bit_cast(f16x8, wb[m]), acc, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = t0 + 4 * j + q;
        if (t < T && tad[q] == ad && r0 + col < rank) zpart[(long)t * MAX_RANK + r0 + col] = acc[q];
    }
}

struct XsideArgs {
    PfGemm router, shared;
    int nb_router, nb_shared, zjobs;
};

// LoRA z jobs of one projection: (adapter, 16-token tile, 16-row rank tile, 256-input chunk).
__host__ __device__ inline int lora_z_jobs(int T, int H, int rank, int nad) {
    return nad * ((T + 15) / 16) * ((rank + 15) / 16) * (H / 256);
}

// x side of the layer in one launch: the router rows plus the shared-gate row (8-bit), the
// shared expert's gate and up (int4), all as split-K partial sums, then the LoRA z's of the
// shared gate and up as partial sums over 256-input chunks (one wave per lora_z_chunk job).
// NT: token tiles of 16 per block (4; 1 for at most 16 tokens, which would otherwise pad
// three of the four tiles).
template <int NS, int NT>
__global__ void __launch_bounds__(256) k_pf_xside(XsideArgs xa, MoeArgs a) {
    __shared__ __align__(16) PfSmem<4, 2, NS> sm;
    const int b = blockIdx.x;
    int rb, item;
    if (b < xa.nb_router) {
        pf_block(b, xa.router.nrb, rb, item);
        pf_gemm_block<1, 8, NT, F_EXTRA, NS, 2>(xa.router, rb, item, sm);
        return;
    }
    if (b < xa.nb_router + xa.nb_shared) {
        pf_block(b - xa.nb_router, xa.shared.nrb, rb, item);
        pf_gemm_block<2, 4, NT, 0, NS, 2>(xa.shared, rb, item, sm);
        return;
    }
    const int jb = (b - xa.nb_router - xa.nb_shared) * 4 + (threadIdx.x >> 6);
    if (jb >= xa.zjobs) return;
    const int ng = a.Ag ? lora_z_jobs(a.T, a.H, a.rg, a.nag) : 0;
    const bool isg = jb < ng;
    int jj = isg ? jb : jb - ng;
    const int rank = isg ? a.rg : a.ru, nad = isg ? a.nag : a.nau;
    const int kc = a.H / 256, rtiles = (rank + 15) / 16, tt = (a.T + 15) / 16;
    const int c = jj % kc;
    jj /= kc;
    const int rt = jj % rtiles;
    jj /= rtiles;
    const int tile = jj % tt, ad = jj / tt;
    lora_z_chunk(a.x, a.T, a.H, isg ? a.Ag : a.Au, rank, nad, ad, a.adapter,
                 (isg ? a.zg : a.zu) + (long)c * a.T * MAX_RANK, tile * 16, rt * 16, c * 256);
}

// The n <= KP split-K partials p[s * stride] of one value, every load issued at once (index
// clamped into the n partials), summed in split order.
template <int KP>
struct Parts {
    float v[KP];
    __device__ __forceinline__ void load(const float* __restrict__ p, long stride, int n) {
#pragma unroll
        for (int s = 0; s < KP; ++s) v[s] = p[(long)min(s, n - 1) * stride];
    }
    __device__ __forceinline__ float sum(int n) const {
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < KP; ++s) acc += s < n ? v[s] : 0.0f;
        return acc;
    }
};

// Wave 0 of k_pf_token: the token's router logits (split-K sums, PER per lane, in registers)
// plus the selection bias, then top-K; lane 0 leaves the experts and weights in sel / sw.
template <int PER, int KP>
__device__ void token_topk(const MoeArgs& a, int t, int ksplit, int* sel, float* sw) {
    const int lane = threadIdx.x & 63;
    TopkKeys<PER, false> keys;
    keys.has_bias = a.rbias != nullptr;
    const float* bias = keys.has_bias ? a.rbias : a.logits;   // read either way, used if bias
    Parts<KP> p[PER];
    float b[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = min(lane * PER + i, a.E - 1);
        p[i].load(a.logits + (long)t * a.Ep + e, (long)a.T * a.Ep, ksplit);
        b[i] = bias[e];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        keys.raw[i] = p[i].sum(ksplit);
        keys.braw[i] = keys.has_bias ? b[i] : 0.0f;
    }
    keys.select(a.E, a.K, sel, sw);
}

// Wave 0 of k_pf_token for a given routing (the caller's selection): lane k < K takes
// expert k of the token's routing (clamped) and its logit (split-K partials plus the bias);
// the weights are the softmax over the K, with the operations and order of given_softmax
// (maximum and sum taken lane by lane in selection order).  Lanes 0 .. K-1 leave the experts
// and weights in sel / sw.
template <int KP>
__device__ void token_given(const MoeArgs& a, int t, int ksplit, int* sel, float* sw) {
    const int lane = threadIdx.x & 63, K = a.K;
    const int e = clamp_expert(a.route[(long)t * K + min(lane, K - 1)], a.E);
    Parts<KP> p;
    p.load(a.logits + (long)t * a.Ep + e, (long)a.T * a.Ep, ksplit);
    float l = p.sum(ksplit);
    if (a.rbias) l += a.rbias[e];
    float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), 0));
    for (int i = 1; i < K; ++i)
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i)));
    const float ex = expf(l - m);
    float total = 0.0f;
    for (int i = 0; i < K; ++i)
        total += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), i));
    if (lane < K) {
        sel[lane] = e;
        sw[lane] = ex / total;
    }
}

// The remaining rank entries 16 .. rank - 1 (rank a multiple of 8) of the same dot.
__device__ __forceinline__ float bdot_tail(const uint16_t* __restrict__ brow, const float* z,
                                           int rank, float d) {
    for (int r = 16; r < rank; r += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(brow + r);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            d = fmaf(half_lo(w4[j]), z[r + 2 * j], d);
            d = fmaf(half_hi(w4[j]), z[r + 2 * j + 1], d);
        }
    }
    return d;
}

constexpr int TOK_HW = 3;   // waves of k_pf_token on the shared expert's h
constexpr int TOK_NPC = 4;  // h outputs per thread whose loads are issued together (few tokens)
constexpr int TOK_WIDE_T = 256;  // up to this many tokens: blocks of 8 waves (7 on h_s, 2 outputs each)

// Per-token finish of the x side, one block of 4 waves per token.  Wave 0 sums the token's
// router-logit partials in registers and runs top-K.  Waves 1-3 sum the shared-gate logit and
// (each for itself, into its own LDS row) the LoRA z's of gate and up, then h_s =
// silu(g_s + LoRA_g) * (u_s + LoRA_u), every load of NPC outputs issued together; h_s goes to
// LDS.  With NPC > 1 every wave meanwhile fetches its first rows of the down LoRA's A.  After
// the one barrier:
// h_s and the selection are written out and z_d = A_down h_s is taken, one wave per four rank
// rows.  Split-K partials are added in split order, LoRA chunks in chunk order.
template <int KP, int PER, int NPC, int HW>
__device__ __forceinline__ void pf_token_body(const MoeArgs& a, int ksplit) {
    constexpr int NTB = 64 * (HW + 1);   // threads per block
    extern __shared__ __align__(16) uint16_t hl[];        // h_s of the token, fp16 [SI]
    __shared__ int sel[MAX_K];
    __shared__ float sw[MAX_K];
    __shared__ float zw[HW][2][MAX_RANK];
    const int t = blockIdx.x, T = a.T, SI = a.SI;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

    // first rows of the down LoRA: rows 4 wave .. + 3, inputs lane * 8 + 512 i (clamped)
    const bool has_d = a.Ad != nullptr;
    const uint16_t* abase = has_d ? a.Ad + (long)adapter_of(a.adapter, t, a.nad) * a.rd * SI : a.hs;
    const long astride = has_d ? SI : 0;
    const int rd = has_d ? a.rd : 0;
    // (few tokens only: with many, the registers go to more tokens in flight instead)
    constexpr bool PRE = NPC > 1;
    uint4 av0[PRE ? 4 : 1][2];
    if constexpr (PRE) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av0[q][i] = *reinterpret_cast<const uint4*>(abase + min(4 * wave + q, max(rd - 1, 0)) * astride +
                                                            min(lane * 8 + i * 512, SI - 8));
    }

    if (wave == 0) {
        if (a.route) token_given<KP>(a, t, ksplit, sel, sw);
        else token_topk<PER, KP>(a, t, ksplit, sel, sw);
    } else {
        const int w = wave - 1, u = threadIdx.x - 64;
        Parts<KP> g;   // the shared-gate logit (every lane loads, one stores)
        g.load(a.gate + t, T, ksplit);
        const long pz = (long)T * MAX_RANK, pgu = (long)T * SI;
        const int kc = a.H / 256;
        Parts<2 * KP> zg, zu;
        zg.load(a.zg + (long)t * MAX_RANK + lane, pz, kc);
        zu.load(a.zu + (long)t * MAX_RANK + lane, pz, kc);
        const int adg = adapter_of(a.adapter, t, a.nag), adu = adapter_of(a.adapter, t, a.nau);
        const bool fg = a.Bg && (a.rg & 7) == 0, fu = a.Bu && (a.ru & 7) == 0;
        const uint16_t* gb = fg ? a.Bg + (long)adg * SI * a.rg : a.hs;
        const uint16_t* ub = fu ? a.Bu + (long)adu * SI * a.ru : a.hs;
        const int gs = fg ? a.rg : 0, us = fu ? a.ru : 0;
        const int g8 = max(min(a.rg, 16) - 8, 0), u8 = max(min(a.ru, 16) - 8, 0);
        bool first = true;
        for (int n0 = u; n0 < SI; n0 += NPC * HW * 64) {
            Parts<KP> pg[NPC], pu[NPC];
            uint4 bg[NPC][2], bu[NPC][2];
#pragma unroll
            for (int c = 0; c < NPC; ++c) {
                const int n = min(n0 + c * HW * 64, SI - 1);
                pg[c].load(a.gs + (long)t * SI + n, pgu, ksplit);
                pu[c].load(a.us + (long)t * SI + n, pgu, ksplit);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    bg[c][i] = *reinterpret_cast<const uint4*>(gb + (long)n * gs + min(8 * i, g8));
                    bu[c][i] = *reinterpret_cast<const uint4*>(ub + (long)n * us + min(8 * i, u8));
                }
            }
            if (first) {   // this wave's LoRA z's, read back by every lane below
                zw[w][0][lane] = zg.sum(kc);
                zw[w][1][lane] = zu.sum(kc);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                first = false;
            }
#pragma unroll
            for (int c = 0; c < NPC; ++c) {
                const int n = n0 + c * HW * 64;
                if (n < SI) {
                    float gv = pg[c].sum(ksplit), uv = pu[c].sum(ksplit);
                    if (a.Bg) {
                        const float d = fg ? bdot_tail(gb + (long)n * gs, zw[w][0], a.rg, bdot16(bg[c], zw[w][0], a.rg))
                                           : lora_b_dot(a.Bg, adg, SI, n, a.rg, zw[w][0]);
                        gv = fmaf(a.lsg, d, gv);
                    }
                    if (a.Bu) {
                        const float d = fu ? bdot_tail(ub + (long)n * us, zw[w][1], a.ru, bdot16(bu[c], zw[w][1], a.ru))
                                           : lora_b_dot(a.Bu, adu, SI, n, a.ru, zw[w][1]);
                        uv = fmaf(a.lsu, d, uv);
                    }
                    hl[n] = f2h(silu(gv) * uv);
                }
            }
        }
        if (u == 0) a.gate[t] = g.sum(ksplit);   // split 0's slot holds the sum
    }
    __syncthreads();

    for (int n = threadIdx.x * 8; n < SI; n += NTB * 8)
        *reinterpret_cast<uint4*>(a.hs + (long)t * SI + n) = *reinterpret_cast<const uint4*>(hl + n);
    if (threadIdx.x < a.K) {
        const long i = (long)t * a.K + threadIdx.x;
        a.idx[i] = sel[threadIdx.x];
        a.wts[i] = sw[threadIdx.x];
        if (a.idx_out) a.idx_out[i] = sel[threadIdx.x];
        if (a.w_out) a.w_out[i] = sw[threadIdx.x];
    }
    if (!has_d) return;
    // z_d: rows r0 .. r0 + 3 per wave, 1024 inputs (2 x 8 per lane) per pass
    auto pass = [&](const auto& av, int k0, float (&acc)[4]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = k0 + lane * 8 + i * 512;
            if (k < SI) {
                const uint4 xv = *reinterpret_cast<const uint4*>(hl + k);
                const f16x2* xh = reinterpret_cast<const f16x2*>(&xv);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x2* ah = reinterpret_cast<const f16x2*>(&av[q][i]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[q] = __builtin_amdgcn_fdot2(ah[e], xh[e], acc[q], false);
                }
            }
        }
    };
    for (int r0 = 4 * wave; r0 < rd; r0 += 4 * (HW + 1)) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < SI; k0 += 1024) {
            if (PRE && r0 == 4 * wave && k0 == 0) {
                pass(av0, 0, acc);
            } else {
                uint4 av[4][2];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        av[q][i] = *reinterpret_cast<const uint4*>(abase + min(r0 + q, rd - 1) * astride +
                                                                   min(k0 + lane * 8 + i * 512, SI - 8));
                pass(av, k0, acc);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v = seg_sum<64>(acc[q]);
            if (lane == 0 && r0 + q < rd) a.zd[(long)t * MAX_RANK + r0 + q] = v;
        }
    }
}

// Few tokens: every block in flight at once, each issuing all its loads together.  PER:
// logits per lane of the top-K (4 up to 256 experts, else 16), fixed per kernel so that one
// kernel holds one selection.
template <int KP, int PER>
__global__ void __launch_bounds__(256) k_pf_token(MoeArgs a, int ksplit) { pf_token_body<KP, PER, TOK_NPC, TOK_HW>(a, ksplit); }

// Few tokens (at most TOK_WIDE_T: all blocks resident at once): eight waves per block, seven
// of them on h_s with two outputs each, so each thread's chain of loads is shorter (measured
// faster at 16 and 256 tokens, slower at 512, where the blocks no longer all fit at once).
template <int KP, int PER>
__global__ void __launch_bounds__(512) k_pf_token_wide(MoeArgs a, int ksplit) { pf_token_body<KP, PER, 2, 7>(a, ksplit); }

// Many tokens (several rounds of blocks): one h output per thread in flight, so that four waves
// fit a SIMD and twice the tokens are in flight.
template <int KP, int PER>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
k_pf_token_many(MoeArgs a, int ksplit) { pf_token_body<KP, PER, 1, TOK_HW>(a, ksplit); }

// The per-token kernel for T tokens: KP split-K partials, PER logits per lane.
template <int PER>
void launch_token(const MoeArgs& a, int ksplit, int kp, size_t tsm, hipStream_t s) {
    // (the eight-wave form for up to 256 experts: with 16 logits per lane it would spill)
    if (PER == 4 && a.T <= TOK_WIDE_T) {
        if constexpr (PER == 4) {
            if (kp <= 2) k_pf_token_wide<2, PER><<<a.T, 512, tsm, s>>>(a, ksplit);
            else if (kp <= 4) k_pf_token_wide<4, PER><<<a.T, 512, tsm, s>>>(a, ksplit);
            else k_pf_token_wide<8, PER><<<a.T, 512, tsm, s>>>(a, ksplit);
        }
    } else if (a.T < PF_MANY_T) {
        if (kp <= 2) k_pf_token<2, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
        else if (kp <= 4) k_pf_token<4, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
        else k_pf_token<8, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
    } else {   // (eight partials do not fit the four-wave budget: the few-token kernel)
        if (kp <= 2) k_pf_token_many<2, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
        else if (kp <= 4) k_pf_token_many<4, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
        else k_pf_token<8, PER><<<a.T, 256, tsm, s>>>(a, ksplit);
    }
}

// Exclusive prefix sum over a block of 1024 threads; the total goes to *total.
__device__ int block_scan_excl(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_scan(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int s = lane < 16 ? wsum[lane] : 0;
        const int si = wave_scan(s);
        if (lane < 16) wsum[16 + lane] = si - s;
        if (lane == 15) *total = si;
    }
    __syncthreads();
    const int r = inc - v + wsum[16 + wave];
    __syncthreads();   // wsum is reused by the next scan
    return r;
}

// Stable ranks, per expert, of one chunk of 1024 pairs (thread tid holds pair s0 + tid of
// expert ex; valid: the pair exists).  Lanes with the same expert are found by ballots on
// the expert's index bits, which gives each pair its rank among them in its wave; the waves'
// counts per expert are then offset by a prefix over the chunk's 16 waves (tab, LDS).
// Returns the pair's rank among the chunk's pairs of its expert; cnt[e] (tid = e < E) gets the
// chunk's count of expert e.  Every thread of the block calls it.
__device__ int chunk_rank(int ex, bool valid, int E, uint16_t (&tab)[16][1024], int* cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ebits = E > 1 ? 32 - __builtin_clz(E - 1) : 0;
    uint64_t same = __ballot(valid);
    for (int bt = 0; bt < ebits; ++bt) {
        const bool bit = (ex >> bt) & 1;
        const uint64_t bb = __ballot(bit);
        same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1));
    if (tid < E)
        for (int w = 0; w < 16; ++w) tab[w][tid] = 0;
    __syncthreads();
    if (valid && rank == 0) tab[wave][ex] = (uint16_t)__popcll(same);
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < 16; ++w) {
            const int v = tab[w][tid];
            tab[w][tid] = (uint16_t)run;
            run += v;
        }
        cnt[tid] = run;
    }
    __syncthreads();
    return valid ? tab[wave][ex] + rank : 0;
}

// The work items of expert e (tid = e < E; count c, first item wex): records (expert,
// tokens) of chunks of at most isz pairs.
__device__ __forceinline__ void write_records(const MoeArgs& a, int c, int wex, int isz) {
    const int nw = (c + isz - 1) / isz;
    for (int w = 0; w < nw; ++w)
        reinterpret_cast<int4*>(a.wrec)[wex + w] = int4{(int)threadIdx.x, min(isz, c - w * isz), 0, 0};
}

// Stable counting sort of the (token, k) pairs by expert (pair p = t * K + k), written as
// GEMM work items: chunks of at most isz pairs of one expert, each a record (expert,
// tokens) and its pair ids (PF_ITEM slots per item); records past the last item get zero
// tokens.  One block of 1024 threads over chunks of 1024 pairs.
__global__ void __launch_bounds__(1024) k_pf_sort(MoeArgs a, int max_items, int isz) {
    __shared__ int cnt[1024], base[1024], ewex[1024], wsum[32], tot;
    __shared__ uint16_t tab[16][1024];
    const int tid = threadIdx.x;
    const int E = a.E, TK = a.T * a.K;
    cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < TK; p += 1024) atomicAdd(&cnt[a.idx[p]], 1);
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    const int wex = block_scan_excl((c + isz - 1) / isz, wsum, &tot);
    if (tid < E) {
        base[tid] = 0;   // pairs of expert tid in the chunks before
        ewex[tid] = wex;
        write_records(a, c, wex, isz);
    }
    __syncthreads();
    for (int it = tot + tid; it < max_items; it += 1024) reinterpret_cast<int4*>(a.wrec)[it] = int4{0, 0, 0, 0};
    for (int s0 = 0; s0 < TK; s0 += 1024) {
        const int p = s0 + tid;
        const bool valid = p < TK;
        const int ex = valid ? a.idx[p] : 0;
        const int r = chunk_rank(ex, valid, E, tab, cnt);
        if (valid) {
            const int q = base[ex] + r;   // the pair's rank among the pairs of its expert
            a.wpairs[(long)(ewex[ex] + q / isz) * PF_ITEM + q % isz] = p;
        }
        __syncthreads();
        if (tid < E) base[tid] += cnt[tid];
        __syncthreads();
    }
}

// Chunks of 1024 pairs per block of the multi-block sort (at most PF_SORT_MAXSEG blocks).
__host__ __device__ inline int sort_chunks_per_block(int TK) {
    const int chunks = (TK + 1023) / 1024;
    return (chunks + PF_SORT_MAXSEG - 1) / PF_SORT_MAXSEG;
}

// Multi-block sort, pass 1: block s counts the experts of its segment (cpb chunks of 1024
// pairs) into scnt[s][e].
__global__ void __launch_bounds__(1024) k_pf_count(MoeArgs a, int cpb) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x, E = a.E, TK = a.T * a.K;
    const int p0 = blockIdx.x * cpb * 1024;
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    for (int c = 0; c < cpb; ++c) {
        const int p = p0 + c * 1024 + tid;
        if (p < TK) atomicAdd(&cnt[a.idx[p]], 1);
    }
    __syncthreads();
    if (tid < E) a.scnt[(long)blockIdx.x * E + tid] = cnt[tid];
}

// Multi-block sort, pass 2: block s places the pairs of its segment.  Each block forms from
// the segments' counts the rank, inside expert e, of its segment's first pair of e (the
// counts of the earlier segments) and the items of every expert (a block scan of the totals);
// block 0 writes the item records.  Inside the segment the ranks are those of k_pf_sort, so
// the items hold the same pairs in the same order.
__global__ void __launch_bounds__(1024) k_pf_place(MoeArgs a, int max_items, int isz, int cpb, int nseg) {
    __shared__ int cnt[1024], base[1024], ewex[1024], wsum[32], tot;
    __shared__ uint16_t tab[16][1024];
    const int tid = threadIdx.x, E = a.E, TK = a.T * a.K, s = blockIdx.x;
    int before = 0, total = 0;
    if (tid < E) {
        for (int q = 0; q < nseg; ++q) {
            const int c = a.scnt[(long)q * E + tid];
            total += c;
            before += q < s ? c : 0;
        }
    }
    const int wex = block_scan_excl((total + isz - 1) / isz, wsum, &tot);
    if (tid < E) {
        base[tid] = before;
        ewex[tid] = wex;
        if (s == 0) write_records(a, total, wex, isz);
    }
    if (s == 0)
        for (int it = tot + tid; it < max_items; it += 1024) reinterpret_cast<int4*>(a.wrec)[it] = int4{0, 0, 0, 0};
    __syncthreads();
    const int p0 = s * cpb * 1024;
    for (int c = 0; c < cpb; ++c) {
        const int p = p0 + c * 1024 + tid;
        const bool valid = p < TK;
        const int ex = valid ? a.idx[p] : 0;
        const int r = chunk_rank(ex, valid, E, tab, cnt);
        if (valid) {
            const int q = base[ex] + r;
            a.wpairs[(long)(ewex[ex] + q / isz) * PF_ITEM + q % isz] = p;
        }
        __syncthreads();
        if (tid < E) base[tid] += cnt[tid];
        __syncthreads();
    }
}

// y = fp16(sum_k w_k o_k + sigmoid(gate) (os + LoRA_down)) (+ residual), k in order, with the
// experts' outputs o_k held in fp16.  FPT outputs of one token per thread (8, or 4 with many
// tokens).  Every load
// of the common case (up to KF experts, LoRA rank a multiple of 8 up to 16) is issued before
// any use, one memory round trip: the experts' rows and weights, the shared output and gate
// logit, the residual, the FPT LoRA-B rows (contiguous) and z_d.  Absent operands are read
// from a valid stand-in and not used; more experts or a larger rank continue with further
// passes.
template <int KF, int FPT>
__device__ __forceinline__ void pf_combine_body(const MoeArgs& a) {
    constexpr int TPR = 128 / FPT, TPB = 256 / TPR, NV = FPT / 4;   // threads per token row, tokens per block
    using XV = std::conditional_t<FPT == 8, uint4, uint2>;          // FPT fp16 values
    // block: TPB tokens x 128 features, so the block's LoRA-B rows (128 x rank) are read
    // from L2 once and shared by its tokens through L1
    const int nch = a.H / 128, ch = blockIdx.x % nch;
    const int t = (blockIdx.x / nch) * TPB + threadIdx.x / TPR;
    if (t >= a.T) return;
    const int n = ch * 128 + (threadIdx.x % TPR) * FPT;
    const long i8 = (long)t * a.H + n;
    const int K = a.K;
    XV p[KF];   // the experts' down outputs, fp16
    float w[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) {
        const int k = min(u, K - 1);
        w[u] = a.wts[(long)t * K + k];
        p[u] = *reinterpret_cast<const XV*>(a.o + ((long)t * K + k) * a.H + n);
    }
    float4 osv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) osv[v] = reinterpret_cast<const float4*>(a.os + i8)[v];
    const float g = a.gate[t];
    const XV xr = *reinterpret_cast<const XV*>(a.x + i8);
    const bool bfast = a.Bd && (a.rd & 7) == 0;
    const int rv = bfast ? a.rd / 8 : 1;   // uint4 per B row
    const int ad = a.Bd ? adapter_of(a.adapter, t, a.nad) : 0;
    // FPT rows of rd halves are FPT rd contiguous halves; stand-in: the shared output
    const uint4* b4 = bfast ? reinterpret_cast<const uint4*>(a.Bd + ((long)ad * a.H + n) * a.rd)
                            : reinterpret_cast<const uint4*>(a.os + i8);
    const float* z = a.zd + (long)t * MAX_RANK;
    uint4 bv[FPT][2];
    float4 zv[4];
#pragma unroll
    for (int q = 0; q < FPT; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i) bv[q][i] = b4[bfast ? q * rv + min(i, rv - 1) : 0];
#pragma unroll
    for (int i = 0; i < 4; ++i) zv[i] = reinterpret_cast<const float4*>(z)[i];

    float ov[FPT];
#pragma unroll
    for (int q = 0; q < FPT; ++q) ov[q] = reinterpret_cast<const float*>(osv)[q];
    if (bfast) {
        float d[FPT];
#pragma unroll
        for (int q = 0; q < FPT; ++q) d[q] = 0.0f;
        const float* zf = reinterpret_cast<const float*>(zv);
        auto add = [&](const uint4 (&v)[FPT], const float* zs) {   // one uint4 per row: 8 ranks
#pragma unroll
            for (int q = 0; q < FPT; ++q) {
                const uint32_t w4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    d[q] = fmaf(half_lo(w4[u]), zs[2 * u], d[q]);
                    d[q] = fmaf(half_hi(w4[u]), zs[2 * u + 1], d[q]);
                }
            }
        };
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i < rv) {
                uint4 v[FPT];
#pragma unroll
                for (int q = 0; q < FPT; ++q) v[q] = bv[q][i];
                add(v, zf + 8 * i);
            }
        }
        for (int r = 2; r < rv; ++r) {   // ranks past 16
            uint4 v[FPT];
#pragma unroll
            for (int q = 0; q < FPT; ++q) v[q] = b4[q * rv + r];
            add(v, z + 8 * r);
        }
#pragma unroll
        for (int q = 0; q < FPT; ++q) ov[q] = fmaf(a.lsd, d[q], ov[q]);
    } else if (a.Bd) {
#pragma unroll
        for (int q = 0; q < FPT; ++q) ov[q] = fmaf(a.lsd, lora_b_dot(a.Bd, ad, a.H, n + q, a.rd, z), ov[q]);
    }
    float acc[FPT];
#pragma unroll
    for (int q = 0; q < FPT; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int u = 0; u < KF; ++u) {
        if (u < K) {
            const uint16_t* pv = reinterpret_cast<const uint16_t*>(&p[u]);
#pragma unroll
            for (int q = 0; q < FPT; ++q) acc[q] = fmaf(w[u], h2f(pv[q]), acc[q]);
        }
    }
    for (int k = KF; k < K; ++k) {   // experts past the KF-th
        const float wk = a.wts[(long)t * K + k];
        const XV qv = *reinterpret_cast<const XV*>(a.o + ((long)t * K + k) * a.H + n);
        const uint16_t* pv = reinterpret_cast<const uint16_t*>(&qv);
#pragma unroll
        for (int q = 0; q < FPT; ++q) acc[q] = fmaf(wk, h2f(pv[q]), acc[q]);
    }
    const float gm = sigmoid(g);
    uint16_t out[FPT];
#pragma unroll
    for (int q = 0; q < FPT; ++q) out[q] = f2h(fmaf(gm, ov[q], acc[q]));
    if (a.add_residual) {
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(&xr);
#pragma unroll
        for (int q = 0; q < FPT; ++q) out[q] = f2h(h2f(xh[q]) + h2f(out[q]));
    }
    *reinterpret_cast<XV*>(a.y + i8) = *reinterpret_cast<const XV*>(out);
}

// Few tokens: up to eight experts' rows per thread in flight at once.
__global__ void __launch_bounds__(256) k_pf_combine(MoeArgs a) { pf_combine_body<8, 8>(a); }

// Many tokens: four outputs per thread and KF experts' rows in flight (KF = top-K when it is
// at most 4), so that four waves fit a SIMD.
template <int KF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
k_pf_combine_many(MoeArgs a) { pf_combine_body<KF, 4>(a); }

// ---------------------------------------------------------------------------- large items
// Grouped GEMM for work items of up to PB_TOK pairs (experts averaging more than 64 pairs),
// where the GEMMs are bound by the matrix cores.  v_mfma_f32_32x32x16_f16 (on gfx950 it
// keeps the matrix pipe about 1.5x busier per instruction than 16x16x32, measured back to
// back), a block of 4 waves covering PB_ROWS = 128 features (32 per wave) of NMAT matrices
// against 32 NTT token rows (NTT tiles of 32: the item's tokens rounded up, one body per
// tile count, so no branch sits between the MFMAs).
//   A (activations, 32 tokens x 16 inputs): lane l supplies token l % 32 and inputs
//     8 (l / 32) .. +7 of the k-slice, from an LDS double buffer staged per 128-input step
//     in the pair order of the nibble unpacking (pf_commit).
//   B (weights, 16 inputs x 32 features): lane l supplies feature l % 32 and the same
//     inputs, dequantized in registers to fp16(s q + b) (pf_q4, pf_dequant).  A lane loads 8
//     consecutive packed words of its feature's 128-input step (the lower 64 inputs for
//     l < 32, the upper 64 otherwise); v_permlane32_swap of word pairs (2i, 2i + 1) then
//     leaves lane l < 32 the even words 0, 8, 2, 10, 4, 12, 6, 14 and lane l + 32 the odd
//     ones 1, 9, 3, 11, ..., i.e. for k-slice s the word 2 s + l / 32 in register 2 s
//     (s < 4) or 2 (s - 4) + 1 (s >= 4).
//   Output tile c of matrix m: 16 floats per lane, token 8 (v / 4) + 4 (l / 32) + v % 4,
//     feature l % 32.
// Each weight is dequantized once per block and feeds NTT MFMAs per matrix; the activation
// fragments of a k-slice feed NMAT MFMAs each.  Weights and scales are loaded two steps
// ahead, the next step's activations one step ahead (staged at the top of the step).
constexpr int PB_TOK = 128;    // pairs per large work item
constexpr int PB_ROWS = 128;   // features per block

template <int NTT>
struct PbSmem {
    f16 tile[2][32 * NTT * PF_PITCH];
    int arow[32 * NTT], orow[32 * NTT];
};

template <int NMAT, int NTT, int NS, int FL, int NTS>
__device__ __forceinline__ void pb_body(const PfGemm& a, int rb, int ntok, int e, PbSmem<NTS>& sm) {
    constexpr int K = NS * PF_KS, G = K / 64, WPS = PF_KS / 8, WPR = K / 8;
    constexpr int NQ = 2 * NTT;   // 16-byte activation units per thread per step
    constexpr int D = 2;          // weight steps in flight
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int n = rb * PB_ROWS + wave * 32 + col;
    const long row = (long)e * a.N + min(n, a.N - 1);   // rows past N clamped, never stored
    const uint32_t* wrow[NMAT];
    const uint32_t* srow[NMAT];
    const uint32_t* brow[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        wrow[m] = a.p[m] + row * WPR + hh * 8;
        srow[m] = reinterpret_cast<const uint32_t*>(a.s[m] + row * G);
        brow[m] = reinterpret_cast<const uint32_t*>(a.b[m] + row * G);
    }
    const int sr = threadIdx.x >> 4, sc = threadIdx.x & 15;
    const uint16_t* xrp[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) xrp[q] = a.act + (long)sm.arow[q * 16 + sr] * K + sc * 8;

    struct Slot {
        uint32_t w[NMAT][8];
        uint32_t s[NMAT], b[NMAT];   // the step's two groups as fp16 pairs
    };
    Slot ws[D];
    uint4 xr[NQ];
    auto load_w = [&](Slot& sl, int ks) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint4* src = reinterpret_cast<const uint4*>(wrow[m] + ks * WPS);
            const uint4 v0 = src[0], v1 = src[1];
            sl.w[m][0] = v0.x; sl.w[m][1] = v0.y; sl.w[m][2] = v0.z; sl.w[m][3] = v0.w;
            sl.w[m][4] = v1.x; sl.w[m][5] = v1.y; sl.w[m][6] = v1.z; sl.w[m][7] = v1.w;
            sl.s[m] = srow[m][ks];
            sl.b[m] = brow[m][ks];
        }
    };
    auto load_x = [&](int ks) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) xr[q] = *reinterpret_cast<const uint4*>(xrp[q] + ks * PF_KS);
    };
    auto commit_x = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) pf_commit<4>(xr[q], q * 16 + sr, sc, sm.tile[buf]);
    };

    f32x16 acc[NMAT][NTT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < NTT; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][c][v] = 0.0f;
    uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;   // fp16 1024 and 64 in both halves (pf_q4)
    asm volatile("" : "+v"(m1024), "+v"(m64));

    load_x(0);
#pragma unroll
    for (int d = 0; d < D; ++d) load_w(ws[d], d);
    commit_x(0);
    if (NS > 1) load_x(1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
        Slot& sl = ws[ks % D];
        uint32_t cw[NMAT][8];
        f16 sh[NMAT][2], bh[NMAT][2];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const auto r = __builtin_amdgcn_permlane32_swap(sl.w[m][2 * i], sl.w[m][2 * i + 1], false, false);
                cw[m][2 * i] = r[0];
                cw[m][2 * i + 1] = r[1];
            }
            const f16x2 s2 = as_h2(sl.s[m]), b2 = as_h2(sl.b[m]);
            sh[m][0] = s2[0]; sh[m][1] = s2[1];
            bh[m][0] = b2[0]; bh[m][1] = b2[1];
        }
        // the next step's activations into the other buffer (every wave finished reading it
        // before the barrier that ended the previous step), then the loads two steps ahead
        // into the registers just consumed
        if (ks + 1 < NS) commit_x((ks + 1) & 1);
        if (ks + 2 < NS) load_x(ks + 2);
        if (ks + D < NS) load_w(sl, ks + D);
        // k-slices of 16 inputs (two waves per SIMD: each covers the other's LDS and memory
        // latency)
        const f16* tb = sm.tile[ks & 1] + col * PF_PITCH + 8 * hh;
#pragma unroll
        for (int s16 = 0; s16 < 8; ++s16) {
            const int g = s16 >> 2, reg = s16 < 4 ? 2 * s16 : 2 * (s16 - 4) + 1;
            f16x8 bw[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) bw[m] = pf_dequant(pf_q4(cw[m][reg], m1024, m64), sh[m][g], bh[m][g]);
#pragma unroll
            for (int c = 0; c < NTT; ++c) {
                const f16x8 av = *reinterpret_cast<const f16x8*>(tb + c * 32 * PF_PITCH + 16 * s16);
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
                    acc[m][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bw[m], acc[m][c], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    if (n >= a.N) return;
#pragma unroll
    for (int c = 0; c < NTT; ++c) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = c * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (t < ntok) {
                const int orow = sm.orow[t];
                if constexpr (FL & F_HOUT)
                    a.hout[(long)orow * a.N + n] = f2h(silu(acc[0][c][v]) * acc[NMAT - 1][c][v]);
                else
                    a.hout[(long)orow * a.ostride + n] = f2h(acc[0][c][v]);
            }
        }
    }
}

// One large work item per (item, row block): its record and pair ids, then the body for the
// item's tile count.
template <int NMAT, int NS, int FL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) k_pf_big(PfGemm a) {
    __shared__ __align__(16) PbSmem<PB_TOK / 32> sm;
    int rb, item;
    pf_block(blockIdx.x, a.nrb, rb, item);
    const int4 rec = reinterpret_cast<const int4*>(a.wrec)[item];
    const int pair = threadIdx.x < PB_TOK ? a.wpairs[(long)item * PF_ITEM + threadIdx.x] : 0;
    if (rec.y == 0) return;   // past the last item
    const int e = rec.x, ntok = rec.y;
    if (threadIdx.x < PB_TOK) sm.orow[threadIdx.x] = pair;
    __syncthreads();
    if (threadIdx.x < PB_TOK) sm.arow[threadIdx.x] = sm.orow[min((int)threadIdx.x, ntok - 1)] / a.act_div;
    __syncthreads();
    switch ((ntok + 31) >> 5) {
        case 1: pb_body<NMAT, 1, NS, FL>(a, rb, ntok, e, sm); break;
        case 2: pb_body<NMAT, 2, NS, FL>(a, rb, ntok, e, sm); break;
        case 3: pb_body<NMAT, 3, NS, FL>(a, rb, ntok, e, sm); break;
        default: pb_body<NMAT, 4, NS, FL>(a, rb, ntok, e, sm); break;
    }
}

// The large-item GEMMs exist for reductions of 512, 1024 and 2048 inputs (4, 8, 16 steps).
bool big_steps_ok(int k) { return k == 512 || k == 1024 || k == 2048; }

template <int NMAT, int FL>
hipError_t launch_big(const PfGemm& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nrb * p.items));
    switch (p.K) {
        case 512: k_pf_big<NMAT, 4, FL><<<grid, 256, 0, s>>>(p); break;
        case 1024: k_pf_big<NMAT, 8, FL><<<grid, 256, 0, s>>>(p); break;
        case 2048: k_pf_big<NMAT, 16, FL><<<grid, 256, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;   // prefill_item_size never selects it then
    }
    return hipSuccess;
}

template <int NMAT, int BITS, int NT, int FL>
void pf_gemm(const PfGemm& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nrb * p.items));
    switch (p.K / PF_KS) {
        case 4: k_pf_gemm<NMAT, BITS, NT, FL, 4><<<grid, 256, 0, s>>>(p); break;
        case 8: k_pf_gemm<NMAT, BITS, NT, FL, 8><<<grid, 256, 0, s>>>(p); break;
        case 16: k_pf_gemm<NMAT, BITS, NT, FL, 16><<<grid, 256, 0, s>>>(p); break;
        default: k_pf_gemm<NMAT, BITS, NT, FL, 0><<<grid, 256, 0, s>>>(p); break;
    }
}

// The grouped fp16-weight GEMM with its parameters staged in LDS (reductions of 512, 1024 or
// 2048 inputs), one or four token tiles: the routed experts' GEMMs in groups of 32 or with
// bf16 parameters.
template <int NMAT, int FL>
hipError_t pf_gemm_staged(const PfGemm& p, int nt, hipStream_t s) {
    const dim3 grid((unsigned)(p.nrb * p.items));
    switch ((p.K / PF_KS) * 8 + nt) {
        case 4 * 8 + 1: k_pf_gemm<NMAT, 4, 1, FL, 4><<<grid, 256, 0, s>>>(p); break;
        case 4 * 8 + 4: k_pf_gemm<NMAT, 4, 4, FL, 4><<<grid, 256, 0, s>>>(p); break;
        case 8 * 8 + 1: k_pf_gemm<NMAT, 4, 1, FL, 8><<<grid, 256, 0, s>>>(p); break;
        case 8 * 8 + 4: k_pf_gemm<NMAT, 4, 4, FL, 8><<<grid, 256, 0, s>>>(p); break;
        case 16 * 8 + 1: k_pf_gemm<NMAT, 4, 1, FL, 16><<<grid, 256, 0, s>>>(p); break;
        case 16 * 8 + 4: k_pf_gemm<NMAT, 4, 4, FL, 16><<<grid, 256, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;   // the layer check admits no other shape
    }
    return hipSuccess;
}

// Arguments of one GEMM over `feat` feature rows (N plus an optional extra row) and `items`
// token groups or work items.
PfGemm gemm_args(const QW& w0, const QW* w1, int N, int K, const uint16_t* act, int feat,
                 int items) {
    PfGemm p{};
    p.p[0] = w0.p; p.s[0] = w0.s; p.b[0] = w0.b;
    if (w1) { p.p[1] = w1->p; p.s[1] = w1->s; p.b[1] = w1->b; }
    p.N = N; p.K = K; p.act = act; p.ostride = N;
    p.ksplit = 1;
    p.nrb = (feat + PF_ROWS - 1) / PF_ROWS;
    p.items = (items + 7) / 8 * 8;
    return p;
}

// ib_isz > 0: items formed in the block (item_in_block) with that many pairs per item.
PfGemm grouped(const MoeArgs& a, const QW& w0, const QW* w1, int N, int K, const uint16_t* act,
               int act_div, int items, int ib_isz) {
    PfGemm p = gemm_args(w0, w1, N, K, act, N, items);
    p.act_div = act_div;
    p.wrec = a.wrec; p.wpairs = a.wpairs;
    if (ib_isz > 0) {
        p.ridx = a.idx;
        p.rtk = a.T * a.K;
        p.risz = ib_isz;
        p.rE = a.E;
    }
    return p;
}

}  // namespace

// Pairs per work item: 16 (one token tile: no activation loads for a second, mostly padding
// tile) while experts average at most 8 pairs, so that few experts need a second item and a
// second pass over their weights; 32 up to an average of 32; 64 up to 64 (four tiles: each
// weight step feeds four times the MFMA work, the regime where the GEMMs turn compute-bound);
// above that PB_TOK = 128, the large-item GEMMs (hidden and inter up to 2048).
int prefill_item_size(int E, int T, int K, int H, int I, bool std_experts) {
    const long tk = (long)T * K;
    // experts in groups of 32 or with bf16 parameters: 16 or 64 pairs (one- or four-tile GEMMs)
    if (!std_experts) return tk <= 8l * E ? 16 : 64;
    if (tk > 64l * E && big_steps_ok(H) && big_steps_ok(I)) return PB_TOK;
    return tk <= 8l * E ? 16 : tk <= 32l * E ? 32 : 64;
}

// Upper bound on the work items of the sort, rounded up to the 8 XCDs of the block order:
// sum over experts of ceil(count / isz) <= E + T K / isz.
int prefill_max_items(int E, int T, int K, int H, int I, bool std_experts) {
    const int isz = prefill_item_size(E, T, K, H, I, std_experts);
    return (E + (T * K + isz - 1) / isz + 7) / 8 * 8;
}

// Inputs per x-side block: 512 (split-K partials keep a few tokens' launch wide), or up to
// 2048 once there are PF_XS_BIG_T tokens (the partials' traffic would grow with T).
static int xs_inputs(int hidden, int T) { return T >= PF_XS_BIG_T ? std::min(hidden, PF_XS_K_BIG) : PF_XS_K; }
int prefill_ksplit(int hidden, int T) { return hidden / xs_inputs(hidden, T); }

hipError_t launch_moe_prefill(const MoeArgs& a, int stage, hipStream_t s) {
    const bool std_experts = a.egroup == 64 && !a.ebf;
    const int items = prefill_max_items(a.E, a.T, a.K, a.H, a.I, std_experts);
    const int isz = prefill_item_size(a.E, a.T, a.K, a.H, a.I, std_experts);
    const int tgroups = (a.T + PF_TOK - 1) / PF_TOK;
    const int ksplit = prefill_ksplit(a.H, a.T);
    const bool all = stage == QMOE_STAGE_ALL;
    // few pairs: no sort launch, each grouped GEMM block forms its work item (item_in_block)
    const int ib = (long)a.T * a.K <= PF_IB_TK && a.E <= 256 && isz <= 64 ? isz : 0;
    const bool fused_down = ib > 0 && std_experts && down_fs_fits(a);
    if (all || stage == QMOE_STAGE_ROUTE) {
        // x side: split-K blocks of PF_XS_K inputs write partial sums, k_pf_token adds them
        XsideArgs xa{};
        // token groups of 64 (four tiles), or one tile of 16 for at most 16 tokens
        const bool x1 = a.T <= 16;
        const int xgroups = x1 ? 1 : tgroups;
        xa.router = gemm_args(a.router, nullptr, a.E, a.H, a.x, a.E + 1, xgroups * ksplit);
        xa.router.T = a.T;
        xa.router.ksplit = ksplit;
        xa.router.out0 = a.logits; xa.router.ostride = a.Ep; xa.router.pstride = (long)a.T * a.Ep;
        xa.router.xp = a.sgate.p; xa.router.xs = a.sgate.s; xa.router.xb = a.sgate.b; xa.router.xout = a.gate;
        xa.shared = gemm_args(a.shg, &a.shu, a.SI, a.H, a.x, a.SI, xgroups * ksplit);
        xa.shared.T = a.T;
        xa.shared.ksplit = ksplit;
        xa.shared.out0 = a.gs; xa.shared.out1 = a.us; xa.shared.pstride = (long)a.T * a.SI;
        xa.nb_router = xa.router.nrb * xa.router.items;
        xa.nb_shared = xa.shared.nrb * xa.shared.items;
        xa.zjobs = (a.Ag ? lora_z_jobs(a.T, a.H, a.rg, a.nag) : 0) + (a.Au ? lora_z_jobs(a.T, a.H, a.ru, a.nau) : 0);
        const unsigned xgrid = (unsigned)(xa.nb_router + xa.nb_shared + (xa.zjobs + 3) / 4);
        switch (xs_inputs(a.H, a.T) / PF_KS) {
            case 4:
                if (x1) k_pf_xside<4, 1><<<xgrid, 256, 0, s>>>(xa, a);
                else k_pf_xside<4, 4><<<xgrid, 256, 0, s>>>(xa, a);
                break;
            case 8: k_pf_xside<8, 4><<<xgrid, 256, 0, s>>>(xa, a); break;
            default: k_pf_xside<16, 4><<<xgrid, 256, 0, s>>>(xa, a); break;
        }
        const size_t tsm = (size_t)a.SI * 2;   // hidden <= 4096: at most 8 splits
        // KP covers the split-K partials (<= hidden / 512) and half the LoRA z chunks
        // (hidden / 256), whatever the split
        const int kp = std::max(ksplit, a.H / 512);
        if (a.E <= 256) launch_token<4>(a, ksplit, kp, tsm, s);
        else launch_token<16>(a, ksplit, kp, tsm, s);
        const int TK = a.T * a.K;
        if (ib > 0) {
            // (few pairs: the GEMM blocks form their items themselves)
        } else if (TK <= 2048) {
            k_pf_sort<<<1, 1024, 0, s>>>(a, items, isz);
        } else {
            const int cpb = sort_chunks_per_block(TK), nseg = (TK + cpb * 1024 - 1) / (cpb * 1024);
            k_pf_count<<<nseg, 1024, 0, s>>>(a, cpb);
            k_pf_place<<<nseg, 1024, 0, s>>>(a, items, isz, cpb, nseg);
        }
    }
    if (!std_experts) {
        // routed experts in groups of 32 and/or with bf16 parameters: the staged
        // fp16-weight GEMM for gate/up and down, the shared expert's dense down apart
        if (all || stage == QMOE_STAGE_GATE_UP) {
            PfGemm p = grouped(a, a.eg, &a.eu, a.I, a.H, a.x, a.K, items, ib);
            p.hout = a.h;
            p.bf = a.ebf;
            const hipError_t e = a.egroup == 32 ? pf_gemm_staged<2, F_GROUPED | F_HOUT | F_G32>(p, isz / 16, s)
                                                : pf_gemm_staged<2, F_GROUPED | F_HOUT>(p, isz / 16, s);
            if (e != hipSuccess) return e;
        }
        if (all || stage == QMOE_STAGE_DOWN) {
            PfGemm p = grouped(a, a.ed, nullptr, a.H, a.I, a.h, 1, items, ib);
            p.hout = a.o;
            p.bf = a.ebf;
            const hipError_t e = a.egroup == 32 ? pf_gemm_staged<1, F_GROUPED | F_O16 | F_G32>(p, isz / 16, s)
                                                : pf_gemm_staged<1, F_GROUPED | F_O16>(p, isz / 16, s);
            if (e != hipSuccess) return e;
            PfGemm q = gemm_args(a.shd, nullptr, a.H, a.SI, a.hs, a.H, (a.T + 31) / 32);
            q.T = a.T;
            q.out0 = a.os;
            pf_gemm<1, 4, 2, 0>(q, s);
        }
    } else if (all || stage == QMOE_STAGE_GATE_UP) {
        PfGemm p = grouped(a, a.eg, &a.eu, a.I, a.H, a.x, a.K, items, ib);
        p.hout = a.h;
        if (isz == PB_TOK) {
            p.nrb = (a.I + PB_ROWS - 1) / PB_ROWS;
            const hipError_t e = launch_big<2, F_HOUT>(p, s);
            if (e != hipSuccess) return e;
        } else if (isz == 16) pf_gemm<2, 4, 1, F_GROUPED | F_HOUT>(p, s);
        else if (isz == 32) pf_gemm<2, 4, 2, F_GROUPED | F_HOUT>(p, s);
        else pf_gemm<2, 4, 4, F_GROUPED | F_HOUT>(p, s);
    }
    if (!std_experts) {
        // (the down GEMMs above)
    } else if ((all || stage == QMOE_STAGE_DOWN) && isz == PB_TOK) {
        // large items: the grouped down on the large-item GEMM, then the shared expert's dense
        // down over 64-token groups (resident activations at inner size 512)
        PfGemm p = grouped(a, a.ed, nullptr, a.H, a.I, a.h, 1, items, ib);
        p.hout = a.o;
        p.nrb = (a.H + PB_ROWS - 1) / PB_ROWS;
        const hipError_t e = launch_big<1, F_O16>(p, s);
        if (e != hipSuccess) return e;
        if (a.SI == 512) {
            PfGemm q = gemm_args(a.shd, nullptr, a.H, a.SI, a.hs, a.H, (a.T + 63) / 64);
            q.T = a.T;
            q.out0 = a.os;
            q.nrb = (a.H + PF_ROWS * PF_RES_RBG64 - 1) / (PF_ROWS * PF_RES_RBG64);
            k_pf_down_res<4, 4, PF_RES_RBG64><<<(unsigned)(q.nrb * q.items), 256, 0, s>>>(q, q, q.nrb * q.items);
        } else {
            PfGemm q = gemm_args(a.shd, nullptr, a.H, a.SI, a.hs, a.H, (a.T + 31) / 32);
            q.T = a.T;
            q.out0 = a.os;
            pf_gemm<1, 4, 2, 0>(q, s);
        }
    } else if ((all || stage == QMOE_STAGE_DOWN) && fused_down) {
        // few pairs: every down projection and the combine in one feature-sliced launch
        const hipError_t e = launch_down_fs(a, s);
        if (e != hipSuccess) return e;
    } else if (all || stage == QMOE_STAGE_DOWN) {
        PfGemm p = grouped(a, a.ed, nullptr, a.H, a.I, a.h, 1, items, ib);
        p.hout = a.o;   // fp16 down outputs of the (token, k) pairs
        PfGemm q = gemm_args(a.shd, nullptr, a.H, a.SI, a.hs, a.H, (a.T + 31) / 32);   // 32-token groups
        q.T = a.T;
        q.out0 = a.os;
        const int nbg = p.nrb * p.items;
        const dim3 grid((unsigned)(nbg + q.nrb * q.items));
        if (a.I == a.SI && (a.I == 512 || (a.I == 1024 && isz == 16))) {
            // resident activations: row groups of PF_RES_RBG row blocks, token groups of isz
            constexpr int RBG = PF_RES_RBG;
            const int nt = isz / 16;
            p.nrb = (a.H + PF_ROWS * RBG - 1) / (PF_ROWS * RBG);
            q = gemm_args(a.shd, nullptr, a.H, a.SI, a.hs, a.H, (a.T + isz - 1) / isz);
            q.T = a.T;
            q.out0 = a.os;
            q.nrb = p.nrb;
            const int nbd = q.nrb * q.items;   // the dense blocks, first in the grid
            const dim3 gr((unsigned)(p.nrb * p.items + nbd));
            switch ((a.I / PF_KS) * 2 + nt - 1) {
                case 8: k_pf_down_res<4, 1, RBG><<<gr, 256, 0, s>>>(p, q, nbd); break;
                case 9: k_pf_down_res<4, 2, RBG><<<gr, 256, 0, s>>>(p, q, nbd); break;
                case 11: k_pf_down_res<4, 4, RBG><<<gr, 256, 0, s>>>(p, q, nbd); break;
                default: k_pf_down_res<8, 1, RBG><<<gr, 256, 0, s>>>(p, q, nbd); break;
            }
        } else if (a.I == a.SI && (a.I == 512 || a.I == 1024 || a.I == 2048)) {
            // both GEMMs in one launch, per-step staging; grouped tiles isz / 16
            switch ((a.I / PF_KS) * 4 + isz / 16) {
                case 20: k_pf_down<4, 4><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                case 33: k_pf_down<8, 1><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                case 34: k_pf_down<8, 2><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                case 36: k_pf_down<8, 4><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                case 65: k_pf_down<16, 1><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                case 66: k_pf_down<16, 2><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
                default: k_pf_down<16, 4><<<grid, 256, 0, s>>>(p, q, q.nrb * q.items); break;
            }
        } else {
            if (isz == 16) pf_gemm<1, 4, 1, F_GROUPED | F_O16>(p, s);
            else if (isz == 32) pf_gemm<1, 4, 2, F_GROUPED | F_O16>(p, s);
            else pf_gemm<1, 4, 4, F_GROUPED | F_O16>(p, s);
            pf_gemm<1, 4, 2, 0>(q, s);
        }
    }
    if ((all || stage == QMOE_STAGE_DOWN) && !fused_down) {
        // blocks of 16 (few tokens) or 8 (many) tokens x 128 features
        if (a.T < PF_MANY_T) {
            k_pf_combine<<<(unsigned)((a.T + 15) / 16 * (a.H / 128)), 256, 0, s>>>(a);
        } else {
            const unsigned cgrid = (unsigned)((a.T + 7) / 8 * (a.H / 128));
            if (a.K <= 4) k_pf_combine_many<4><<<cgrid, 256, 0, s>>>(a);
            else k_pf_combine_many<8><<<cgrid, 256, 0, s>>>(a);
        }
    }
    return hipGetLastError();
}

}  // namespace qmoe
