// Feature-sliced down projection and combine of the MoE SwitchGLU layer, for calls with few
// routed (token, expert) pairs (T*K <= 256 with at most 256 experts, inner sizes 512).
//
// The layer is the one of moe.hip (pages: "Edge0-35B-A3B Preview model repository guide",
// model spec: routed experts' down projections and the routing-weighted sum; "Recover-LoRA
// ..." sections 1-2: the shared expert, its LoRA on down_proj and the sigmoid gate; "Edge0
// project review" highlight 3: the per-token adapter).
//
// With a few pairs per call most used experts serve one or two tokens.  The grouped down GEMM
// (one block per (expert, feature block)) then leaves blocks of unequal length and a tail, and
// its per-pair outputs make a round trip through memory to a combine launch.  Here a block
// owns FR output features n0 .. n0 + FR - 1 for every token instead:
//   * it streams those FR rows of every used expert's down matrix and of the shared expert's,
//     so the weights are still read once per call and every block has the same work (the grid
//     of hidden / FR blocks has no tail);
//   * each (token, k) pair's FR outputs o and the shared expert's os stay in LDS (fp32);
//   * the block finishes the combine of its features in place:
//       y[t][n] = fp16( sum_k w[t][k] o[t,k][n]
//                       + sigmoid(gate_t) (os[t][n] + (alpha/r) B_d[a_t][n] . z_d[t]) )
//     (+ x[t][n] when residual stacking is on), k in order.
// Weights stay exact (the 1 + q/16 codes of the GEMV core meet v_dot2, the group's affine
// terms are applied per 32-input chunk in fp32).
//
// Work inside a block, in the order that hides the most latency:
//   1. every load that needs nothing computed in the launch is issued at once: the routing,
//      the combine's inputs (gate logit, routing weights, residual, LoRA z_d), the shared
//      expert's FR rows and a first token's h_s;
//   2. the routed pairs are grouped by expert in LDS (histogram, scans); each used expert is a
//      "job";
//   3. the first jobs' rows are issued, then the shared expert's outputs are computed (its rows
//      arrived during step 2); 16-lane segments (lane l owns inputs 32 l .. 32 l + 31 of a
//      512-input row) take tokens sg, sg + 16, ...;
//   4. the segments take jobs sg, sg + 16, ..., each with two job slots: the rows and the first
//      pair's activations of job m + 1 are issued before job m is computed;
//   5. the combine, from registers loaded in step 1.
#include "gemv_core.hpp"
#include "launch.hpp"
#include "moe_common.hpp"

namespace qmoe {

namespace {

// global-memory pointers (address space 1): pointers that pass through an asm would otherwise
// become generic ones, whose flat loads are also counted with LDS accesses, so that every LDS
// wait would wait for them
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 GU4;
typedef __attribute__((address_space(1))) const uint32_t GU32;
typedef __attribute__((address_space(1))) const uint16_t GU16;
typedef __attribute__((address_space(1))) const uint8_t GU8;

__device__ __forceinline__ uint4 ldg(const GU4* p) { return __builtin_bit_cast(uint4, *p); }

constexpr int FS_ROWS = 4;    // output features per block
constexpr int FS_NTH = 256;   // threads per block
constexpr int FS_MAXP = 256;  // routed pairs per call
constexpr int FS_MAXE = 256;  // experts
constexpr int FS_MAXT = 256;  // tokens (T <= T K)
constexpr int FS_KW = 8;      // routing weights per token held in registers by the combine
constexpr int FS_IN = 512;    // inner size (routed and shared)

// One job's FR weight rows for this lane: 32 inputs (four packed words) per row and the
// row's scale and bias of the lane's group (fp16 bits, scale low).
// The FR rows' scales (and biases) are one contiguous block of FR * 8 fp16 values (rows are
// consecutive, 8 groups each): lane l of the segment loads dword l of each block (FR = 4: one
// dword per lane, one load instead of FR per array) and the lanes exchange them by shuffles.
template <int FR>
struct FsSlot {
    static_assert(FR % 4 == 0, "whole dwords of each parameter block per lane");
    static constexpr int PD = FR / 4;   // dwords of each parameter block per lane
    uint4 w[FR];
    uint32_t sd[PD], bd[PD];   // dwords l, l + 16, ... of the scale and bias blocks, as loaded
    uint4 h[4];                // the job's first pair's 32 activations (raw fp16)
};

// Exclusive prefix sum over the block's NW waves; `total` gets the sum of all.
template <int NW>
__device__ __forceinline__ int fs_block_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        base += w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
    return base + incl - v;
}

template <int FR, int NTH>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) k_fs_down(MoeArgs a) {
    constexpr int NSEG = NTH / 16;   // 16-lane segments per block
    QMOE_SGPR_USE4(a.idx, a.wts, a.h, a.hs);
    QMOE_SGPR_USE4(a.ed.p, a.ed.s, a.ed.b, a.shd.p);
    QMOE_SGPR_USE4(a.shd.s, a.shd.b, a.gate, a.zd);
    QMOE_SGPR_USE4(a.T, a.K, a.H, a.E);
    QMOE_SGPR_USE4(a.x, a.adapter, a.Bd, a.y);
    __shared__ int s_cnt[FS_MAXE];    // pairs per expert
    __shared__ int s_off[FS_MAXE];    // first index of the expert's pairs in s_plist
    __shared__ int s_plist[FS_MAXP];  // pair ids grouped by expert
    __shared__ int s_jexp[FS_MAXE], s_joff[FS_MAXE], s_jcnt[FS_MAXE];   // jobs: the used experts
    __shared__ int s_wsum[NTH / 64];
    __shared__ __align__(16) float s_o[(FS_MAXP + FS_MAXT) * FR];   // pair outputs, then shared
    const int T = a.T, K = a.K, H = a.H, E = a.E, P = T * K;
    const int tid = threadIdx.x;
    const int sg = tid >> 4, sl = tid & 15;
    const int n0 = blockIdx.x * FR;
    constexpr int RW = FS_IN / 8, RG = FS_IN / 64;   // words and groups per row

    // the matrices' base pointers as values in scalar registers (global address space)
    const GU32 *edp = (const GU32*)a.ed.p, *shp = (const GU32*)a.shd.p;
    const GU16 *eds = (const GU16*)a.ed.s, *eb = (const GU16*)a.ed.b;
    const GU16 *shs = (const GU16*)a.shd.s, *shb = (const GU16*)a.shd.b;
    const GU16 *hbase = (const GU16*)a.h, *hsbase = (const GU16*)a.hs;
    asm volatile("" : "+s"(edp), "+s"(shp), "+s"(eds), "+s"(eb));
    asm volatile("" : "+s"(shs), "+s"(shb), "+s"(hbase), "+s"(hsbase));

    // ---- phase 1: every load that needs nothing computed in this launch, issued at once.
    // Loads complete in issue order, so the routing goes first: the grouping below then waits
    // for it alone.  All are unconditional (clamped indices, stand-in addresses).
    const int e_raw = a.idx[tid < P ? tid : 0];
    // the combine's inputs for thread (token ct, feature cn), first pass (tid < T FR)
    const int ct = min(tid / FR, T - 1), cr = tid % FR, cn = n0 + cr;
    const float c_gate = a.gate[ct];
    const uint16_t c_x = a.x[(long)ct * H + cn];
    float c_w[FS_KW];
#pragma unroll
    for (int k = 0; k < FS_KW; ++k) c_w[k] = a.wts[(long)ct * K + min(k, K - 1)];
    const int c_ad_raw = *(a.adapter ? a.adapter + ct : a.idx);
    float4 c_z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c_z[i] = reinterpret_cast<const float4*>(a.zd + (long)ct * MAX_RANK)[i];
    // the shared expert's FR rows (the same for every token) and this segment's first token
    FsSlot<FR> sh;
    {
        const uint32_t wo = (uint32_t)n0 * RW + 4 * sl, go = (uint32_t)n0 * RG + 2 * sl;
#pragma unroll
        for (int r = 0; r < FR; ++r) sh.w[r] = ldg(reinterpret_cast<const GU4*>(shp + wo + r * RW));
#pragma unroll
        for (int i = 0; i < FsSlot<FR>::PD; ++i) {
            sh.sd[i] = *reinterpret_cast<const GU32*>(shs + go + 32 * i);
            sh.bd[i] = *reinterpret_cast<const GU32*>(shb + go + 32 * i);
        }
        const GU4* hp = reinterpret_cast<const GU4*>(hsbase + (long)min(sg, T - 1) * FS_IN + 32 * sl);
#pragma unroll
        for (int q = 0; q < 4; ++q) sh.h[q] = ldg(hp + q);
    }

    // ---- phase 2: the routed pairs grouped by expert (the order inside an expert is free:
    // every pair's outputs are computed alone)
    if (tid < FS_MAXE) s_cnt[tid] = 0;
    const int my_e = e_raw < 0 ? 0 : (e_raw >= E ? E - 1 : e_raw);
    __syncthreads();
    int my_slot = 0;
    if (tid < P) my_slot = atomicAdd(&s_cnt[my_e], 1);
    __syncthreads();
    const int c = tid < E ? s_cnt[tid] : 0;
    int tot = 0;
    const int pre = fs_block_scan<NTH / 64>(c | ((c > 0 ? 1 : 0) << 16), s_wsum, tot);
    const int nu = tot >> 16;   // used experts: the jobs (at least one)
    if (c > 0) {
        const int j = pre >> 16, off = pre & 0xFFFF;
        s_jexp[j] = tid;
        s_joff[j] = off;
        s_jcnt[j] = c;
        s_off[tid] = off;
    }
    __syncthreads();
    if (tid < P) s_plist[s_off[my_e] + my_slot] = tid;
    __syncthreads();

    // the combine's LoRA-B rows (they need the adapter index)
    const int c_ad = a.adapter ? (c_ad_raw < 0 ? 0 : (c_ad_raw >= a.nad ? a.nad - 1 : c_ad_raw)) : 0;
    const bool bfast = a.Bd && (a.rd & 7) == 0 && a.rd <= 16;
    uint4 c_b[2];
    {
        const uint4* brow = bfast ? reinterpret_cast<const uint4*>(a.Bd + ((long)c_ad * H + cn) * a.rd)
                                  : reinterpret_cast<const uint4*>(a.x + (long)ct * H);
#pragma unroll
        for (int i = 0; i < 2; ++i) c_b[i] = brow[bfast ? min(i, a.rd / 8 - 1) : 0];
    }

    // job j (a used expert; past the last one, the last one again, unused)
    const int niter = (nu + NSEG - 1) / NSEG;   // jobs per segment, at most
    auto jc = [&](int j) { return min(j, nu - 1); };
    auto job_cnt = [&](int j) { return j < nu ? s_jcnt[jc(j)] : 0; };
    auto load_rows = [&](FsSlot<FR>& S, int j) {
        const uint32_t row = (uint32_t)s_jexp[jc(j)] * H + n0;
        const uint32_t wo = row * RW + 4 * sl, go = row * RG + 2 * sl;
#pragma unroll
        for (int r = 0; r < FR; ++r) S.w[r] = ldg(reinterpret_cast<const GU4*>(edp + wo + r * RW));
#pragma unroll
        for (int i = 0; i < FsSlot<FR>::PD; ++i) {
            S.sd[i] = *reinterpret_cast<const GU32*>(eds + go + 32 * i);
            S.bd[i] = *reinterpret_cast<const GU32*>(eb + go + 32 * i);
        }
    };
    auto h_src = [&](int j, int i) -> const GU4* {
        const int p = s_plist[min(max(s_joff[jc(j)] + min(i, s_jcnt[jc(j)] - 1), 0), FS_MAXP - 1)];
        return reinterpret_cast<const GU4*>(hbase + (long)p * FS_IN + 32 * sl);
    };
    auto out_slot = [&](int j, int i) { return s_plist[min(s_joff[jc(j)] + i, FS_MAXP - 1)]; };

    // Codes as fp16 64 + q: a nibble moved to mantissa bits 4..7 under the exponent of 64, one
    // v_and_or_b32 per pair of codes on the word shifted by 4, 0, -4 and -8 bits (nibbles j and
    // j + 4 land in the low and high half together, the pair order of pair_perm8_w).  Products
    // with fp16 activations are exact in fp32, and sum (64 + q) x = 64 sum x + sum q x keeps the
    // constant part within a few bits of the code part.  Mask and exponent are held in VGPRs:
    // a gfx9 VOP3 instruction takes no literal.
    uint32_t nmask = 0x00F000F0u, nexp = 0x54005400u;
    asm volatile("" : "+v"(nmask), "+v"(nexp));
    auto dot_codes = [&](uint32_t w, const uint4& xp, float acc) {
        acc = __builtin_amdgcn_fdot2(as_h2(((w << 4) & nmask) | nexp), as_h2(xp.x), acc, false);
        acc = __builtin_amdgcn_fdot2(as_h2((w & nmask) | nexp), as_h2(xp.y), acc, false);
        acc = __builtin_amdgcn_fdot2(as_h2(((w >> 4) & nmask) | nexp), as_h2(xp.z), acc, false);
        acc = __builtin_amdgcn_fdot2(as_h2(((w >> 8) & nmask) | nexp), as_h2(xp.w), acc, false);
        return acc;
    };
    // the FR row outputs of one pair (activations hv, raw): segment totals in every lane
    auto pair_dot = [&](const FsSlot<FR>& S, const uint4 (&hv)[4], float (&v)[FR]) {
        const f16x2 one = {(f16)1.0f, (f16)1.0f};
        float xs = 0.0f;
        uint4 hp[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xs = __builtin_amdgcn_fdot2(as_h2(hv[q].x), one, xs, false);
            xs = __builtin_amdgcn_fdot2(as_h2(hv[q].y), one, xs, false);
            xs = __builtin_amdgcn_fdot2(as_h2(hv[q].z), one, xs, false);
            xs = __builtin_amdgcn_fdot2(as_h2(hv[q].w), one, xs, false);
            hp[q] = pair_perm8_w(hv[q]);
        }
#pragma unroll
        for (int r = 0; r < FR; ++r) {
            const uint32_t wd[4] = {S.w[r].x, S.w[r].y, S.w[r].z, S.w[r].w};
            float d = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) d = dot_codes(wd[q], hp[q], d);
            // row r, group sl / 2: dword 4 r + sl / 4 of the blocks (lane 4 (r % 4) + sl / 4,
            // its register r / 4), half (sl / 2) & 1
            const int src = 4 * (r & 3) + (sl >> 2);
            const uint32_t sw = (uint32_t)__shfl((int)S.sd[r >> 2], src, 16);
            const uint32_t bw = (uint32_t)__shfl((int)S.bd[r >> 2], src, 16);
            const int sh16 = (sl & 2) << 3;
            const float s = h2f((uint16_t)(sw >> sh16)), b = h2f((uint16_t)(bw >> sh16));
            // s sum q x + b sum x = s d + (b - 64 s) sum x
            v[r] = seg_sum<16>(fmaf(s, d, fmaf(-64.0f, s, b) * xs));
        }
    };
    auto store = [&](int slot, const float (&v)[FR]) {
        if (sl == 0) {
            if constexpr (FR == 4) *reinterpret_cast<float4*>(&s_o[slot * FR]) = float4{v[0], v[1], v[2], v[3]};
            else {
#pragma unroll
                for (int r = 0; r < FR; ++r) s_o[slot * FR + r] = v[r];
            }
        }
    };

    // ---- phase 3: the first routed job's rows and activations in flight, then the shared
    // expert's outputs (its rows arrived during the grouping).  Each segment keeps two job
    // slots: while job m is computed, job m + 1's loads are in flight.  A third slot (two jobs
    // in flight) ran the 16-token stack 2 % slower: with more requests outstanding from every
    // block, the rows arrived later.
    FsSlot<FR> S0, S1;
    load_rows(S0, sg);
    {
        const GU4* hp = h_src(sg, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) S0.h[q] = ldg(hp + q);
    }
    __builtin_amdgcn_sched_barrier(0);
    {
        float v[FR];
        pair_dot(sh, sh.h, v);
        if (sg < T) store(P + sg, v);
        for (int t = sg + NSEG; t < T; t += NSEG) {   // tokens past the first NSEG (loaded here)
            const GU4* hp = reinterpret_cast<const GU4*>(hsbase + (long)t * FS_IN + 32 * sl);
            uint4 hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = ldg(hp + q);
            pair_dot(sh, hv, v);
            store(P + t, v);
        }
    }

    // ---- phase 4: the routed jobs.  One step: issue the first activations and the rows of
    // job m + 1 (into `nxt`), then compute job m from `cur`.
    auto step = [&](FsSlot<FR>& cur, FsSlot<FR>& nxt, int m) {
        const int j = sg + NSEG * m;
        {
            const GU4* hp = h_src(j + NSEG, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) nxt.h[q] = ldg(hp + q);
        }
        load_rows(nxt, j + NSEG);
        __builtin_amdgcn_sched_barrier(0);   // the loads above are issued before any wait below
        const int cnt = job_cnt(j);
        float v[FR];
        pair_dot(cur, cur.h, v);
        if (cnt > 0) store(out_slot(j, 0), v);
        for (int i = 1; i < cnt; ++i) {   // further pairs of the job (rare): loaded here
            const GU4* hp = h_src(j, i);
            uint4 hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = ldg(hp + q);
            pair_dot(cur, hv, v);
            store(out_slot(j, i), v);
        }
    };
    int m = 0;
    for (; m + 2 <= niter; m += 2) {
        step(S0, S1, m);
        step(S1, S0, m + 1);
    }
    if (m < niter) step(S0, S1, m);   // (niter is the same in every lane of the block)
    __syncthreads();

    // ---- phase 5: combine, thread (t, r) for feature n0 + r of token t; the first pass from
    // the registers loaded in phase 1
    auto finish = [&](int t, int r, float gate, uint16_t xr, float lora, const float* w8) {
        const int n = n0 + r;
        float ov = s_o[(P + t) * FR + r];
        if (a.Bd) ov = fmaf(a.lsd, lora, ov);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < FS_KW; ++k)
            if (k < K) acc = fmaf(w8[k], s_o[(t * K + k) * FR + r], acc);
        for (int k = FS_KW; k < K; ++k) acc = fmaf(a.wts[(long)t * K + k], s_o[(t * K + k) * FR + r], acc);
        uint16_t out = f2h(fmaf(sigmoid(gate), ov, acc));
        if (a.add_residual) out = f2h(h2f(xr) + h2f(out));
        a.y[(long)t * H + n] = out;
    };
    if (tid < T * FR) {
        float lora = 0.0f;
        if (bfast) {
            float zf[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zf[4 * i] = c_z[i].x; zf[4 * i + 1] = c_z[i].y; zf[4 * i + 2] = c_z[i].z; zf[4 * i + 3] = c_z[i].w;
            }
            lora = bdot16(c_b, zf, a.rd);
        } else if (a.Bd) {
            lora = lora_b_dot(a.Bd, c_ad, H, cn, a.rd, a.zd + (long)ct * MAX_RANK);
        }
        finish(ct, cr, c_gate, c_x, lora, c_w);
    }
    for (int u = tid + NTH; u < T * FR; u += NTH) {   // tokens past the first NTH / FR
        const int t = u / FR, r = u % FR, n = n0 + r;
        float w8[FS_KW];
#pragma unroll
        for (int k = 0; k < FS_KW; ++k) w8[k] = a.wts[(long)t * K + min(k, K - 1)];
        const float lora = a.Bd ? lora_b_dot(a.Bd, adapter_of(a.adapter, t, a.nad), H, n, a.rd,
                                             a.zd + (long)t * MAX_RANK) : 0.0f;
        finish(t, r, a.gate[t], a.x[(long)t * H + n], lora, w8);
    }
}

}  // namespace

bool down_fs_fits(const MoeArgs& a) {
    return (long)a.T * a.K <= FS_MAXP && a.E <= FS_MAXE && a.I == FS_IN && a.SI == FS_IN &&
           a.H % FS_ROWS == 0 && a.egroup == 64 && !a.ebf;
}

hipError_t launch_down_fs(const MoeArgs& a, hipStream_t s) {
    k_fs_down<FS_ROWS, FS_NTH><<<(unsigned)(a.H / FS_ROWS), FS_NTH, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace qmoe
