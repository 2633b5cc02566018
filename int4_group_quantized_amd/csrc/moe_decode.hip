// Decode path of the MoE SwitchGLU layer (a few tokens per call): three launches, no sort,
// no atomics, top-K taken once per token in the gate/up launch and published to the down
// launch through the workspace.
//
// The layer is the one described in moe.hip (pages: "Edge0-35B-A3B Preview model repository
// guide" model spec; "Recover-LoRA ..." sections 1-2; "Edge0 project review" highlights 2-3).
// At decode sizes every launch is bound by memory latency, not bandwidth: the design goal
// is the shortest chain of dependent memory round trips per kernel.
//
//   D1 x-side  : router logits (8-bit), shared-gate logit (8-bit), the shared expert's raw
//                gate/up projections (int4), LoRA z = A x.  Each wave issues its weight
//                loads before staging x, so the two memory round trips overlap.
//   D2 gate/up : one block per (row block, routed pair (t, k) or the shared expert).  Every
//                wave reads token t's logits and takes the selection up to round k (the
//                same deterministic selection in every block), so it issues the gate and up
//                rows of expert idx[t][k] before x is staged and the block synchronises;
//                then h = silu(g) * u is stored (fp16).  Shared blocks (one wave per 64
//                rows of a token) add the LoRA up-projections, store h_s and, for LoRA ranks
//                up to 16, their rows' share of the down LoRA's z_down = A_down h_s.
//   D3 down    : one block per (row block, token).  It reads the token's published routing
//                and sums the z_down shares (or takes A_down h_s itself), stages the token's
//                K expert activations h and h_s, streams the K + 1 down matrices' rows, and
//                combines y = sum_k w_k o_k + sigmoid(gate) (o_s + LoRA) (+ residual)
//                in-block.
#include <algorithm>

#include "gemv_core.hpp"
#include "launch.hpp"
#include "moe_common.hpp"

namespace qmoe {

namespace {

constexpr int MT = GEMV_MT;

// ------------------------------------------------------------------------------ D1 x-side

// One x-side block's rows of a BITS-bit matrix: each lane segment owns row n of w (weights
// loaded before x is staged, so the two memory round trips overlap), then the dot over the
// staged tokens.  One body per width: loaded registers never meet at a branch merge, where the
// compiler would copy them and so wait for every load in flight.
template <int BITS>
__device__ __forceinline__ void xside_rows(const MoeArgs& a, const QW& w, int n, bool ok, float* out,
                                           int ostride, f16x2* xs, float* xsum, int xs_halves2) {
    const int H = a.H;
    const int lane = threadIdx.x & 63;
    const int lpr = lanes_per_row(H), sl = lane % lpr;
    RowRegs<BITS, 2> rw;
    rw.load(w.p, w.s, w.b, H, n, lpr, sl, ok);
    const int mt_max = min(MT, xs_halves2 / (H / 2));
    for (int t0 = 0; t0 < a.T; t0 += mt_max) {
        const int mt = min(mt_max, a.T - t0);
        if (t0 > 0) __syncthreads();
        const uint4* xb = reinterpret_cast<const uint4*>(a.x + (long)t0 * H);
        auto rowp = [=](int i) { return xb + (long)i * (H / 8); };
        stage_rows<BITS, 8>(rowp, mt, H, xs, xsum);
        __syncthreads();
        rw.hold();   // the weights are first used here, after x is staged
        float acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
        rw.dot(H, lpr, sl, xs, xsum, mt, acc);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < mt) {
                const float v = segment_sum(acc[t], lpr);
                if (sl == 0 && ok) out[(long)(t0 + t) * ostride + n] = v;
            }
        }
    }
}

// Every argument field of the x side in one batch of scalar loads (one round trip).
#define QMOE_XSIDE_ARGS()                                                                        \
    asm volatile("" ::"s"(a.router.p), "s"(a.router.s), "s"(a.router.b), "s"(a.x), "s"(a.shg.p), \
                 "s"(a.shg.s), "s"(a.shg.b), "s"(a.logits), "s"(a.shu.p), "s"(a.shu.s),         \
                 "s"(a.shu.b), "s"(a.gs), "s"(a.us), "s"(a.T), "s"(a.H), "s"(a.E), "s"(a.SI),   \
                 "s"(a.Ep), "s"(a.Ag), "s"(a.Au), "s"(a.rg), "s"(a.ru), "s"(a.gate),            \
                 "s"(a.sgate.p), "s"(a.sgate.s), "s"(a.sgate.b), "s"(a.zg), "s"(a.zu))

// Block b of the x side: router rows, the shared-gate row, the shared expert's raw gate/up
// rows, or LoRA z jobs.
__device__ __forceinline__ void xside_block(const MoeArgs& a, int b, f16x2* xs, float* xsum) {
    const int H = a.H;
    const int zjobs = (a.Ag ? a.T * a.rg : 0) + (a.Au ? a.T * a.ru : 0);
    const XsideGrid g = xside_grid(a.T, H, a.E, a.SI, zjobs);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = lanes_per_row(H), rpw = 64 / lpr, seg = lane / lpr;

    if (b >= g.nb_router + g.nb_gate + g.nb_shared) {
        xside_lora_z(a, (b - g.nb_router - g.nb_gate - g.nb_shared) * 4 + wave, zjobs);
        return;
    }
    // the row this lane segment owns (block-uniform role); the matrix chosen by value (a
    // pointer into the argument struct would read its fields through dependent vector loads)
    if (b < g.nb_router + g.nb_gate) {
        const bool router = b < g.nb_router;
        const int r = router ? (b * 4 + wave) * rpw + seg : wave * rpw + seg;
        const bool ok = r < (router ? a.E : 1);
        xside_rows<8>(a, router ? a.router : a.sgate, ok ? r : 0, ok, router ? a.logits : a.gate,
                      router ? a.Ep : 1, xs, xsum, 8192);
    } else {
        const int r = ((b - g.nb_router - g.nb_gate) * 4 + wave) * rpw + seg;
        const bool ok = r < 2 * a.SI;
        const int rr = ok ? r : 0;
        const bool up = rr >= a.SI;
        xside_rows<4>(a, up ? a.shu : a.shg, up ? rr - a.SI : rr, ok, up ? a.us : a.gs, a.SI, xs, xsum, 8192);
    }
}

__global__ void __launch_bounds__(256) k_dec_xside(MoeArgs a) {
    __shared__ __align__(16) f16x2 xs[8192];   // 32 KB: 8192 / (hidden / 2) tokens per pass
    __shared__ float xsum[MT * 128];
    QMOE_XSIDE_ARGS();
    xside_block(a, blockIdx.x, xs, xsum);
}

int xside_blocks(const MoeArgs& a) {
    const int zjobs = (a.Ag ? a.T * a.rg : 0) + (a.Au ? a.T * a.ru : 0);
    const XsideGrid g = xside_grid(a.T, a.H, a.E, a.SI, zjobs);
    return g.nb_router + g.nb_gate + g.nb_shared + g.nb_z;
}

// ------------------------------------------------------------------------------ D2 gate/up

constexpr int GU_RPW = 1;  // gate/up row pairs per wave

// 64 rows n = 64 rb + lane of token t's shared expert after the x side, one wave:
//   h_s[n] = fp16( silu(gs + (alpha/r) B_g z_g) * (us + (alpha/r) B_u z_u) )   (to memory)
// and, for LoRA ranks up to DEC_ZP_RANK, these rows' share of the down LoRA's z_d:
//   zp[t][rb][r] = sum over the 64 rows of A_d[a_t][r][n] h_s[n]   (fixed order)
// which the down launch adds over rb in order, instead of every down block taking A_d . h_s
// from the whole of A_d.  Every load is issued before any arithmetic (the A_d column loads
// are unconditional, from a stand-in row without them).  `lds`: 64 x 16 floats.
__device__ __forceinline__ void dec_shared_rows(const MoeArgs& a, int t, int rb, float* lds) {
    const int lane = threadIdx.x & 63, SI = a.SI, n = rb * 64 + lane;
    const int ad = adapter_of(a.adapter, t, a.nad);
    const bool zpart = a.Ad && a.rd <= DEC_ZP_RANK;
    float gv = a.gs[(long)t * SI + n];
    float uv = a.us[(long)t * SI + n];
    uint16_t ac[DEC_ZP_RANK];
#pragma unroll
    for (int r = 0; r < DEC_ZP_RANK; ++r)
        ac[r] = zpart ? a.Ad[((long)ad * a.rd + min(r, a.rd - 1)) * SI + n] : a.x[(long)t * a.H + lane];
    // the B rows of both projections (ranks up to 16 in registers, loaded unconditionally from
    // a stand-in row without them: a load under a branch is waited for at the branch's end,
    // which would put the second projection's rows a round trip behind the first's)
    const int ag = adapter_of(a.adapter, t, a.nag), au = adapter_of(a.adapter, t, a.nau);
    const bool gfast = a.Bg && (a.rg & 7) == 0 && a.rg <= 16, ufast = a.Bu && (a.ru & 7) == 0 && a.ru <= 16;
    const uint4* xst = reinterpret_cast<const uint4*>(a.x + (long)t * a.H);
    const uint4* bgp = gfast ? reinterpret_cast<const uint4*>(a.Bg + ((long)ag * SI + n) * a.rg) : xst;
    const uint4* bup = ufast ? reinterpret_cast<const uint4*>(a.Bu + ((long)au * SI + n) * a.ru) : xst;
    uint4 bg[2], bu[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        bg[i] = bgp[gfast ? min(i, a.rg / 8 - 1) : 0];
        bu[i] = bup[ufast ? min(i, a.ru / 8 - 1) : 0];
    }
    const float* zg = a.zg + t * MAX_RANK;
    const float* zu = a.zu + t * MAX_RANK;
    if (gfast) gv = fmaf(a.lsg, bdot16(bg, zg, a.rg), gv);
    else if (a.Bg) gv = fmaf(a.lsg, lora_b_dot(a.Bg, ag, SI, n, a.rg, zg), gv);
    if (ufast) uv = fmaf(a.lsu, bdot16(bu, zu, a.ru), uv);
    else if (a.Bu) uv = fmaf(a.lsu, lora_b_dot(a.Bu, au, SI, n, a.ru, zu), uv);
    const uint16_t hv = f2h(silu(gv) * uv);
    a.hs[(long)t * SI + n] = hv;
    if (zpart) {
        const float hf = h2f(hv);
        // the 16 sums over the wave's lanes through LDS (one wave: LDS accesses complete in
        // order, so only the compiler needs a fence): lane l adds rank l % 16 over lanes
        // 16 (l / 16) .. + 15, then the four partial sums meet in a fixed order
        float4* pl = reinterpret_cast<float4*>(lds + lane * DEC_ZP_RANK);
#pragma unroll
        for (int i = 0; i < DEC_ZP_RANK / 4; ++i)
            pl[i] = make_float4(h2f(ac[4 * i]) * hf, h2f(ac[4 * i + 1]) * hf, h2f(ac[4 * i + 2]) * hf,
                                h2f(ac[4 * i + 3]) * hf);
        asm volatile("" ::: "memory");
        const int r = lane & 15, g = lane >> 4;
        float zs = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) zs += lds[(16 * g + i) * DEC_ZP_RANK + r];
        zs += __shfl_xor(zs, 16, 64);
        zs += __shfl_xor(zs, 32, 64);
        if (lane < DEC_ZP_RANK && lane < a.rd) a.zd[((long)t * DEC_ZP_BLOCKS + rb) * DEC_ZP_RANK + lane] = zs;
    }
}

template <int PER>
__global__ void __launch_bounds__(256) k_dec_gate_up(MoeArgs a) {
    __shared__ __align__(16) f16x2 xs[2048];   // one token, hidden <= 4096
    __shared__ float xsum[128];
    QMOE_SGPR_USE4(a.logits, a.x, a.eg.p, a.eg.s);
    QMOE_SGPR_USE4(a.eg.b, a.eu.p, a.eu.s, a.eu.b);
    QMOE_SGPR_USE4(a.h, a.idx, a.wts, a.rbias);
    QMOE_SGPR_USE4(a.T, a.H, a.I, a.K);
    QMOE_SGPR_USE2(a.E, a.Ep);
    const int H = a.H, I = a.I, K = a.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.y;
    const int TK = a.T * K;
    const int lpr = lanes_per_row(H), rpw = 64 / lpr, seg = lane / lpr, sl = lane % lpr;
    const int rows_per_block = 4 * rpw * GU_RPW;

    if (pair == TK) {  // shared expert: wave 0 of block b finishes rows 64 (b % nbs) .. of token b / nbs
        const int nbs = a.SI / 64;
        if (blockIdx.x < (unsigned)(a.T * nbs) && wave == 0)
            dec_shared_rows(a, blockIdx.x / nbs, blockIdx.x % nbs, reinterpret_cast<float*>(xs));
        return;
    }
    if (blockIdx.x * rows_per_block >= I) return;
    const int t = pair / K, k = pair % K;
    // phase 1: wave 0's logit loads and the block's x[t] loads in flight together
    __shared__ int sel[MAX_K];
    __shared__ float selw[MAX_K];
    TopkKeys<PER> keys;
    keys.load(a.logits + (long)t * a.Ep, a.rbias, a.E);
    const uint4* xt = reinterpret_cast<const uint4*>(a.x + (long)t * H);
    StageRegs<4, 2> st;
    st.load([=](int) { return xt; }, 1, H);
    __builtin_amdgcn_sched_barrier(0);
    // phase 2: every wave takes the selection up to its pair's round k itself and issues its
    // weight loads at once, before x goes to LDS and the barrier; the first row block's wave 0
    // also takes the whole top-K, to publish it
    if (blockIdx.x == 0 && wave == 0) keys.select(a.E, K, sel, selw);
    const int e = keys.pick(a.E, k);
    RowRegs<4, 2> rg[GU_RPW], ru[GU_RPW];
    int n[GU_RPW];
#pragma unroll
    for (int j = 0; j < GU_RPW; ++j) {
        n[j] = blockIdx.x * rows_per_block + (j * 4 + wave) * rpw + seg;
        const bool ok = n[j] < I;
        const long row = (long)e * I + (ok ? n[j] : 0);
        rg[j].load(a.eg.p, a.eg.s, a.eg.b, H, row, lpr, sl, ok);
        ru[j].load(a.eu.p, a.eu.s, a.eu.b, H, row, lpr, sl, ok);
    }
    st.commit(1, H, xs, xsum);
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // publish the decision for the down stage and the caller
        a.idx[pair] = e;
        a.wts[pair] = selw[k];
        if (a.idx_out) a.idx_out[pair] = e;
        if (a.w_out) a.w_out[pair] = selw[k];
    }
#pragma unroll
    for (int j = 0; j < GU_RPW; ++j) {
        float ag[MT], au[MT];
        ag[0] = au[0] = 0.0f;
        rg[j].dot(H, lpr, sl, xs, xsum, 1, ag);
        ru[j].dot(H, lpr, sl, xs, xsum, 1, au);
        const float gv = segment_sum(ag[0], lpr), uv = segment_sum(au[0], lpr);
        if (sl == 0 && n[j] < I) a.h[(long)pair * I + n[j]] = f2h(silu(gv) * uv);
    }
}

// One block of the shared expert for a given routing: rows bx * rows_per_block .. of the
// shared gate and up for token t, their LoRA deltas and h_s = silu(g) * u, stored for the
// down launch (which then reads h_s as in the top-K path).  The LoRA z's of the token are
// taken in every such block (the x side, which runs in the same launch, cannot hand them
// over): wave w the ranks 8 w .. 8 w + 7 of the gate's then the up's, each as the x side's
// LoRA z jobs take it (a lane's inputs lane * 8 + 512 i, then the wave sum).
__device__ void rt_shared_block(const MoeArgs& a, int t, int bx, f16x2* xs, float* xsum, float (*zs)[MAX_RANK]) {
    const int H = a.H, SI = a.SI;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = lanes_per_row(H), rpw = 64 / lpr, seg = lane / lpr, sl = lane % lpr;
    const int n = bx * (4 * rpw) + wave * rpw + seg;
    const bool ok = n < SI;
    const int nn = ok ? n : 0;
    // phase 1: the adapter index (first: the LoRA rows wait for it), x, the rows of the shared
    // gate and up, and this lane's x chunks for the z's (loaded unconditionally: a stand-in
    // address without adapters)
    const int araw_l = *(a.adapter ? a.adapter + t : reinterpret_cast<const int32_t*>(a.x));
    __builtin_amdgcn_sched_barrier(0);
    const uint4* xt = reinterpret_cast<const uint4*>(a.x + (long)t * H);
    StageRegs<4, 2> st;
    st.load([=](int) { return xt; }, 1, H);
    RowRegs<4, 2> rg, ru;
    rg.load(a.shg.p, a.shg.s, a.shg.b, H, nn, lpr, sl, ok);
    ru.load(a.shu.p, a.shu.s, a.shu.b, H, nn, lpr, sl, ok);
    constexpr int ZI = 4;   // 512-input chunks per pass: hidden 2048 in one pass
    uint4 xz[ZI];
#pragma unroll
    for (int i = 0; i < ZI; ++i) xz[i] = xt[min(lane * 8 + 512 * i, H - 8) / 8];
    __builtin_amdgcn_sched_barrier(0);
    int araw = araw_l;
    asm volatile("" : "+v"(araw));
    auto clamp_ad = [&](int na) { const int v = a.adapter ? araw : 0; return v < 0 ? 0 : (v >= na ? na - 1 : v); };
    const int adg = clamp_ad(a.nag), adu = clamp_ad(a.nau);
    const int rgk = a.Ag ? a.rg : 0, ruk = a.Au ? a.ru : 0, nz = rgk + ruk;
    // phase 2: the LoRA rows (they need the adapter index): the B rows of this lane's output
    // (ranks up to 16, a multiple of 8) and the A rows of this wave's ranks
    const bool bgf = a.Bg && (a.rg & 7) == 0 && a.rg <= 16;
    const bool buf = a.Bu && (a.ru & 7) == 0 && a.ru <= 16;
    uint4 bgv[2], buv[2];
    {
        const uint16_t* gb = bgf ? a.Bg + ((long)adg * SI + nn) * a.rg : a.x;
        const uint16_t* ub = buf ? a.Bu + ((long)adu * SI + nn) * a.ru : a.x;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            bgv[i] = *reinterpret_cast<const uint4*>(gb + (bgf ? min(8 * i, a.rg - 8) : 0));
            buv[i] = *reinterpret_cast<const uint4*>(ub + (buf ? min(8 * i, a.ru - 8) : 0));
        }
    }
    st.commit(1, H, xs, xsum);
    __syncthreads();
    // the rows' dot products first: the A rows (one round trip later than the weights) arrive
    // meanwhile
    float ag[MT], au[MT];
    ag[0] = au[0] = 0.0f;
    rg.dot(H, lpr, sl, xs, xsum, 1, ag);
    ru.dot(H, lpr, sl, xs, xsum, 1, au);
    float gv = segment_sum(ag[0], lpr), uv = segment_sum(au[0], lpr);
    for (int j0 = wave * 8; j0 < nz; j0 += 32) {   // passes of 32 ranks (one for ranks <= 16)
        uint4 av[8][ZI];
        auto arow = [&](int j) {   // rank row j of the concatenated gate and up ranks (clamped)
            const int jj = min(j, nz - 1);
            return jj < rgk ? a.Ag + ((long)adg * a.rg + jj) * H : a.Au + ((long)adu * a.ru + (jj - rgk)) * H;
        };
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int i = 0; i < ZI; ++i) av[r][i] = *reinterpret_cast<const uint4*>(arow(j0 + r) + min(lane * 8 + 512 * i, H - 8));
        float acc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            acc[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < ZI; ++i) {
                if (lane * 8 + 512 * i < H) {
                    const f16x2* ah = reinterpret_cast<const f16x2*>(&av[r][i]);
                    const f16x2* xh = reinterpret_cast<const f16x2*>(&xz[i]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[r] = __builtin_amdgcn_fdot2(ah[q], xh[q], acc[r], false);
                }
            }
        }
        for (int c0 = ZI * 512; c0 < H; c0 += ZI * 512) {   // hidden above 2048: further chunks
#pragma unroll
            for (int r = 0; r < 8; ++r) {
#pragma unroll
                for (int i = 0; i < ZI; ++i) {
                    const int k = c0 + lane * 8 + 512 * i;
                    if (k < H) {
                        const uint4 av2 = *reinterpret_cast<const uint4*>(arow(j0 + r) + k);
                        const uint4 xv2 = xt[k / 8];
                        const f16x2* ah = reinterpret_cast<const f16x2*>(&av2);
                        const f16x2* xh = reinterpret_cast<const f16x2*>(&xv2);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[r] = __builtin_amdgcn_fdot2(ah[q], xh[q], acc[r], false);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float v = seg_sum<64>(acc[r]);
            const int j = j0 + r;
            if (lane == 0 && j < nz) zs[j < rgk ? 0 : 1][j < rgk ? j : j - rgk] = v;
        }
    }
    __syncthreads();
    if (sl == 0 && ok) {
        if (a.Bg) gv = fmaf(a.lsg, bgf ? bdot16(bgv, zs[0], a.rg) : lora_b_dot(a.Bg, adg, SI, n, a.rg, zs[0]), gv);
        if (a.Bu) uv = fmaf(a.lsu, buf ? bdot16(buv, zs[1], a.ru) : lora_b_dot(a.Bu, adu, SI, n, a.ru, zs[1]), uv);
        a.hs[(long)t * SI + n] = f2h(silu(gv) * uv);
    }
}

// The x side and the routed gate/up of a GIVEN routing in one launch (the caller's selection,
// e.g. the prerouter head's prediction, which is then the route itself: "Edge0 project
// review", highlight 1).  Blocks below nx are x-side blocks; every other block is one
// (row block, pair) of the routed gate/up: it reads its expert from the given routing at
// entry and issues that expert's gate and up rows at once, so no block waits for another
// and the router's logits are needed only by the down launch (the routing weights).  The
// shared expert's h_s, which needs the x side's LoRA z's, is finished by the down launch.
__global__ void __launch_bounds__(256) k_dec_rt_gate_up(MoeArgs a, int nx, int ns) {
    __shared__ __align__(16) f16x2 xs[8192];
    __shared__ float xsum[MT * 128];
    if ((int)blockIdx.x < nx) {   // the router and shared-gate rows of the x side
        QMOE_XSIDE_ARGS();
        xside_block(a, blockIdx.x, xs, xsum);
        return;
    }
    if ((int)blockIdx.x < nx + ns) {   // the shared expert, row block b % nrb of token b / nrb
        __shared__ float zs[2][MAX_RANK];
        const int b = blockIdx.x - nx, nrbs = ns / a.T;
        rt_shared_block(a, b / nrbs, b % nrbs, xs, xsum, zs);
        return;
    }
    QMOE_SGPR_USE4(a.route, a.x, a.eg.p, a.eg.s);
    QMOE_SGPR_USE4(a.eg.b, a.eu.p, a.eu.s, a.eu.b);
    QMOE_SGPR_USE4(a.h, a.H, a.I, a.E);
    const int H = a.H, I = a.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = lanes_per_row(H), rpw = 64 / lpr, seg = lane / lpr, sl = lane % lpr;
    const int rows_per_block = 4 * rpw * GU_RPW;
    const int nrb = (I + rows_per_block - 1) / rows_per_block;
    const int b = blockIdx.x - nx - ns;
    const int pair = b / nrb, bx = b % nrb;
    const int t = pair / a.K;
    const int e = clamp_expert(a.route[pair], a.E);
    const uint4* xt = reinterpret_cast<const uint4*>(a.x + (long)t * H);
    StageRegs<4, 2> st;
    st.load([=](int) { return xt; }, 1, H);
    RowRegs<4, 2> rg[GU_RPW], ru[GU_RPW];
    int n[GU_RPW];
#pragma unroll
    for (int j = 0; j < GU_RPW; ++j) {
        n[j] = bx * rows_per_block + (j * 4 + wave) * rpw + seg;
        const bool ok = n[j] < I;
        const long row = (long)e * I + (ok ? n[j] : 0);
        rg[j].load(a.eg.p, a.eg.s, a.eg.b, H, row, lpr, sl, ok);
        ru[j].load(a.eu.p, a.eu.s, a.eu.b, H, row, lpr, sl, ok);
    }
    st.commit(1, H, xs, xsum);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GU_RPW; ++j) {
        float ag[MT], au[MT];
        ag[0] = au[0] = 0.0f;
        rg[j].dot(H, lpr, sl, xs, xsum, 1, ag);
        ru[j].dot(H, lpr, sl, xs, xsum, 1, au);
        const float gv = segment_sum(ag[0], lpr), uv = segment_sum(au[0], lpr);
        if (sl == 0 && n[j] < I) a.h[(long)pair * I + n[j]] = f2h(silu(gv) * uv);
    }
}

// ------------------------------------------------------------------------------ D3 down

constexpr int DN_ROWS = 8;     // output rows per block
constexpr int DN_ITEMS = 4;    // routed (expert, row) items per lane segment per pass (at most)
constexpr int DN_STAGE = 3;    // 16-byte staging loads per thread: (K + 1) * inter / 8 <= 768

// ROUTED: the routing is the caller's (a.route): the experts come from it and the weights are
// the softmax of the router logits over it (h_s comes from the shared blocks of
// k_dec_rt_gate_up, as from the gate/up launch otherwise).
// ZP: the down LoRA's z_d is the sum of the gate/up launch's per-64-row shares (top-K path,
// rank <= DEC_ZP_RANK); otherwise every block takes A_d . h_s itself.
// NI: routed items per lane segment per pass (2 when K DN_ROWS fits twice the segments).
template <bool ROUTED, bool ZP, int NI>
__global__ void __launch_bounds__(256) k_dec_down(MoeArgs a) {
    // staged activations: the token's K routed h rows and h_s (as matrix K), pair layout
    __shared__ __align__(16) f16x2 hs_l[(MAX_DEC_K + 1) * 1024];   // inter <= 2048
    if constexpr (ROUTED) {
        QMOE_SGPR_USE4(a.route, a.logits, a.h, a.hs);
        QMOE_SGPR_USE2(a.E, a.Ep);
        QMOE_SGPR_USE2(a.rbias, a.w_out);
    } else {
        QMOE_SGPR_USE4(a.idx, a.wts, a.h, a.hs);
    }
    QMOE_SGPR_USE4(a.ed.p, a.ed.s, a.ed.b, a.shd.p);
    QMOE_SGPR_USE4(a.shd.s, a.shd.b, a.Ad, a.Bd);
    QMOE_SGPR_USE4(a.gate, a.x, a.y, a.adapter);
    QMOE_SGPR_USE4(a.H, a.K, a.I, a.rd);
    __shared__ float hsum[(MAX_DEC_K + 1) * 64];
    __shared__ float o_l[(MAX_DEC_K + 1) * DN_ROWS];
    __shared__ float zd[MAX_RANK];
    const int H = a.H, K = a.K, Kd = a.I;   // the decode path requires inter == shared_inter
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.y;
    const int n0 = blockIdx.x * DN_ROWS;
    const int lpr = lanes_per_row(Kd), rpw = 64 / lpr, seg = lane / lpr, sl = lane % lpr;
    const int n_staged = K + 1;   // rows staged from memory: the K routed h rows and h_s
    const bool one_pass = n_staged * (Kd / 8) <= 256 * DN_STAGE;
    // expert of routing entry m (< K) of token t
    auto expert_of = [&](int m) {
        if constexpr (ROUTED) return clamp_expert(a.route[(long)t * K + m], a.E);
        else return a.idx[(long)t * K + m];
    };

    // phase 1: every load that needs no other load's value, issued before any wait: the
    // routing (published by the gate/up stage, or given), the adapter index, the shared
    // expert's down rows, the K + 1 activation rows, the combine's own inputs.  Each lane
    // loads the expert of its own first-pass items (per-lane loads: a per-lane pick from a
    // uniform array would become an indexed scratch access whose wait drains every load in
    // flight).  Loads complete in issue order, so the routing and the adapter index go first:
    // the waits for them below then do not wait for the rest.
    const int n_items = K * DN_ROWS;      // routed (expert, row) items
    const int slots = 4 * rpw;            // lane segments in the block
    const int slot = wave * rpw + seg;
    int eit[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int m = min(i * slots + slot, n_items - 1) / DN_ROWS;
        eit[i] = expert_of(min(m, K - 1));
    }
    // (ROUTED) lane r < K of wave 0 takes the logit of the token's given expert r; the logit
    // loads wait for the routing, so they are issued with the expert rows, and the values reach
    // LDS only after the dot products
    __shared__ float lgs[MAX_DEC_K];
    const int my_e = ROUTED ? expert_of(min((int)threadIdx.x, K - 1)) : 0;
    float my_l = 0.0f;
    // one load of the adapter index, clamped per projection (every further load of it would be
    // a round trip of its own before the rows it addresses)
    // (loaded unconditionally, from a stand-in address without adapters: a load under a branch
    // is waited for inside the branch)
    const int araw_l = *(a.adapter ? a.adapter + t : reinterpret_cast<const int32_t*>(a.x));
    __builtin_amdgcn_sched_barrier(0);   // the routing and the adapter index are issued first
    // the shared expert's rows: slot s takes rows s and s + slots (< DN_ROWS); slots past
    // them read the block's first row again, unused
    RowRegs<4, 1> rsh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = slot + j * slots;
        const bool ok = r < DN_ROWS && n0 + r < H;
        rsh[j].load(a.shd.p, a.shd.s, a.shd.b, Kd, (long)(ok ? n0 + r : n0), lpr, sl, ok);
    }
    int araw = 0;
    auto clamp_ad = [&](int n) {
        const int v = a.adapter ? araw : 0;
        return v < 0 ? 0 : (v >= n ? n - 1 : v);
    };
    // routing weights: published by the gate/up launch, or (ROUTED) the softmax of the router
    // logits over the given set (below)
    float selw[MAX_DEC_K];
    if constexpr (!ROUTED) {
#pragma unroll
        for (int r = 0; r < MAX_DEC_K; ++r) selw[r] = a.wts[(long)t * K + min(r, K - 1)];
    }
    const uint16_t* hsrow = a.hs + (long)t * Kd;
    const uint4* hbase4 = reinterpret_cast<const uint4*>(a.h + (long)t * K * Kd);
    const uint4* hsrow4 = reinterpret_cast<const uint4*>(hsrow);
    auto rowp = [=](int m) { return m < K ? hbase4 + (long)m * (Kd / 8) : hsrow4; };
    StageRegs<4, DN_STAGE> st;
    st.load(rowp, n_staged, Kd);   // always (clamped, in bounds): loads under a branch are
                                   // waited for at its merge; unused unless one_pass
    // (ZP) z_d shares: thread i < 16 nbs holds share i / 16 of rank row i % 16
    __shared__ float zpl[DEC_ZP_BLOCKS * DEC_ZP_RANK];
    const int nbs = Kd / 64;
    float zpv[2];
    if constexpr (ZP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = (int)threadIdx.x + NT * j;
            zpv[j] = a.zd[((long)t * DEC_ZP_BLOCKS + min(i / DEC_ZP_RANK, nbs - 1)) * DEC_ZP_RANK + i % DEC_ZP_RANK];
        }
    }
    // the combine's own inputs (gate logit, residual x) now, not after the dots
    float gate_t;
    uint16_t x_res;
    {   // every thread loads (rows clamped; only threads < DN_ROWS use them): no branch
        const int nn = min(n0 + (int)(threadIdx.x % DN_ROWS), H - 1);
        gate_t = a.gate[t];
        x_res = a.x[(long)t * H + nn];
    }
    // nothing below may be scheduled above this point: what follows waits for the routing or
    // the adapter index, and a wait placed earlier would hold back the loads above
    __builtin_amdgcn_sched_barrier(0);
    // the adapter index is first read here (the compiler would otherwise move it to a scalar
    // register right after its load, and wait for the load there)
    araw = araw_l;
    asm volatile("" : "+v"(araw));

    // phase 1b: the LoRA rows (they need the adapter index)
    const int ad = clamp_ad(a.nad);
    constexpr int ZI = 4;                      // A_down slice: Kd/16 <= 32 inputs per lane
    const int lane16 = threadIdx.x & 15, zrow = threadIdx.x >> 4;
    const int zper = Kd / 16;
    const bool zfast = !ZP && a.Ad && a.rd <= 16 && zper <= 8 * ZI;
    constexpr int BQ = 2;   // prefetched B rows up to rank 16; larger ranks read B at the end
    uint4 bq[BQ];
    const bool bfast = a.Bd && (a.rd & 7) == 0 && a.rd <= 8 * BQ;
    {   // loaded unconditionally (stand-in: the token's x row): under a branch the compiler
        // copies the loaded registers at the merge, and a copy waits for every load in flight
        const int nn = min(n0 + (int)(threadIdx.x % DN_ROWS), H - 1);
        const uint4* brow = bfast ? reinterpret_cast<const uint4*>(a.Bd + ((long)ad * H + nn) * a.rd)
                                  : reinterpret_cast<const uint4*>(a.x + (long)t * H);
#pragma unroll
        for (int i = 0; i < BQ; ++i) bq[i] = brow[bfast ? min(i, a.rd / 8 - 1) : 0];
    }
    uint4 av[ZI];
    if constexpr (!ZP) {   // unconditional as well (stand-in: the token's x row)
        const uint16_t* arow = zfast ? a.Ad + ((long)ad * a.rd + min(zrow, a.rd - 1)) * Kd + lane16 * zper
                                     : a.x + (long)t * H;
#pragma unroll
        for (int i = 0; i < ZI; ++i) av[i] = *reinterpret_cast<const uint4*>(arow + (zfast ? min(i * 8, zper - 8) : 0));
    }
    // the LoRA-B term of the block's output row threadIdx.x (< DN_ROWS): B_d row . z_d (LDS)
    auto bz_dot = [&]() {
#pragma unroll
        for (int i = 0; i < BQ; ++i) hold(bq[i]);
        float zv[8 * BQ];   // read unconditionally (entries past the rank are not used)
#pragma unroll
        for (int j = 0; j < 8 * BQ; ++j) zv[j] = zd[j];
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < BQ; ++i) {
            if (i < a.rd / 8) {
                const uint32_t w4[4] = {bq[i].x, bq[i].y, bq[i].z, bq[i].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    d = fmaf(half_lo(w4[u]), zv[i * 8 + 2 * u], d);
                    d = fmaf(half_hi(w4[u]), zv[i * 8 + 2 * u + 1], d);
                }
            }
        }
        return d;
    };
    float lora_pre = 0.0f, sig_pre = 0.0f;   // (ZP) taken before the dot products
    // phase 2: the K + 1 down rows' loads (they need only the routing)
    RowRegs<4, 1> rr[NI];
    int mi[NI], ri[NI];
    auto load_items = [&](int base) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int item = base + i * slots + slot;
            const int ic = min(item, n_items - 1);
            const int m = ic / DN_ROWS, r = ic % DN_ROWS;
            const bool ok = item < n_items && n0 + r < H;
            const int nn = ok ? n0 + r : 0;
            const int e = base == 0 ? eit[i] : expert_of(min(m, K - 1));
            mi[i] = ok ? m : -1;
            ri[i] = r;
            rr[i].load(a.ed.p, a.ed.s, a.ed.b, Kd, (long)e * H + nn, lpr, sl, ok);
        }
    };
    load_items(0);
#pragma unroll
    for (int j = 0; j < 2; ++j) rsh[j].hold();   // their first use after the routed rows' issue
    float my_b = 0.0f;   // the bias, added at the end (a branch around its load would wait for it)
    if constexpr (ROUTED) {
        my_l = a.logits[(long)t * a.Ep + my_e];
        my_b = (a.rbias ? a.rbias : a.logits)[my_e];
    }
    // phase 3: activations to LDS
    if (one_pass) st.commit(n_staged, Kd, hs_l, hsum);
    else stage_rows<4, 4>(rowp, n_staged, Kd, hs_l, hsum);
    if constexpr (ZP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = (int)threadIdx.x + NT * j;
            if (i < nbs * DEC_ZP_RANK) zpl[i] = zpv[j];
        }
    }
    __syncthreads();
    // z_down = A_down[ad] . h_s[t], from the staged h_s in the pair order of A's registers
    if (zfast) {
#pragma unroll
        for (int i = 0; i < ZI; ++i) hold(av[i]);
        const f16x2* hp = hs_l + K * (Kd / 2) + lane16 * (zper / 2);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < ZI; ++i) {
            if (i * 8 < zper) {
                const uint4 ap = pair_perm8_w(av[i]);
                acc = __builtin_amdgcn_fdot2(as_h2(ap.x), hp[i * 4 + 0], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ap.y), hp[i * 4 + 1], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ap.z), hp[i * 4 + 2], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ap.w), hp[i * 4 + 3], acc, false);
            }
        }
        acc = seg_sum<16>(acc);
        if (lane16 == 0 && zrow < a.rd) zd[zrow] = acc;
    } else if (ZP) {
        if (threadIdx.x < DEC_ZP_RANK) {   // the shares in row-block order
            float z = 0.0f;
            for (int b = 0; b < nbs; ++b) z += zpl[b * DEC_ZP_RANK + threadIdx.x];
            zd[threadIdx.x] = z;
        }
        // the combine's LoRA term and gate now, while the weight rows are in flight (wave 0
        // wrote zd and reads it back: the LDS accesses of one wave complete in order, so only
        // the compiler needs a fence)
        asm volatile("" ::: "memory");
        if (threadIdx.x < DN_ROWS) {
            if (bfast) lora_pre = bz_dot();
            sig_pre = sigmoid(gate_t);
        }
    } else if (a.Ad) {
        lora_rows16(a.Ad + (long)ad * a.rd * Kd, a.rd, hsrow, Kd, zd);
    }
    // the shared expert's outputs first (its rows were issued before the routing arrived)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = slot + j * slots;
        if (r < DN_ROWS) {   // uniform over each wave (slots of a wave are consecutive)
            float acc[MT];
            acc[0] = 0.0f;
            rsh[j].dot(Kd, lpr, sl, hs_l + K * (Kd / 2), hsum + K * (Kd / 32), 1, acc);
            const float v = segment_sum(acc[0], lpr);
            if (sl == 0) o_l[K * DN_ROWS + r] = v;
        }
    }
    for (int base = 0; base < n_items; base += slots * NI) {
        if (base > 0) load_items(base);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float acc[MT];
            acc[0] = 0.0f;
            const int m = mi[i] < 0 ? 0 : mi[i];
            rr[i].dot(Kd, lpr, sl, hs_l + m * (Kd / 2), hsum + m * (Kd / 32), 1, acc);
            const float v = segment_sum(acc[0], lpr);
            if (sl == 0 && mi[i] >= 0) o_l[mi[i] * DN_ROWS + ri[i]] = v;
        }
    }
    if (ROUTED && threadIdx.x < K) lgs[threadIdx.x] = a.rbias ? my_l + my_b : my_l;
    __syncthreads();
    if constexpr (ROUTED) {
        if (threadIdx.x < DN_ROWS) {
            float lg[MAX_DEC_K];
#pragma unroll
            for (int r = 0; r < MAX_DEC_K; ++r) lg[r] = lgs[min(r, K - 1)];
            given_softmax<MAX_DEC_K>(K, lg, selw);
        }
    }
    if (threadIdx.x < DN_ROWS) {
        const int r = threadIdx.x, n = n0 + r;
        if (n < H) {
            // every LDS read first (a read under a branch would be a round trip of its own)
            float ov[MAX_DEC_K];
#pragma unroll
            for (int k = 0; k < MAX_DEC_K; ++k) ov[k] = o_l[min(k, K - 1) * DN_ROWS + r];
            float os = o_l[K * DN_ROWS + r];
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < MAX_DEC_K; ++k)
                if (k < K) acc = fmaf(selw[k], ov[k], acc);
            if (bfast) {
                os = fmaf(a.lsd, ZP ? lora_pre : bz_dot(), os);
            } else if (a.Bd) {
                os = fmaf(a.lsd, lora_b_dot(a.Bd, ad, H, n, a.rd, zd), os);
            }
            acc = fmaf(ZP ? sig_pre : sigmoid(gate_t), os, acc);
            uint16_t outv = f2h(acc);
            if (a.add_residual) outv = f2h(h2f(x_res) + h2f(outv));
            a.y[(long)t * H + n] = outv;
        }
    }
    if (ROUTED && a.w_out && blockIdx.x == 0 && threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < MAX_DEC_K; ++k)
            if (k < K) a.w_out[(long)t * K + k] = selw[k];
    }
}

}  // namespace

static int chunks_per_lane(int K) { return (K / 32) / lanes_per_row(K); }

// routed items per lane segment per pass of the down kernel: 2 when the K experts' rows of a
// block fill at most two passes' worth of segments, else DN_ITEMS
static int dn_items(const MoeArgs& a) {
    const int slots = 4 * (64 / lanes_per_row(a.I));
    return a.K * DN_ROWS <= 2 * slots ? 2 : DN_ITEMS;
}

// The register and LDS budgets of the decode kernels: hidden rows of at most two 32-input
// chunks per lane (hidden <= 4096), down rows of one chunk per lane (inter <= 2048, a power
// of two), equal routed and shared intermediate sizes.
// The decode path re-reads an expert for every (token, k) pair that uses it; from about 32
// pairs on, the token-sorted path (each used expert read once, MFMA) is faster on MI355X
// (measured at 16 x 8, 8 x 8, 8 x 4 and 4 x 8 pairs), below it its fixed route cost loses.
bool decode_path_fits(const qmoe_moe_layer& L, int T) {
    // routed experts in groups of 32 or with bf16 parameters run the token-sorted path
    const bool std_experts = L.exp_gate.group == 64 && L.exp_gate.param_dtype == QMOE_PARAM_F16;
    return std_experts && T * L.top_k < 32 && T <= MAX_DEC_T && L.top_k <= MAX_DEC_K && L.inter == L.shared_inter &&
           L.hidden <= 4096 && L.inter <= 2048 && chunks_per_lane(L.hidden) <= 2 &&
           chunks_per_lane(L.inter) <= 1;
}

hipError_t launch_moe_decode(const MoeArgs& a, int stage, hipStream_t s) {
    const int nx = xside_blocks(a);
    if (a.route) {   // the caller's routing: two launches
        const int rpb = 4 * (64 / lanes_per_row(a.H)) * GU_RPW;
        const int nrb = (a.I + rpb - 1) / rpb;
        // x side: the router and shared-gate rows only (the shared expert's gate/up and LoRA
        // z's run in the shared blocks, which finish h_s)
        const XsideGrid g = xside_grid(a.T, a.H, a.E, a.SI, 0);
        const int nxr = g.nb_router + g.nb_gate;
        const int ns = a.T * ((a.SI + rpb - 1) / rpb);
        k_dec_rt_gate_up<<<(unsigned)(nxr + ns + nrb * a.T * a.K), 256, 0, s>>>(a, nxr, ns);
        dim3 grid((unsigned)((a.H + DN_ROWS - 1) / DN_ROWS), (unsigned)a.T);
        if (dn_items(a) == 2) k_dec_down<true, false, 2><<<grid, 256, 0, s>>>(a);
        else k_dec_down<true, false, DN_ITEMS><<<grid, 256, 0, s>>>(a);
        return hipGetLastError();
    }
    if (stage == QMOE_STAGE_ALL || stage == QMOE_STAGE_ROUTE)
        k_dec_xside<<<nx, 256, 0, s>>>(a);
    const int per = topk_per_lane(a.E);
    if (stage == QMOE_STAGE_ALL || stage == QMOE_STAGE_GATE_UP) {
        const int rpb = 4 * (64 / lanes_per_row(a.H)) * GU_RPW;
        // x: the routed row blocks, and for the shared slot (y = T K) SI / 64 blocks per token
        dim3 grid((unsigned)std::max((a.I + rpb - 1) / rpb, a.T * (a.SI / 64)), (unsigned)(a.T * a.K + 1));
        switch (per) {
            case 1: k_dec_gate_up<1><<<grid, 256, 0, s>>>(a); break;
            case 2: k_dec_gate_up<2><<<grid, 256, 0, s>>>(a); break;
            case 4: k_dec_gate_up<4><<<grid, 256, 0, s>>>(a); break;
            case 8: k_dec_gate_up<8><<<grid, 256, 0, s>>>(a); break;
            default: k_dec_gate_up<16><<<grid, 256, 0, s>>>(a); break;
        }
    }
    if (stage == QMOE_STAGE_ALL || stage == QMOE_STAGE_DOWN) {
        dim3 grid((unsigned)((a.H + DN_ROWS - 1) / DN_ROWS), (unsigned)a.T);
        const bool zp = a.Ad && a.rd <= DEC_ZP_RANK;
        if (dn_items(a) == 2) {
            if (zp) k_dec_down<false, true, 2><<<grid, 256, 0, s>>>(a);
            else k_dec_down<false, false, 2><<<grid, 256, 0, s>>>(a);
        } else {
            if (zp) k_dec_down<false, true, DN_ITEMS><<<grid, 256, 0, s>>>(a);
            else k_dec_down<false, false, DN_ITEMS><<<grid, 256, 0, s>>>(a);
        }
    }
    return hipGetLastError();
}

}  // namespace qmoe
