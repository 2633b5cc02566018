// Decode path of the MoE SwitchGLU layer (a few tokens per call): three launches, no sort,
// no atomics, top-K recomputed where it is needed.
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
//                then h = silu(g) * u is stored (fp16).  Shared blocks add the LoRA
//                up-projections and store h_s.
//   D3 down    : one block per (row block, token).  It recomputes the token's top-K,
//                stages the token's K expert activations h and h_s, computes the shared
//                expert's LoRA z_down, streams the K + 1 down matrices' rows, and combines
//                y = sum_k w_k o_k + sigmoid(gate) (o_s + LoRA) (+ residual) in-block.
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

__global__ void __launch_bounds__(256) k_dec_xside(MoeArgs a) {
    __shared__ __align__(16) f16x2 xs[8192];   // 32 KB: 8192 / (hidden / 2) tokens per pass
    __shared__ float xsum[MT * 128];
    // every argument field of the kernel in one batch of scalar loads (one round trip)
    asm volatile("" ::"s"(a.router.p), "s"(a.router.s), "s"(a.router.b), "s"(a.x), "s"(a.shg.p),
                 "s"(a.shg.s), "s"(a.shg.b), "s"(a.logits), "s"(a.shu.p), "s"(a.shu.s), "s"(a.shu.b),
                 "s"(a.gs), "s"(a.us), "s"(a.T), "s"(a.H), "s"(a.E), "s"(a.SI), "s"(a.Ep), "s"(a.Ag),
                 "s"(a.Au), "s"(a.rg), "s"(a.ru), "s"(a.gate), "s"(a.sgate.p), "s"(a.sgate.s),
                 "s"(a.sgate.b), "s"(a.zg), "s"(a.zu));
    const int H = a.H;
    const int zjobs = (a.Ag ? a.T * a.rg : 0) + (a.Au ? a.T * a.ru : 0);
    const XsideGrid g = xside_grid(a.T, H, a.E, a.SI, zjobs);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = lanes_per_row(H), rpw = 64 / lpr, seg = lane / lpr;
    const int b = blockIdx.x;

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

// ------------------------------------------------------------------------------ D2 gate/up

constexpr int GU_RPW = 1;  // gate/up row pairs per wave

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

    if (pair == TK) {  // shared expert: LoRA up-projections, silu(g) * u
        const int n0 = blockIdx.x * rows_per_block;
        for (int it = threadIdx.x; it < rows_per_block * a.T; it += NT) {
            const int n = n0 + it % rows_per_block, t = it / rows_per_block;
            if (n >= a.SI) continue;
            float gv = a.gs[(long)t * a.SI + n];
            float uv = a.us[(long)t * a.SI + n];
            if (a.Bg) gv = fmaf(a.lsg, lora_b_dot(a.Bg, adapter_of(a.adapter, t, a.nag), a.SI, n, a.rg, a.zg + t * MAX_RANK), gv);
            if (a.Bu) uv = fmaf(a.lsu, lora_b_dot(a.Bu, adapter_of(a.adapter, t, a.nau), a.SI, n, a.ru, a.zu + t * MAX_RANK), uv);
            a.hs[(long)t * a.SI + n] = f2h(silu(gv) * uv);
        }
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

// ------------------------------------------------------------------------------ D3 down

constexpr int DN_ROWS = 8;     // output rows per block
constexpr int DN_ITEMS = 4;    // (matrix, row) items per lane segment per pass
constexpr int DN_STAGE = 3;    // 16-byte staging loads per thread: (K + 1) * inter / 8 <= 768

__global__ void __launch_bounds__(256) k_dec_down(MoeArgs a) {
    // staged activations: the token's K routed h rows and h_s (as matrix K), pair layout
    __shared__ __align__(16) f16x2 hs_l[(MAX_DEC_K + 1) * 1024];   // inter <= 2048
    QMOE_SGPR_USE4(a.idx, a.wts, a.h, a.hs);
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
    const bool one_pass = (K + 1) * (Kd / 8) <= 256 * DN_STAGE;

    // phase 1: the routing decision (published by the gate/up stage), the K + 1 activation
    // rows and the LoRA A_down slices in flight together.  Each lane loads the expert of its
    // own first-pass items first (per-lane loads: a per-lane pick from a uniform array would
    // become an indexed scratch access whose wait drains every load in flight).
    // the token's adapter first: the addresses of the LoRA rows wait for it, and loads
    // complete in issue order, so a load issued later would make that wait longer
    const int ad = adapter_of(a.adapter, t, a.nad);
    const int n_items = (K + 1) * DN_ROWS;
    const int slots = 4 * rpw;            // lane segments in the block
    const int slot = wave * rpw + seg;
    int eit[DN_ITEMS];
#pragma unroll
    for (int i = 0; i < DN_ITEMS; ++i) {
        const int m = min(i * slots + slot, n_items - 1) / DN_ROWS;
        eit[i] = a.idx[(long)t * K + min(m, K - 1)];
    }
    float selw[MAX_DEC_K];
#pragma unroll
    for (int r = 0; r < MAX_DEC_K; ++r) selw[r] = a.wts[(long)t * K + min(r, K - 1)];
    const uint16_t* hsrow = a.hs + (long)t * Kd;
    const uint4* hbase4 = reinterpret_cast<const uint4*>(a.h + (long)t * K * Kd);
    const uint4* hsrow4 = reinterpret_cast<const uint4*>(hsrow);
    auto rowp = [=](int m) { return m < K ? hbase4 + (long)m * (Kd / 8) : hsrow4; };
    StageRegs<4, DN_STAGE> st;
    if (one_pass) st.load(rowp, K + 1, Kd);
    constexpr int ZI = 4;                      // A_down slice: Kd/16 <= 32 inputs per lane
    const int lane16 = threadIdx.x & 15, zrow = threadIdx.x >> 4;
    const int zper = Kd / 16;
    const bool zfast = a.Ad && a.rd <= 16 && zper <= 8 * ZI;
    // the combine's own inputs (gate logit, residual x, LoRA-B rows of this block's outputs)
    // are loaded now, not after the dots: one round trip less at the end
    constexpr int BQ = 2;   // prefetched B rows up to rank 16; larger ranks read B at the end
    uint4 bq[BQ];
    float gate_t = 0.0f;
    uint16_t x_res = 0;
    const bool bfast = a.Bd && (a.rd & 7) == 0 && a.rd <= 8 * BQ;
    {   // every thread loads (rows clamped; only threads < DN_ROWS use them): no branch
        const int nn = min(n0 + (int)(threadIdx.x % DN_ROWS), H - 1);
        gate_t = a.gate[t];
        x_res = a.x[(long)t * H + nn];
        // loaded unconditionally (stand-in: the token's x row): under a branch the compiler
        // copies the loaded registers at the merge, and a copy waits for every load in flight
        const uint4* brow = bfast ? reinterpret_cast<const uint4*>(a.Bd + ((long)ad * H + nn) * a.rd)
                                  : reinterpret_cast<const uint4*>(a.x + (long)t * H);
#pragma unroll
        for (int i = 0; i < BQ; ++i) bq[i] = brow[bfast ? min(i, a.rd / 8 - 1) : 0];
    }
    uint4 av[ZI];
    {   // unconditional as well (stand-in: the token's x row)
        const uint16_t* arow = zfast ? a.Ad + ((long)ad * a.rd + min(zrow, a.rd - 1)) * Kd + lane16 * zper
                                     : a.x + (long)t * H;
#pragma unroll
        for (int i = 0; i < ZI; ++i) av[i] = *reinterpret_cast<const uint4*>(arow + (zfast ? min(i * 8, zper - 8) : 0));
    }
    // phase 2: the K + 1 down rows' loads (they need only the routing)
    RowRegs<4, 1> rr[DN_ITEMS];
    int mi[DN_ITEMS], ri[DN_ITEMS];
    auto load_items = [&](int base) {
#pragma unroll
        for (int i = 0; i < DN_ITEMS; ++i) {
            const int item = base + i * slots + slot;
            const int ic = min(item, n_items - 1);
            const int m = ic / DN_ROWS, r = ic % DN_ROWS;
            const bool ok = item < n_items && n0 + r < H;
            const int nn = ok ? n0 + r : 0;
            const int e = base == 0 ? eit[i] : a.idx[(long)t * K + min(m, K - 1)];
            mi[i] = ok ? m : -1;
            ri[i] = r;
            const bool routed = m < K;
            rr[i].load(routed ? a.ed.p : a.shd.p, routed ? a.ed.s : a.shd.s,
                       routed ? a.ed.b : a.shd.b, Kd, routed ? (long)e * H + nn : (long)nn,
                       lpr, sl, ok);
        }
    };
    load_items(0);
    // phase 3: activations to LDS
    if (one_pass) st.commit(K + 1, Kd, hs_l, hsum);
    else stage_rows<4, 4>(rowp, K + 1, Kd, hs_l, hsum);
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
    } else if (a.Ad) {
        lora_rows16(a.Ad + (long)ad * a.rd * Kd, a.rd, hsrow, Kd, zd);
    }
    for (int base = 0; base < n_items; base += slots * DN_ITEMS) {
        if (base > 0) load_items(base);
#pragma unroll
        for (int i = 0; i < DN_ITEMS; ++i) {
            float acc[MT];
            acc[0] = 0.0f;
            const int m = mi[i] < 0 ? 0 : mi[i];
            rr[i].dot(Kd, lpr, sl, hs_l + m * (Kd / 2), hsum + m * (Kd / 32), 1, acc);
            const float v = segment_sum(acc[0], lpr);
            if (sl == 0 && mi[i] >= 0) o_l[mi[i] * DN_ROWS + ri[i]] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x < DN_ROWS) {
        const int r = threadIdx.x, n = n0 + r;
        if (n < H) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < MAX_DEC_K; ++k)
                if (k < K) acc = fmaf(selw[k], o_l[k * DN_ROWS + r], acc);
            float os = o_l[K * DN_ROWS + r];
            if (bfast) {
#pragma unroll
                for (int i = 0; i < BQ; ++i) hold(bq[i]);
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < BQ; ++i) {
                    if (i < a.rd / 8) {
                        const uint32_t w4[4] = {bq[i].x, bq[i].y, bq[i].z, bq[i].w};
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            d = fmaf(half_lo(w4[u]), zd[i * 8 + 2 * u], d);
                            d = fmaf(half_hi(w4[u]), zd[i * 8 + 2 * u + 1], d);
                        }
                    }
                }
                os = fmaf(a.lsd, d, os);
            } else if (a.Bd) {
                os = fmaf(a.lsd, lora_b_dot(a.Bd, ad, H, n, a.rd, zd), os);
            }
            acc = fmaf(sigmoid(gate_t), os, acc);
            uint16_t outv = f2h(acc);
            if (a.add_residual) outv = f2h(h2f(x_res) + h2f(outv));
            a.y[(long)t * H + n] = outv;
        }
    }
}

}  // namespace

static int chunks_per_lane(int K) { return (K / 32) / lanes_per_row(K); }

// The register and LDS budgets of the decode kernels: hidden rows of at most two 32-input
// chunks per lane (hidden <= 4096), down rows of one chunk per lane (inter <= 2048, a power
// of two), equal routed and shared intermediate sizes.
// The decode path re-reads an expert for every (token, k) pair that uses it; from about 32
// pairs on, the token-sorted path (each used expert read once, MFMA) is faster on MI355X
// (measured at 16 x 8, 8 x 8, 8 x 4 and 4 x 8 pairs), below it its fixed route cost loses.
bool decode_path_fits(const qmoe_moe_layer& L, int T) {
    return T * L.top_k < 32 && T <= MAX_DEC_T && L.top_k <= MAX_DEC_K && L.inter == L.shared_inter &&
           L.hidden <= 4096 && L.inter <= 2048 && chunks_per_lane(L.hidden) <= 2 &&
           chunks_per_lane(L.inter) <= 1;
}

hipError_t launch_moe_decode(const MoeArgs& a, int stage, hipStream_t s) {
    const int zjobs = (a.Ag ? a.T * a.rg : 0) + (a.Au ? a.T * a.ru : 0);
    const XsideGrid g = xside_grid(a.T, a.H, a.E, a.SI, zjobs);
    if (stage == QMOE_STAGE_ALL || stage == QMOE_STAGE_ROUTE)
        k_dec_xside<<<g.nb_router + g.nb_gate + g.nb_shared + g.nb_z, 256, 0, s>>>(a);
    const int per = topk_per_lane(a.E);
    if (stage == QMOE_STAGE_ALL || stage == QMOE_STAGE_GATE_UP) {
        const int rpb = 4 * (64 / lanes_per_row(a.H)) * GU_RPW;
        dim3 grid((unsigned)((std::max(a.I, a.SI) + rpb - 1) / rpb), (unsigned)(a.T * a.K + 1));
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
        k_dec_down<<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace qmoe
