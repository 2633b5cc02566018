// MoE SwitchGLU layer with int4 group-affine experts, a sigmoid-gated shared expert and
// unmerged LoRA deltas on the shared expert's projections.
//
// What the layer computes follows the pages: 256 routed experts with gate/up/down
// projections stored as switch_mlp.{gate,up,down}_proj plus a shared expert with
// shared_expert_gate ("Edge0-35B-A3B Preview model repository guide", model spec table
// and shared-expert paragraph); int4 group-64 affine weights with the router and the
// shared-expert gate at 8 bits ("Recover-LoRA ..." section 1); K experts per token under
// the SOFTMAX_TOPK routing family, SiLU(gate) * up as in _swiglu(up, gate), routing that
// never leaves the device, empty experts contributing nothing ("Edge0 project review",
// highlight 2 and MoE spec); the recovery LoRA as a parallel, never-merged delta
// ("Recover-LoRA ..." section 2).
//
// Two launch sequences on the caller's stream, neither with a host synchronisation:
//   decode (moe_decode.hip, up to 32 tokens): three launches, top-K once per token inside
//     the gate/up kernel; with a routing given by the caller, two;
//   prefill (moe_prefill.hip, any count): router / shared-expert GEMMs on MFMA, top-K, a
//     stable sort of the (token, k) pairs by expert, grouped expert GEMMs, combine.
// This file owns the workspace layout and the choice between the two.
#include <algorithm>
#include <mutex>

#include "gemv_core.hpp"
#include "launch.hpp"
#include "moe_common.hpp"

namespace qmoe {

namespace {

struct Layout {
    size_t logits, gate, zg, zu, zd, gs, us, idx, wts, scnt, wrec, wpairs, h, hs, o, os,
        total;
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout layout_of(const qmoe_moe_layer& L, int T) {
    Layout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t r = off; off = up256(off + bytes); return r; };
    const size_t TK = (size_t)T * L.top_k;
    // sized for the largest split and the smallest work items at any token count, so that a
    // workspace sized for max_tokens serves every smaller call (the offsets depend on T only
    // through T itself)
    const size_t ks = (size_t)L.hidden / 512;   // split-K partials of the x side (at most)
    l.logits = take(ks * T * ((L.n_experts + 63) / 64 * 64) * 4);
    l.gate = take(ks * T * 4);
    // LoRA z of gate and up: partial sums per 256 inputs (prefill), the first slice for decode
    l.zg = take((size_t)(L.hidden / 256) * T * MAX_RANK * 4);
    l.zu = take((size_t)(L.hidden / 256) * T * MAX_RANK * 4);
    // z_down (prefill), or the decode path's per-row-block shares of it (at most MAX_DEC_T tokens)
    l.zd = take((size_t)std::max(T * MAX_RANK, std::min(T, MAX_DEC_T) * DEC_ZP_BLOCKS * DEC_ZP_RANK) * 4);
    l.gs = take(ks * T * L.shared_inter * 4);
    l.us = take(ks * T * L.shared_inter * 4);
    l.idx = take(TK * 4);
    l.wts = take(TK * 4);
    l.scnt = take((size_t)PF_SORT_MAXSEG * L.n_experts * 4);
    const size_t items = ((size_t)L.n_experts + (TK + 15) / 16 + 7) / 8 * 8;   // >= the sort's items
    l.wrec = take(items * 16);
    l.wpairs = take(items * PF_ITEM * 4);
    l.h = take(TK * L.inter * 2);
    l.hs = take((size_t)T * L.shared_inter * 2);
    l.o = take(TK * L.hidden * 2);
    l.os = take((size_t)T * L.hidden * 4);
    l.total = off;
    return l;
}

}  // namespace

size_t moe_workspace_bytes(const qmoe_moe_layer& L, int max_tokens) {
    return layout_of(L, max_tokens).total;
}

}  // namespace qmoe

// Workspace of the allocation-free layer call: one copy per device, held from the first
// call on that device until the process ends.  Host code never uses this name as an
// address (on the host it is a stand-in, not device memory); it uses the device address
// that moe_noalloc_scratch() looks up once per device.
static __device__ __align__(256) unsigned char scratch[qmoe::MOE_NOALLOC_SCRATCH_BYTES];

namespace qmoe {

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES];
}  // namespace

hipError_t moe_noalloc_scratch(hipStream_t s, void** ptr) {
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

hipError_t launch_moe(const qmoe_moe_layer& L, int stage, const uint16_t* x, int T,
                      const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                      float* w_out, void* ws, hipStream_t s, const int32_t* route) {
    const Layout lo = layout_of(L, T);
    char* base = static_cast<char*>(ws);
    MoeArgs a{};
    a.T = T; a.H = L.hidden; a.I = L.inter; a.SI = L.shared_inter; a.E = L.n_experts;
    a.K = L.top_k; a.add_residual = L.add_residual;
    a.Ep = (L.n_experts + 63) / 64 * 64;
    a.x = x; a.y = y; a.adapter = adapter_idx;
    auto qw = [](const qmoe_qweight& w) { return QW{w.packed, w.scales, w.biases}; };
    a.router = qw(L.router); a.sgate = qw(L.shared_gate);
    a.eg = qw(L.exp_gate); a.eu = qw(L.exp_up); a.ed = qw(L.exp_down);
    a.shg = qw(L.sh_gate); a.shu = qw(L.sh_up); a.shd = qw(L.sh_down);
    if (L.lora_gate) { a.Ag = L.lora_gate->A; a.Bg = L.lora_gate->B; a.rg = L.lora_gate->rank; a.lsg = L.lora_gate->scale; a.nag = L.lora_gate->n_adapters; }
    if (L.lora_up) { a.Au = L.lora_up->A; a.Bu = L.lora_up->B; a.ru = L.lora_up->rank; a.lsu = L.lora_up->scale; a.nau = L.lora_up->n_adapters; }
    if (L.lora_down) { a.Ad = L.lora_down->A; a.Bd = L.lora_down->B; a.rd = L.lora_down->rank; a.lsd = L.lora_down->scale; a.nad = L.lora_down->n_adapters; }
    a.rbias = L.router_bias;
    a.logits = reinterpret_cast<float*>(base + lo.logits);
    a.gate = reinterpret_cast<float*>(base + lo.gate);
    a.zg = reinterpret_cast<float*>(base + lo.zg);
    a.zu = reinterpret_cast<float*>(base + lo.zu);
    a.zd = reinterpret_cast<float*>(base + lo.zd);
    a.gs = reinterpret_cast<float*>(base + lo.gs);
    a.us = reinterpret_cast<float*>(base + lo.us);
    a.idx = reinterpret_cast<int32_t*>(base + lo.idx);
    a.wts = reinterpret_cast<float*>(base + lo.wts);
    a.scnt = reinterpret_cast<int32_t*>(base + lo.scnt);
    a.wrec = reinterpret_cast<int32_t*>(base + lo.wrec);
    a.wpairs = reinterpret_cast<int32_t*>(base + lo.wpairs);
    a.h = reinterpret_cast<uint16_t*>(base + lo.h);
    a.hs = reinterpret_cast<uint16_t*>(base + lo.hs);
    a.o = reinterpret_cast<uint16_t*>(base + lo.o);
    a.os = reinterpret_cast<float*>(base + lo.os);
    a.idx_out = idx_out;
    a.w_out = w_out;
    a.route = route;
    a.egroup = L.exp_gate.group;
    a.ebf = L.exp_gate.param_dtype == QMOE_PARAM_BF16;
    if (decode_path_fits(L, T)) return launch_moe_decode(a, stage, s);
    return launch_moe_prefill(a, stage, s);
}

}  // namespace qmoe
