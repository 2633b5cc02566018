// C ABI of libqmoe: argument validation, then the internal launchers (launch.hpp).
// Every check happens before anything is enqueued; a failed check returns a negative
// status and leaves the outputs untouched.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"
#include "qmoe.h"

namespace {

constexpr int MAX_COLS = 16384;
static_assert(qmoe::MOE_NOALLOC_SCRATCH_BYTES == QMOE_NOALLOC_SCRATCH_BYTES,
              "the header states the allocation-free call's scratch size");
constexpr int MAX_MOE_DIM = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
thread_local const char* g_last_error = "";

int hip_status(hipError_t e) {
    if (e == hipSuccess) return QMOE_OK;
    g_last_error = hipGetErrorString(e);
    return QMOE_ERR_HIP;
}

// A quantized matrix that the GEMV/GEMM kernels read: group 64 with fp16 parameters, or
// for the dense linear (`dense`) also group 32 and bf16 parameters.
int check_qweight(const qmoe_qweight* w, int bits_required, bool dense = false) {
    if (!w || !w->packed || !w->scales || !w->biases) return QMOE_ERR_INVALID_ARG;
    if (w->rows <= 0 || w->cols <= 0 || w->n_experts <= 0) return QMOE_ERR_INVALID_ARG;
    if (w->bits != 4 && w->bits != 8) return QMOE_ERR_UNSUPPORTED;
    if (bits_required && w->bits != bits_required) return QMOE_ERR_UNSUPPORTED;
    if (w->param_dtype != QMOE_PARAM_F16 && w->param_dtype != QMOE_PARAM_BF16) return QMOE_ERR_UNSUPPORTED;
    if (dense ? (w->group != 64 && w->group != 32) : (w->group != 64 || w->param_dtype != QMOE_PARAM_F16))
        return QMOE_ERR_UNSUPPORTED;
    if (w->cols % 512 != 0 || w->cols > MAX_COLS) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(w->packed) || !aligned16(w->scales) || !aligned16(w->biases)) return QMOE_ERR_MISALIGNED;
    return QMOE_OK;
}

int check_shape(const qmoe_qweight& w, int rows, int cols, int n_experts, int bits, bool any_format = false) {
    int st = check_qweight(&w, bits, any_format);
    if (st) return st;
    if (w.rows != rows || w.cols != cols || w.n_experts != n_experts) return QMOE_ERR_INVALID_ARG;
    return QMOE_OK;
}

bool steps_staged(int k) { return k == 512 || k == 1024 || k == 2048; }

int check_lora(const qmoe_lora* l, int in_dim, int out_dim) {
    if (!l) return QMOE_OK;
    if (!l->A || !l->B) return QMOE_ERR_INVALID_ARG;
    if (l->rank < 1 || l->n_adapters < 1) return QMOE_ERR_INVALID_ARG;
    if (l->rank > 64) return QMOE_ERR_UNSUPPORTED;
    if (l->in_dim != in_dim || l->out_dim != out_dim) return QMOE_ERR_INVALID_ARG;
    if (l->in_dim % 512 != 0) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(l->A) || !aligned16(l->B)) return QMOE_ERR_MISALIGNED;
    return QMOE_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

int check_layer(const qmoe_moe_layer* L) {
    if (!L) return QMOE_ERR_INVALID_ARG;
    const int H = L->hidden, I = L->inter, SI = L->shared_inter, E = L->n_experts;
    if (H <= 0 || I <= 0 || SI <= 0 || E <= 0 || L->top_k <= 0) return QMOE_ERR_INVALID_ARG;
    if (H % 512 || I % 512 || SI % 512) return QMOE_ERR_UNSUPPORTED;
    if (H > MAX_MOE_DIM || I > MAX_MOE_DIM || SI > MAX_MOE_DIM) return QMOE_ERR_UNSUPPORTED;
    if (E > 1024 || L->top_k > 32 || L->top_k > E) return QMOE_ERR_UNSUPPORTED;
    int st;
    if ((st = check_shape(L->router, E, H, 1, 8))) return st;
    if ((st = check_shape(L->shared_gate, 1, H, 1, 8))) return st;
    // routed expert stacks: group 64 with fp16 parameters, or (the port page's checkpoint
    // format) group 32 and/or bf16 parameters, the same for all three, for hidden and inter
    // of 512, 1024 or 2048
    if ((st = check_shape(L->exp_gate, I, H, E, 4, true))) return st;
    if ((st = check_shape(L->exp_up, I, H, E, 4, true))) return st;
    if ((st = check_shape(L->exp_down, H, I, E, 4, true))) return st;
    if (L->exp_up.group != L->exp_gate.group || L->exp_down.group != L->exp_gate.group ||
        L->exp_up.param_dtype != L->exp_gate.param_dtype || L->exp_down.param_dtype != L->exp_gate.param_dtype)
        return QMOE_ERR_UNSUPPORTED;
    if ((L->exp_gate.group != 64 || L->exp_gate.param_dtype != QMOE_PARAM_F16) && !(steps_staged(H) && steps_staged(I)))
        return QMOE_ERR_UNSUPPORTED;
    if ((st = check_shape(L->sh_gate, SI, H, 1, 4))) return st;
    if ((st = check_shape(L->sh_up, SI, H, 1, 4))) return st;
    if ((st = check_shape(L->sh_down, H, SI, 1, 4))) return st;
    if ((st = check_lora(L->lora_gate, H, SI))) return st;
    if ((st = check_lora(L->lora_up, H, SI))) return st;
    if ((st = check_lora(L->lora_down, SI, H))) return st;
    if (!aligned4(L->router_bias)) return QMOE_ERR_MISALIGNED;
    return QMOE_OK;
}

}  // namespace

extern "C" {

int qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char* qmoe_status_string(int status) {
    switch (status) {
        case QMOE_OK: return "ok";
        case QMOE_ERR_INVALID_ARG: return "invalid argument";
        case QMOE_ERR_UNSUPPORTED: return "unsupported shape or format";
        case QMOE_ERR_MISALIGNED: return "pointer not aligned (16 bytes; 4 for int32/fp32 arrays)";
        case QMOE_ERR_WORKSPACE: return "workspace missing or too small";
        case QMOE_ERR_HIP: return "kernel launch failed";
        default: return "unknown status";
    }
}

const char* qmoe_last_error(void) { return g_last_error; }

size_t qmoe_abi_struct_size(int which) {
    switch (which) {
        case 0: return sizeof(qmoe_qweight);
        case 1: return sizeof(qmoe_lora);
        case 2: return sizeof(qmoe_moe_layer);
        case 3: return sizeof(qmoe_prerouter);
        default: return 0;
    }
}

int qmoe_quantize_affine(const float* w, int32_t rows, int32_t cols, int32_t bits,
                         int32_t group, uint32_t* packed, uint16_t* scales,
                         uint16_t* biases, void* stream) {
    if (!w || !packed || !scales || !biases) return QMOE_ERR_INVALID_ARG;
    if (rows <= 0 || cols <= 0) return QMOE_ERR_INVALID_ARG;
    if ((bits != 4 && bits != 8) || (group != 64 && group != 32) || cols % 64) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(w) || !aligned16(packed)) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_quantize_affine(w, rows, cols, bits, group, packed, scales,
                                                   biases, as_stream(stream)));
}

int qmoe_unpack(const uint32_t* packed, int32_t rows, int32_t cols, int32_t bits, uint8_t* q,
                void* stream) {
    if (!packed || !q || rows <= 0 || cols <= 0) return QMOE_ERR_INVALID_ARG;
    if ((bits != 4 && bits != 8) || cols % 64) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(packed) || !aligned16(q)) return QMOE_ERR_MISALIGNED;
    const long n_words = (long)rows * cols * bits / 32;
    return hip_status(qmoe::launch_unpack(packed, n_words, bits, q, as_stream(stream)));
}

int qmoe_dequantize(const qmoe_qweight* w, float* out, void* stream) {
    if (!w || !w->packed || !w->scales || !w->biases || !out) return QMOE_ERR_INVALID_ARG;
    if (w->rows <= 0 || w->cols <= 0 || w->n_experts <= 0) return QMOE_ERR_INVALID_ARG;
    if ((w->bits != 4 && w->bits != 8) || (w->group != 64 && w->group != 32) || w->cols % 64)
        return QMOE_ERR_UNSUPPORTED;
    if (w->param_dtype != QMOE_PARAM_F16 && w->param_dtype != QMOE_PARAM_BF16) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(out) || !aligned16(w->packed)) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_dequantize(*w, out, as_stream(stream)));
}

int qlinear_int4(const uint16_t* x, int32_t m, const qmoe_qweight* w, const qmoe_lora* lora,
                 const int32_t* adapter_idx, uint16_t* y, void* stream) {
    if (!x || !y || m <= 0) return QMOE_ERR_INVALID_ARG;
    if (m > 4096) return QMOE_ERR_UNSUPPORTED;
    int st = check_qweight(w, 0, true);
    if (st) return st;
    if (w->n_experts != 1) return QMOE_ERR_INVALID_ARG;
    if ((st = check_lora(lora, w->cols, w->rows))) return st;
    if (!aligned16(x) || !aligned16(y)) return QMOE_ERR_MISALIGNED;
    if (overlap(x, (size_t)m * w->cols * 2, y, (size_t)m * w->rows * 2)) return QMOE_ERR_INVALID_ARG;
    return hip_status(qmoe::launch_qlinear_gemv(x, m, *w, lora, adapter_idx, y, as_stream(stream)));
}

int router_topk(const float* logits, int32_t t, int32_t e, int32_t k, const float* bias,
                int32_t* idx, float* weights, void* stream) {
    if (!logits || !idx || !weights || t <= 0 || e <= 0 || k <= 0) return QMOE_ERR_INVALID_ARG;
    if (e > 1024 || k > 32 || k > e) return QMOE_ERR_UNSUPPORTED;
    return hip_status(qmoe::launch_router_topk(logits, t, e, k, bias, idx, weights, as_stream(stream)));
}

int lora_apply(const uint16_t* x, int32_t t, const qmoe_lora* l, const int32_t* adapter_idx,
               float* y_acc, void* stream) {
    if (!x || !l || !y_acc || t <= 0) return QMOE_ERR_INVALID_ARG;
    if (t > 65535) return QMOE_ERR_UNSUPPORTED;
    int st = check_lora(l, l->in_dim, l->out_dim);
    if (st) return st;
    if (l->out_dim <= 0) return QMOE_ERR_INVALID_ARG;
    if (!aligned16(x)) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_lora_apply(x, t, *l, adapter_idx, y_acc, as_stream(stream)));
}

size_t moe_switchglu_int4_workspace_bytes(const qmoe_moe_layer* L, int32_t max_tokens) {
    if (max_tokens <= 0 || check_layer(L)) return 0;
    return qmoe::moe_workspace_bytes(*L, max_tokens);
}

int moe_switchglu_int4(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                       const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                       float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return moe_switchglu_int4_stage(L, QMOE_STAGE_ALL, x, t, adapter_idx, y, idx_out, w_out, ws,
                                    ws_bytes, stream);
}

int moe_switchglu_int4_stage(const qmoe_moe_layer* L, int32_t stage, const uint16_t* x,
                             int32_t t, const int32_t* adapter_idx, uint16_t* y,
                             int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                             void* stream) {
    if (stage < QMOE_STAGE_ALL || stage > QMOE_STAGE_DOWN) return QMOE_ERR_INVALID_ARG;
    if (!x || !y || t <= 0) return QMOE_ERR_INVALID_ARG;
    if (t > 65536) return QMOE_ERR_UNSUPPORTED;
    int st = check_layer(L);
    if (st) return st;
    if (!aligned16(x) || !aligned16(y)) return QMOE_ERR_MISALIGNED;
    if (!aligned4(adapter_idx) || !aligned4(idx_out) || !aligned4(w_out)) return QMOE_ERR_MISALIGNED;
    const size_t xb = (size_t)t * L->hidden * 2;
    if (overlap(x, xb, y, xb)) return QMOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < qmoe::moe_workspace_bytes(*L, t)) return QMOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_moe(*L, stage, x, t, adapter_idx, y, idx_out, w_out, ws,
                                       as_stream(stream)));
}

int moe_switchglu_int4_routed(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                              const int32_t* adapter_idx, const int32_t* route_idx, uint16_t* y,
                              float* w_out, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !route_idx || t <= 0) return QMOE_ERR_INVALID_ARG;
    if (t > 65536) return QMOE_ERR_UNSUPPORTED;
    int st = check_layer(L);
    if (st) return st;
    if (!aligned16(x) || !aligned16(y)) return QMOE_ERR_MISALIGNED;
    if (!aligned4(adapter_idx) || !aligned4(route_idx) || !aligned4(w_out)) return QMOE_ERR_MISALIGNED;
    const size_t xb = (size_t)t * L->hidden * 2;
    if (overlap(x, xb, y, xb)) return QMOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < qmoe::moe_workspace_bytes(*L, t)) return QMOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_moe(*L, QMOE_STAGE_ALL, x, t, adapter_idx, y, nullptr, w_out, ws,
                                       as_stream(stream), route_idx));
}

int moe_switchglu_int4_noalloc(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                               const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                               float* w_out, void* stream) {
    if (!x || !y || t <= 0) return QMOE_ERR_INVALID_ARG;
    if (t > 65536) return QMOE_ERR_UNSUPPORTED;
    int st = check_layer(L);
    if (st) return st;
    if (!aligned16(x) || !aligned16(y)) return QMOE_ERR_MISALIGNED;
    if (!aligned4(adapter_idx) || !aligned4(idx_out) || !aligned4(w_out)) return QMOE_ERR_MISALIGNED;
    const size_t xb = (size_t)t * L->hidden * 2;
    if (overlap(x, xb, y, xb)) return QMOE_ERR_INVALID_ARG;
    if (qmoe::moe_workspace_bytes(*L, t) > qmoe::MOE_NOALLOC_SCRATCH_BYTES) {
        g_last_error = "the layer needs more workspace for this token count than the "
                       "allocation-free call's fixed scratch holds";
        return QMOE_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    st = hip_status(qmoe::moe_noalloc_scratch(as_stream(stream), &ws));
    if (st) return st;
    return hip_status(qmoe::launch_moe(*L, QMOE_STAGE_ALL, x, t, adapter_idx, y, idx_out, w_out,
                                       ws, as_stream(stream)));
}

int qmoe_quantize_supergroup(const float* w, int32_t rows, int32_t cols, int32_t period,
                             uint32_t* p4, uint32_t* p2, uint16_t* scales, void* stream) {
    if (!w || !p4 || !scales || rows <= 0 || cols <= 0 || period <= 0) return QMOE_ERR_INVALID_ARG;
    if (period > 64 || rows % period || cols % 512) return QMOE_ERR_UNSUPPORTED;
    if (period > 1 && !p2) return QMOE_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(p4) || (p2 && !aligned16(p2))) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_quantize_supergroup(w, rows, cols, period, p4, p2, scales,
                                                       as_stream(stream)));
}

int qlinear_supergroup(const uint16_t* x, int32_t b, const uint32_t* p4, const uint32_t* p2,
                       const uint16_t* scales, int32_t rows, int32_t cols, int32_t period,
                       uint16_t* y, void* stream) {
    if (!x || !p4 || !scales || !y || b <= 0 || rows <= 0 || cols <= 0 || period <= 0)
        return QMOE_ERR_INVALID_ARG;
    if (b > 4096 || period > 64 || rows % period || cols % 512 || cols > 8192) return QMOE_ERR_UNSUPPORTED;
    if (period > 1 && !p2) return QMOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y) || !aligned16(p4) || (p2 && !aligned16(p2)))
        return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_qlinear_supergroup(x, b, p4, p2, scales, rows, cols, period, y,
                                                      as_stream(stream)));
}

int prerouter_forward(const qmoe_prerouter* P, const uint16_t* h, int32_t t, int32_t k,
                      const int32_t* topk_now, const int32_t* topk_prev, uint16_t* act,
                      float* logits, int32_t* pred_idx, float* pred_w, void* stream) {
    if (!P || !h || !topk_now || !topk_prev || !act || !logits || t <= 0 || k <= 0)
        return QMOE_ERR_INVALID_ARG;
    if (!P->w_init || !P->b_init || !P->w1 || !P->b1 || !P->w2 || !P->b2) return QMOE_ERR_INVALID_ARG;
    if (P->hidden <= 0 || P->n_experts <= 0 || P->ffn <= 0) return QMOE_ERR_INVALID_ARG;
    if ((pred_idx == nullptr) != (pred_w == nullptr)) return QMOE_ERR_INVALID_ARG;
    if (P->hidden % 512 || P->hidden > 8192 || P->ffn % 512 || P->n_experts % 4 ||
        P->n_experts > 1024 || k > 32 || k > P->n_experts || t > 4096)
        return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(act) || !aligned16(P->w_init) || !aligned16(P->w1) ||
        !aligned16(P->w2))
        return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_prerouter(*P, h, t, k, topk_now, topk_prev, act, logits,
                                             pred_idx, pred_w, as_stream(stream)));
}

int qmoe_quantize_act8(const uint16_t* x, int32_t b, int32_t cols, int8_t* qx, uint16_t* sx,
                       void* stream) {
    if (!x || !qx || !sx || b <= 0 || cols <= 0) return QMOE_ERR_INVALID_ARG;
    if (b > 65536 || cols % 512 || cols > 65536) return QMOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(qx)) return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_quantize_act8(x, b, cols, qx, sx, as_stream(stream)));
}

int qlinear_supergroup_a8(const uint16_t* x, int32_t b, const uint32_t* p4, const uint32_t* p2,
                          const uint16_t* scales, int32_t rows, int32_t cols, int32_t period,
                          uint16_t* y, void* stream) {
    if (!x || !p4 || !scales || !y || b <= 0 || rows <= 0 || cols <= 0 || period <= 0)
        return QMOE_ERR_INVALID_ARG;
    if (b > 4096 || period > 64 || rows % period || cols % 512 || cols > 8192) return QMOE_ERR_UNSUPPORTED;
    if (period > 1 && !p2) return QMOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y) || !aligned16(p4) || (p2 && !aligned16(p2)))
        return QMOE_ERR_MISALIGNED;
    return hip_status(qmoe::launch_qlinear_supergroup_a8(x, b, p4, p2, scales, rows, cols, period,
                                                         y, as_stream(stream)));
}

}  // extern "C"
