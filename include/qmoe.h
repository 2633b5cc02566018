/*
 * qmoe.h — C ABI of libqmoe: group-wise affine int4 quantized matmul inside a MoE
 * SwitchGLU expert layer with a shared expert and unmerged LoRA deltas, for AMD MI355X
 * (gfx950).
 *
 * Sources of the operations (web pages; cited by title and section):
 *  [R1] "Recover-LoRA: how Edge0 recovers the precision lost to 4-bit compression"
 *       (bjdmk.com.cn), section 1: 4-bit affine quantization with group_size 64, each
 *       linear layer stored as `weight` (packed integers), `scales` and `biases`; router
 *       gate and shared-expert gate kept at 8-bit; K = 4 experts per token of 256.
 *       Section 2: frozen int4 base plus an unmerged LoRA delta; one read-only base serves
 *       many adapter sets.
 *  [R2] "Edge0-35B-A3B Preview model repository guide" (trdm.cn), "model spec" table:
 *       hidden 2048, 256 experts, expert and shared-expert intermediate 512, 40 layers,
 *       experts stored as switch_mlp.gate_proj/up_proj/down_proj with scales and biases.
 *  [R3] "Bit-exact MLX 4-bit port of d1a-e2b-it-qat-4bit" (gtnt.cn), "4-bit group
 *       quantization" and "how 0.0 dequantization error is achieved": integers kept as
 *       packed words with one scale and one bias per group; dequantized weight = scale
 *       times integer plus bias.
 *  [R4] "Edge0 project review" (blog.kxstl.cn), highlight 2: routing indices never leave
 *       the device (no host sync per layer and step); a missing expert contributes
 *       nothing; the expert combine is _swiglu(up, gate).  Highlight 3: LoRA as a
 *       parallel delta, never merged; --no-lora runs the plain base.  MoE spec: routing
 *       family SOFTMAX_TOPK.
 *  [R5] "EDGERAZOR deep dive" (zhichai.net), section 2.1 SQMP: super-group allocation
 *       (one 4-bit channel in every floor(1/rho) consecutive output channels, the rest
 *       ternary), the ternary and 4-bit symmetric quantizers, and the factorisation of the
 *       matmul into a scale product times an integer dot product; section 3.1, the
 *       weight-activation results with 8-bit activations.
 *
 * Conventions for every entry point
 *  - Array pointers are DEVICE pointers unless stated otherwise; `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream).  Struct arguments
 *    (qmoe_qweight, qmoe_lora, qmoe_moe_layer) are HOST pointers to host structs whose
 *    array members are device pointers.
 *  - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *  - The caller owns every buffer, workspaces included.  The library allocates and frees
 *    no device memory, keeps no state between calls (apart from the fixed per-device
 *    scratch of moe_switchglu_int4_noalloc), never copies to the host and never
 *    synchronises: work is enqueued on `stream` and the call returns.
 *  - Errors: 0 on success, a negative QMOE_ERR_* code otherwise.  Arguments are validated
 *    before anything is enqueued; on error nothing is enqueued and outputs are untouched.
 *    Faults inside kernels surface asynchronously at the caller's next synchronisation.
 *    NaN/Inf inputs give undefined (but memory-safe) results.
 *  - Determinism: no atomics on any reduction path; identical inputs give bit-identical
 *    outputs on the same device.
 *  - Alignment (QMOE_ERR_MISALIGNED otherwise): the packed words, scales and biases of
 *    every quantized matrix handed to a GEMV/GEMM entry point, LoRA A and B, activations
 *    and fp16 outputs must be 16-byte aligned; the MoE workspace 256-byte aligned; int32 and
 *    fp32 index, weight and bias arrays 4-byte aligned.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 1

#define QMOE_OK 0
#define QMOE_ERR_INVALID_ARG (-1) /* NULL pointer, non-positive or inconsistent size   */
#define QMOE_ERR_UNSUPPORTED (-2) /* bits/group/shape outside what the kernels support */
#define QMOE_ERR_MISALIGNED (-3)  /* a pointer is not aligned as required below       */
#define QMOE_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than required           */
#define QMOE_ERR_HIP (-5)         /* a kernel launch failed                            */

/*
 * One group-wise affine quantized matrix W [rows x cols] (output x input), or a stack of
 * `n_experts` such matrices stored back to back ([R1] section 1, [R3]).
 *
 *   packed  uint32 [n_experts][rows][cols*bits/32]; element 8m+j of a row (bits = 4) is
 *           bits [4j, 4j+4) of word m, lowest nibble first; for bits = 8 element 4m+j is
 *           byte j of word m.
 *   scales  fp16 or bf16 [n_experts][rows][cols/group] (param_dtype)
 *   biases  fp16 or bf16 [n_experts][rows][cols/group]
 *   W[n][k] = scale[n][k/group] * q[n][k] + bias[n][k/group].
 *
 * Supported: bits in {4, 8}; cols a multiple of 512; rows >= 1; group 64 with fp16
 * parameters everywhere.  qlinear_int4 and qmoe_dequantize also take group 32 and bf16
 * parameters (QMOE_PARAM_BF16), the format of the bit-exact port page's QAT checkpoint
 * ([R3] "4-bit group quantization": 32 weights per group, scale and bias in bf16), whose
 * packed words and parameters are used as given, without requantization.  The MoE layer
 * takes them for its routed expert stacks (exp_gate, exp_up, exp_down: one format for all
 * three, hidden and inter each 512, 1024 or 2048; such a layer runs the token-sorted path at
 * every token count); its router, shared gate and shared expert are group 64, fp16.  bf16
 * parameters are converted to fp16 before use, which is exact inside fp16's normal range.
 * param_dtype 0 (the zero-initialised default) is fp16.
 */
#define QMOE_PARAM_F16 0
#define QMOE_PARAM_BF16 1
typedef struct qmoe_qweight {
    const uint32_t* packed;
    const uint16_t* scales;
    const uint16_t* biases;
    int32_t rows;
    int32_t cols;
    int32_t bits;
    int32_t group;
    int32_t n_experts;   /* 1 for a single matrix */
    int32_t param_dtype; /* QMOE_PARAM_F16 or QMOE_PARAM_BF16 */
} qmoe_qweight;

/*
 * Unmerged LoRA adapter set(s) on one projection ([R1] section 2, [R4] highlight 3):
 * delta[t] = scale * B[a] (A[a] v[t]) with a = adapter_idx[t] (0 when adapter_idx is NULL).
 *
 *   A  fp16 [n_adapters][rank][in_dim]
 *   B  fp16 [n_adapters][out_dim][rank]
 *   scale = alpha / rank.   Supported: 1 <= rank <= 64, in_dim a multiple of 512.
 */
typedef struct qmoe_lora {
    const uint16_t* A;
    const uint16_t* B;
    int32_t rank;
    int32_t n_adapters;
    int32_t in_dim;
    int32_t out_dim;
    float scale;
} qmoe_lora;

/*
 * One MoE SwitchGLU layer ([R1], [R2], [R4]).  For each token x (hidden):
 *   logits = x Wr^T (+ router_bias); S = the top_k largest logits (an exact tie goes to the
 *   lower expert index); w_k = softmax over S; for each e in S:
 *   o_e = down_e( silu(gate_e x) * up_e x );
 *   shared = sh_down( silu(sh_gate x + dG) * (sh_up x + dU) ) + dD, the d's being the LoRA
 *   deltas of each projection on that projection's input;
 *   gamma = sigmoid(x w_sg^T);
 *   y = fp16( sum_k w_k o_k + gamma * shared ), and with add_residual != 0
 *   y = fp16( x + that fp16 value ).
 *
 * Shapes: router [n_experts x hidden] 8-bit; shared_gate [1 x hidden] 8-bit;
 * exp_gate/exp_up stacks of n_experts [inter x hidden]; exp_down stack [hidden x inter];
 * sh_gate/sh_up [shared_inter x hidden]; sh_down [hidden x shared_inter]; all int4
 * group 64.  The lora_* pointers may be NULL (no adapter on that projection; all NULL is
 * the plain base).  router_bias is a device fp32 [n_experts] array or NULL.
 */
typedef struct qmoe_moe_layer {
    int32_t hidden;
    int32_t inter;
    int32_t shared_inter;
    int32_t n_experts;
    int32_t top_k;
    int32_t add_residual;
    qmoe_qweight router;
    qmoe_qweight shared_gate;
    qmoe_qweight exp_gate;
    qmoe_qweight exp_up;
    qmoe_qweight exp_down;
    qmoe_qweight sh_gate;
    qmoe_qweight sh_up;
    qmoe_qweight sh_down;
    const qmoe_lora* lora_gate;
    const qmoe_lora* lora_up;
    const qmoe_lora* lora_down;
    const float* router_bias;
} qmoe_moe_layer;

/* ABI version (QMOE_ABI_VERSION) and a static string for a status code. */
int qmoe_abi_version(void);
const char* qmoe_status_string(int status);

/* sizeof of the ABI structs as compiled into the library, for bindings to check their
 * own layout: which = 0 qmoe_qweight, 1 qmoe_lora, 2 qmoe_moe_layer, 3 qmoe_prerouter;
 * 0 otherwise. */
size_t qmoe_abi_struct_size(int which);

/* Text of the HIP error behind the calling thread's most recent QMOE_ERR_HIP ("" if none).
 * The string is static or thread-local; it stays valid until the thread's next call. */
const char* qmoe_last_error(void);

/*
 * Min-max affine quantization of an fp32 matrix w [rows x cols] ([R1] section 1, [R3]).
 * Per row and group of `group` inputs: scale = fp16((max - min) / (2^bits - 1)) and
 * bias = fp16(min), both from float32 arithmetic; q = clip(rint((w - bias) / scale), 0,
 * 2^bits - 1) in float32 on the stored fp16 scale and bias (q = 0 where scale == 0).
 * Outputs packed [rows][cols*bits/32], scales and biases [rows][cols/group] in the layout
 * of qmoe_qweight (fp16 parameters).  bits in {4, 8}; group 64 or 32; cols % 64 == 0.
 */
int qmoe_quantize_affine(const float* w, int32_t rows, int32_t cols, int32_t bits,
                         int32_t group, uint32_t* packed, uint16_t* scales,
                         uint16_t* biases, void* stream);

/* Unpack words into one byte per code: q uint8 [rows][cols] ([R3] packed words). */
int qmoe_unpack(const uint32_t* packed, int32_t rows, int32_t cols, int32_t bits, uint8_t* q,
                void* stream);

/* Dequantize every matrix of w into fp32: out [n_experts][rows][cols] =
 * fp32(scale * q + bias), one rounding of the exact value ([R3]). */
int qmoe_dequantize(const qmoe_qweight* w, float* out, void* stream);

/*
 * Quantized linear y [m x rows] = fp16( x W^T + delta ), x fp16 [m x cols], with the
 * optional LoRA delta on x (lora may be NULL; adapter_idx is a device int32 [m] array or
 * NULL for adapter 0).  w->n_experts must be 1.  Accumulation in fp32.  1 <= m <= 4096.
 */
int qlinear_int4(const uint16_t* x, int32_t m, const qmoe_qweight* w, const qmoe_lora* lora,
                 const int32_t* adapter_idx, uint16_t* y, void* stream);

/*
 * Top-K routing on given fp32 logits [t x e] ([R4] SOFTMAX_TOPK; [R1] K = 4 of 256):
 * idx int32 [t x k] = the k largest of (logits + bias), in decreasing order, an exact tie
 * going to the lower expert index; weights fp32 [t x k] = exp(l_i - l_max) / sum over the
 * selected (the softmax renormalized over the selection).  bias: device fp32 [e] or NULL.
 * 1 <= k <= min(e, 32); 1 <= e <= 1024.
 */
int router_topk(const float* logits, int32_t t, int32_t e, int32_t k, const float* bias,
                int32_t* idx, float* weights, void* stream);

/*
 * LoRA delta accumulated in place ([R1] section 2, [R4] highlight 3):
 * y_acc[t][n] += scale * sum_r B[a_t][n][r] * sum_k A[a_t][r][k] * x[t][k],
 * x fp16 [t x in_dim], y_acc fp32 [t x out_dim], a_t = adapter_idx[t] (device int32 [t],
 * or NULL for adapter 0; values must lie in [0, n_adapters)).
 */
int lora_apply(const uint16_t* x, int32_t t, const qmoe_lora* l, const int32_t* adapter_idx,
               float* y_acc, void* stream);

/* Workspace bytes moe_switchglu_int4 needs for up to max_tokens tokens (0 on bad args). */
size_t moe_switchglu_int4_workspace_bytes(const qmoe_moe_layer* L, int32_t max_tokens);

/*
 * One MoE SwitchGLU layer forward for t tokens (see qmoe_moe_layer).  x fp16 [t x hidden],
 * y fp16 [t x hidden] (must not overlap x).  adapter_idx: device int32 [t] or NULL.
 * idx_out (int32 [t x top_k]) and w_out (fp32 [t x top_k]) are optional device outputs of
 * the routing decision.  ws: device workspace of at least
 * moe_switchglu_int4_workspace_bytes(L, t) bytes, 256-byte aligned.  Routing stays on the
 * device ([R4] highlight 2).  Supported: hidden and inter multiples of 512, top_k <= 32,
 * n_experts <= 1024, 1 <= t <= 65536.
 */
int moe_switchglu_int4(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                       const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                       float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The same layer as moe_switchglu_int4, one stage at a time, on the same workspace:
 *   QMOE_STAGE_ROUTE   (1): router and shared-gate logits, the shared expert's raw gate/up
 *                           projections, LoRA down-projections of x, top-K + softmax and the
 *                           sort of (token, k) pairs by expert (writes idx_out / w_out);
 *                           above 32 tokens also the shared expert's h (below);
 *   QMOE_STAGE_GATE_UP (2): h = silu(gate x) * (up x) for every routed pair; up to 32 tokens
 *                           also for the shared expert (LoRA up-projections added);
 *   QMOE_STAGE_DOWN    (3): down projections, LoRA down delta, routing-weighted combine and
 *                           the gated shared expert, y written.
 * Stage s reads what stages < s left in `ws` for the same x, t and adapter_idx; running the
 * three in order is exactly moe_switchglu_int4, and re-running one stage alone repeats its
 * work on the same inputs (how a single stage is timed).  QMOE_STAGE_ALL (0) runs all.
 */
#define QMOE_STAGE_ALL 0
#define QMOE_STAGE_ROUTE 1
#define QMOE_STAGE_GATE_UP 2
#define QMOE_STAGE_DOWN 3
int moe_switchglu_int4_stage(const qmoe_moe_layer* L, int32_t stage, const uint16_t* x,
                             int32_t t, const int32_t* adapter_idx, uint16_t* y,
                             int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * The same layer under a routing given by the caller instead of the router's top-K: token
 * t runs experts route_idx[t][0 .. top_k-1] (device int32 [t x top_k]).  This is the
 * prerouter's use ("Edge0 project review", highlight 1): the head of layer N predicts, at
 * token t-1, the experts of layer N+1 for token t, and that prediction is the route itself
 * (the staged experts are exactly the predicted set), so the expert loads need not wait for
 * the router.  The router still runs: the routing weights are the softmax of its logits
 * (+ router_bias) over the given set, w_k = exp(l_k - m) / sum_j exp(l_j - m), written to
 * w_out (fp32 [t x top_k]) when it is not NULL.  Entries outside [0, n_experts) are clamped
 * into it; an expert given twice counts twice.  Workspace, limits and the rest of the
 * output as moe_switchglu_int4.  Up to 32 (token, expert) pairs this is two launches.
 */
int moe_switchglu_int4_routed(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                              const int32_t* adapter_idx, const int32_t* route_idx, uint16_t* y,
                              float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_switchglu_int4 with its workspace in
 * a fixed scratch array inside the library instead of a caller buffer.  Same arguments,
 * outputs, limits and results as moe_switchglu_int4 without ws / ws_bytes.  The scratch
 * holds QMOE_NOALLOC_SCRATCH_BYTES per device and is kept from the first call on a device
 * until the process ends; a call whose workspace (moe_switchglu_int4_workspace_bytes of the
 * layer at t tokens) exceeds it fails with QMOE_ERR_WORKSPACE before anything is enqueued
 * (hidden 2048, 256 experts, top-4: up to 609 tokens).  The call allocates and frees
 * nothing.  All calls on one device share that device's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap in time on one
 * device (two streams, two host threads) race, and the caller must serialise them.
 */
#define QMOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moe_switchglu_int4_noalloc(const qmoe_moe_layer* L, const uint16_t* x, int32_t t,
                               const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                               float* w_out, void* stream);

/*
 * Mixed ternary / 4-bit super-group quantization of fp32 w [rows x cols] ([R5] 2.1).
 * Channel n is 4-bit symmetric when n % period == 0: s = fp16(max(max|w| / 7, 1e-5)),
 * q = clip(rint(w / s), -7, 7); otherwise ternary: s = fp16(max(2 * mean|w|, 1e-5)) (mean
 * summed in fp64, rounded to fp32), q = clip(rint(w / s), -1, 1); codes against the
 * stored fp16 scale, in fp32.  Outputs: p4 uint32 [rows/period][cols/8] (nibble q + 8,
 * lowest first), p2 uint32 [rows - rows/period][cols/16] (2-bit field q + 1, lowest
 * first), both in channel order; scales fp16 [rows].  rows % period == 0,
 * cols % 512 == 0, 1 <= period <= 64.
 */
int qmoe_quantize_supergroup(const float* w, int32_t rows, int32_t cols, int32_t period,
                             uint32_t* p4, uint32_t* p2, uint16_t* scales, void* stream);

/*
 * Super-group weight-only GEMM ([R5] 2.1, the scale/integer factorisation with s_X = 1):
 * y [b x rows] = fp16( s_n * sum_k q[n][k] * x[b][k] ), x fp16 [b x cols], fp32
 * accumulation.  Same layout and limits as qmoe_quantize_supergroup; 1 <= b <= 4096.
 */
int qlinear_supergroup(const uint16_t* x, int32_t b, const uint32_t* p4, const uint32_t* p2,
                       const uint16_t* scales, int32_t rows, int32_t cols, int32_t period,
                       uint16_t* y, void* stream);

/*
 * 8-bit activation quantization of the weight-activation integer path ([R5] 2.1, the
 * matmul as (s_W s_X) Q(W)^T Q(X); [R5] 3.1 runs activations at 8 bits): per token b,
 * s_X[b] = fp16(max(max_k |x[b][k]| / 127, 1e-5)) and qx[b][k] = clip(rint(x[b][k] /
 * s_X[b]), -127, 127), the division in fp32 against the stored fp16 scale, ties to even.
 * x fp16 [b x cols] (16-byte aligned), qx int8 [b x cols] (16-byte aligned), sx fp16 [b];
 * cols % 512 == 0, cols <= 65536, 1 <= b <= 65536.  Deterministic.
 */
int qmoe_quantize_act8(const uint16_t* x, int32_t b, int32_t cols, int8_t* qx, uint16_t* sx,
                       void* stream);

/*
 * Super-group GEMM on the weight-activation integer path ([R5] 2.1): the activations are
 * quantized as by qmoe_quantize_act8 inside the call, the sum over the inputs is an exact
 * integer dot product of the weight codes and the activation codes, and the scale product
 * is applied once: y[b][n] = fp16((sum_k q_W[n][k] q_X[b][k]) * s_X[b] * s_W[n]) (the two
 * multiplications in fp32).  Same weight layout and limits as qlinear_supergroup.
 */
int qlinear_supergroup_a8(const uint16_t* x, int32_t b, const uint32_t* p4, const uint32_t* p2,
                          const uint16_t* scales, int32_t rows, int32_t cols, int32_t period,
                          uint16_t* y, void* stream);

/*
 * Prerouter head of one layer ("Edge0 project review", highlight 1): f = [h (hidden),
 * one-hot of the token's executed top-k (n_experts), one-hot of the previous token's top-k
 * (n_experts)]; logits = linear_init(f) + fc2(gelu_erf(fc1(f))), every layer's output
 * rounded to fp16 (fp32 accumulation).  Weights fp16, row-major [out][in], with biases:
 *   w_init [n_experts][hidden + 2 n_experts], b_init [n_experts]
 *   w1     [ffn][hidden + 2 n_experts],       b1 [ffn]
 *   w2     [n_experts][ffn],                  b2 [n_experts]
 */
typedef struct qmoe_prerouter {
    const uint16_t* w_init;
    const uint16_t* b_init;
    const uint16_t* w1;
    const uint16_t* b1;
    const uint16_t* w2;
    const uint16_t* b2;
    int32_t hidden;
    int32_t n_experts;
    int32_t ffn;
} qmoe_prerouter;

/*
 * The head's forward for t tokens: h fp16 [t][hidden]; topk_now and topk_prev int32 [t][k]
 * (the executed routing of each token and of its previous token; indices outside
 * [0, n_experts) are clamped).  Outputs: act fp16 [t][ffn] = fp16(gelu_erf(fp16(fc1 f)))
 * and logits fp32 [t][n_experts] holding the fp16-rounded head logits; when pred_idx is
 * not NULL, also the predicted routing of the next layer: the top-k of the logits with
 * router_topk's rule (lower index on ties) into pred_idx int32 [t][k] and pred_w fp32
 * [t][k] (softmax over the k).  Supported: hidden % 512 == 0, hidden <= 8192,
 * ffn % 512 == 0, n_experts % 4 == 0, n_experts <= 1024, 1 <= k <= 32, k <= n_experts,
 * 1 <= t <= 4096; h, act and every weight 16-byte aligned.
 */
int prerouter_forward(const qmoe_prerouter* P, const uint16_t* h, int32_t t, int32_t k,
                      const int32_t* topk_now, const int32_t* topk_prev, uint16_t* act,
                      float* logits, int32_t* pred_idx, float* pred_w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
