// Internal launchers (host side) of libqmoe's kernels.  Arguments are validated by the
// C-ABI layer (capi.cpp) before any of these is called; each returns hipGetLastError()
// after enqueueing on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

// quant.hip
hipError_t launch_quantize_affine(const float* w, int rows, int cols, int bits, int group,
                                  uint32_t* packed, uint16_t* scales, uint16_t* biases,
                                  hipStream_t s);
hipError_t launch_unpack(const uint32_t* packed, long n_words, int bits, uint8_t* q,
                         hipStream_t s);
hipError_t launch_dequantize(const qmoe_qweight& w, float* out, hipStream_t s);
hipError_t launch_quantize_supergroup(const float* w, int rows, int cols, int period,
                                      uint32_t* p4, uint32_t* p2, uint16_t* scales,
                                      hipStream_t s);

// gemv.hip: y = fp16(x W^T + lora) for a small number of tokens, fp32 accumulation
hipError_t launch_qlinear_gemv(const uint16_t* x, int m, const qmoe_qweight& w,
                               const qmoe_lora* lora, const int32_t* adapter_idx,
                               uint16_t* y, hipStream_t s);

// router.hip
hipError_t launch_router_topk(const float* logits, int t, int e, int k, const float* bias,
                              int32_t* idx, float* weights, hipStream_t s);

// lora.hip
hipError_t launch_lora_apply(const uint16_t* x, int t, const qmoe_lora& l,
                             const int32_t* adapter_idx, float* y_acc, hipStream_t s);

// moe.hip
size_t moe_workspace_bytes(const qmoe_moe_layer& L, int max_tokens);
// the allocation-free call's workspace: a static device array of this size per device, its
// device address looked up on the first call on the stream's device
constexpr size_t MOE_NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
hipError_t moe_noalloc_scratch(hipStream_t s, void** ptr);
// route: a given selection [t][top_k] (the caller's routing) in place of the top-K, or null
hipError_t launch_moe(const qmoe_moe_layer& L, int stage, const uint16_t* x, int t,
                      const int32_t* adapter_idx, uint16_t* y, int32_t* idx_out,
                      float* w_out, void* ws, hipStream_t s, const int32_t* route = nullptr);

// supergroup.hip
hipError_t launch_qlinear_supergroup(const uint16_t* x, int b, const uint32_t* p4,
                                     const uint32_t* p2, const uint16_t* scales, int rows,
                                     int cols, int period, uint16_t* y, hipStream_t s);

// prerouter.hip
hipError_t launch_prerouter(const qmoe_prerouter& P, const uint16_t* h, int t, int k,
                            const int32_t* now, const int32_t* prev, uint16_t* act,
                            float* logits, int32_t* pred_idx, float* pred_w, hipStream_t s);

// supergroup_a8.hip
hipError_t launch_quantize_act8(const uint16_t* x, int b, int cols, int8_t* qx, uint16_t* sx,
                                hipStream_t s);
hipError_t launch_qlinear_supergroup_a8(const uint16_t* x, int b, const uint32_t* p4,
                                        const uint32_t* p2, const uint16_t* scales, int rows,
                                        int cols, int period, uint16_t* y, hipStream_t s);

}  // namespace qmoe
