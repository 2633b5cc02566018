// Device-side helpers shared by the gfx950 kernels of libqmoe.
//
// Code unpacking uses exact fp16 construction: a 4-bit code q placed in the four top
// mantissa bits of 1.0 gives the fp16 value 1 + q/16 exactly (8-bit: 1 + q/256).  A dot
// product against x then yields sum(x) + sum(q x)/16, from which the affine group term
// s*sum(q x) + b*sum(x) = 16 s * dot + (b - 16 s) * sum(x) follows with fp32 arithmetic.
// Keeping the constant 1 (not 1024, as with the usual exponent trick) makes the constant
// part of the dot the same size as the code part, so fp32 accumulation loses nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default rounding mode)
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }

// bf16 bits -> fp32 (exact): the upper half of the fp32 pattern
__device__ __forceinline__ float bf2f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
// Two bf16 values (low and high half) as two fp16 values, rounded to nearest (exact for bf16
// values inside fp16's normal range, whose 8 significant bits fit fp16's 11).
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t v) {
    return (uint32_t)f2h(bf2f((uint16_t)(v & 0xFFFFu))) | ((uint32_t)f2h(bf2f((uint16_t)(v >> 16))) << 16);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// 4-bit word w holds codes q0..q7 (q_j in bits [4j, 4j+4)).  Pair j in 0..3 returns the
// fp16 pair (1 + q_j/16, 1 + q_{j+4}/16): nibble j moved to mantissa bits 6..9 of the low
// half, nibble j+4 to bits 6..9 of the high half, exponent of 1.0 ORed in.
template <int J>
__device__ __forceinline__ uint32_t nib_pair(uint32_t w) {
    uint32_t s;
    if constexpr (J == 0) s = w << 6;
    else if constexpr (J == 1) s = w << 2;
    else if constexpr (J == 2) s = w >> 2;
    else s = w >> 6;
    return (s & 0x03C003C0u) | 0x3C003C00u;
}

// 8-bit word w holds codes b0..b3 (byte j).  Pair 0 = (1 + b0/256, 1 + b2/256),
// pair 1 = (1 + b1/256, 1 + b3/256).
template <int J>
__device__ __forceinline__ uint32_t byte_pair(uint32_t w) {
    uint32_t s = (J == 0) ? (w << 2) : (w >> 6);
    return (s & 0x03FC03FCu) | 0x3C003C00u;
}

// Dot of one packed word against its x values, x given as the matching pairs.
__device__ __forceinline__ float dot_word4(uint32_t w, const f16x2* xp, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2(nib_pair<0>(w)), xp[0], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(nib_pair<1>(w)), xp[1], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(nib_pair<2>(w)), xp[2], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(nib_pair<3>(w)), xp[3], acc, false);
    return acc;
}
__device__ __forceinline__ float dot_word8(uint32_t w, const f16x2* xp, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2(byte_pair<0>(w)), xp[0], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(byte_pair<1>(w)), xp[1], acc, false);
    return acc;
}

// The code scale 16 (4-bit) or 256 (8-bit) of the 1 + q/C construction.
template <int BITS>
__device__ __forceinline__ constexpr float code_div() { return BITS == 4 ? 16.0f : 256.0f; }

// Permute 8 consecutive x values (x0..x7, one 4-bit word's worth) into the pair order of
// nib_pair: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ void pair_perm8(const f16* x, f16x2* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = f16x2{x[j], x[j + 4]};
}
// 4 consecutive x values (one 8-bit word) into (x0,x2) (x1,x3).
__device__ __forceinline__ void pair_perm4(const f16* x, f16x2* out) {
    out[0] = f16x2{x[0], x[2]};
    out[1] = f16x2{x[1], x[3]};
}

// The same permutations on whole dwords (v_perm_b32), for data fresh from a load: taking a
// loaded register apart into 16-bit halves lets the compiler schedule that split right after
// the load, and the wait for it then also waits for every load issued before.
// v = 8 halves x0..x7 as dwords (x0,x1) (x2,x3) (x4,x5) (x6,x7).
__device__ __forceinline__ uint4 pair_perm8_w(const uint4& v) {   // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
    return uint4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}
__device__ __forceinline__ uint4 pair_perm4x2_w(const uint4& v) {  // (x0,x2) (x1,x3) (x4,x6) (x5,x7)
    return uint4{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.z, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
}
// Sum of the 8 halves in fp32 by dot products against ones (no 16-bit extraction).
__device__ __forceinline__ float sum8_w(const uint4& v) {
    const f16x2 one = {(f16)1.0f, (f16)1.0f};
    float s = __builtin_amdgcn_fdot2(as_h2(v.x), one, 0.0f, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    return __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
}
// fp32 value of half j (0 = low) of a dword
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)as_h2(w)[1]; }

// ---- cross-lane sums without LDS round trips -------------------------------------------
// DPP controls (gfx9): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i <-> 7-i
// in each 8), row_mirror (i <-> 15-i in each 16).  After the first two steps the four lanes
// of a quad hold equal values, so each mirror step pairs every lane with a lane of the
// neighbouring quad / half-row: the result is the segment total in every lane, the same
// bits in every lane (fp add is commutative), and the same order on every run.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

// Sum over aligned segments of WIDTH lanes (a power of two <= 64), total in every lane.
// Segments of 32 and 64 lanes combine their 16-lane rows through scalar readlanes in a
// fixed order.
template <int WIDTH>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (WIDTH >= 2) v += dpp<DPP_XOR1>(v);
    if constexpr (WIDTH >= 4) v += dpp<DPP_XOR2>(v);
    if constexpr (WIDTH >= 8) v += dpp<DPP_HALF_MIRROR>(v);
    if constexpr (WIDTH >= 16) v += dpp<DPP_MIRROR>(v);
    if constexpr (WIDTH >= 32) {
        const int bits = __builtin_bit_cast(int, v);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 48));
        if constexpr (WIDTH == 32) v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
        else v = (r0 + r1) + (r2 + r3);
    }
    return v;
}

// Adapter of token t: adapter_idx[t] clamped into [0, n) (0 when no index array), so an
// out-of-range index can never address memory outside the adapter stack.
__device__ __forceinline__ int adapter_of(const int32_t* adapter_idx, int t, int n) {
    if (!adapter_idx) return 0;
    const int a = adapter_idx[t];
    return a < 0 ? 0 : (a >= n ? n - 1 : a);
}

// Pins the first use of a loaded value to this point.  The compiler may otherwise schedule
// work on a loaded register (splitting it into halves, converting it) right after the load,
// and the wait for that load then also waits for every load issued before it, since memory
// waits count in issue order.  After hold(), every read of `v` is of the asm's output, so the
// wait lands here.
__device__ __forceinline__ void hold(uint4& v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace qmoe
