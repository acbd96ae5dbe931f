// common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Element i of a q/k/v tensor that is either bf16 or fp32.
__device__ __forceinline__ float load_qkv(const void *p, int64_t i, int bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p)[i])
                : static_cast<const float *>(p)[i];
}

// fp32 -> bf16 bits, rounded to nearest even (the carry of the dropped half
// into the kept one); a NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Output element i of o: fp32, or bf16 when o_bf16 (o then points at bf16).
__device__ __forceinline__ void store_out(float *o, int64_t i, float x, int o_bf16) {
    if (o_bf16)
        reinterpret_cast<uint16_t *>(o)[i] = f32_to_bf16(x);
    else
        o[i] = x;
}

// Output elements i .. i+3 (i a multiple of 4): one 16-byte or 8-byte store.
__device__ __forceinline__ void store_out4(float *o, int64_t i, float x0, float x1, float x2, float x3,
                                           int o_bf16) {
    if (o_bf16) {
        const uint2 w = {f32_to_bf16(x0) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16),
                         f32_to_bf16(x2) | (static_cast<uint32_t>(f32_to_bf16(x3)) << 16)};
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(o) + i) = w;
    } else {
        *reinterpret_cast<float4 *>(o + i) = make_float4(x0, x1, x2, x3);
    }
}

// Gate value of token-head `row` at key channel c: per key channel or one
// value per token-head.
__device__ __forceinline__ float load_gate(const float *g, int per_key, int64_t row, int64_t dk,
                                           int64_t c) {
    return per_key ? g[row * dk + c] : g[row];
}

// Gate activations of the fused input preparation: log a = -softplus(x)
// (so a = exp(log a) in (0, 1)) and sigmoid(x) for the erase / write gates,
// on the hardware exp2 / log2 / reciprocal (about 1 ulp each):
//   -softplus(x) = -(max(x, 0) + ln 2 * log2(1 + 2^(-|x| log2 e))),
// where the log2 argument lies in (1, 2] (no denormal or range handling is
// needed; for large |x| it rounds to 1 and the result is max(x, 0) within
// 2^-24), and sigmoid(x) = 1 / (1 + 2^(-x log2 e)), which is 0 or 1 where
// the power overflows or vanishes.
__device__ __forceinline__ float neg_softplus(float x) {
    const float t = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return -(fmaxf(x, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.f + t));
}
__device__ __forceinline__ float sigmoid_gate(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Gate value of token-head `row` at channel c: the fp32 value as stored, or,
// with `logits`, the activation of the bf16 logit there (act 0: decay,
// -softplus; act 1: sigmoid).
__device__ __forceinline__ float load_gate_x(const float *g, int per_key, int64_t row, int64_t width,
                                             int64_t c, int logits, int act) {
    if (!logits) return load_gate(g, per_key, row, width, c);
    const uint16_t *p = reinterpret_cast<const uint16_t *>(g);
    const float x = bf16_to_f32(per_key ? p[row * width + c] : p[row]);
    return act == 0 ? neg_softplus(x) : sigmoid_gate(x);
}

}  // namespace gdn2
