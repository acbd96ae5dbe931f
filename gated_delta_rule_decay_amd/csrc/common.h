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

// Gate value of token-head `row` at key channel c: per key channel or one
// value per token-head.
__device__ __forceinline__ float load_gate(const float *g, int per_key, int64_t row, int64_t dk,
                                           int64_t c) {
    return per_key ? g[row * dk + c] : g[row];
}

}  // namespace gdn2
