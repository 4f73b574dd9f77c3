// dsa3d_mfma.h -- operand types of the bf16 matrix-core products
// (v_mfma_f32_16x16x32_bf16) shared by the fixed-window and the hybrid
// kernels (internal; gfx950 only).
//
// Layout of one 16x16x32 product D = A B + C, per lane l of the wave: A row
// l%16 with k-slice 8*(l/16) .. +7, B column l%16 with the same k-slice (eight
// bf16 each), and D[4*(l/16) + r][l%16] in accumulator element r.
#pragma once

#include "dsa3d_device.h"

namespace dsa3d {

typedef __attribute__((ext_vector_type(8))) __bf16 mf_bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 mf_bf16x2;
typedef __attribute__((ext_vector_type(4))) float mf_f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t mf_u32x4;

// Online softmax on the matrix cores: the running maximum is raised only when
// a logit exceeds it by more than this, so most key tiles skip the rescale of
// the accumulators; the weights then stay below e^8.
constexpr float kMfmaLazyMax = 8.0f;

__device__ __forceinline__ uint32_t mf_pack(float lo, float hi) {  // two RNE bf16 in one word
    const mf_bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Weights w0, w1 as a bf16 part and the bf16 rounding of the remainder, each
// pair in one word: w = hi + lo to about 2^-17 relative, so a product with
// the two parts carries the weights at nearly float32 precision.
// Returns (part, remainder).
__device__ __forceinline__ uint2 mf_split(float w0, float w1) {
    const uint32_t hi = mf_pack(w0, w1);
    return make_uint2(hi, mf_pack(w0 - bf16_lo(hi), w1 - bf16_hi(hi)));
}

}  // namespace dsa3d
