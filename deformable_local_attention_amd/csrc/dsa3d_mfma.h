// dsa3d_mfma.h -- operand types and reads of the bf16 matrix-core products
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

// A first operand read from a row-major tile in LDS with gfx950's transposing
// read (ds_read_b64_tr_b16): in each 16-lane block, lane L addresses p = row
// r0 + L/4, columns c0 + 4(L%4) .. +3, and lane j receives column c0 + j of
// rows r0 .. r0+3; the second read starts `rows2_elems` elements further on
// (a whole number of rows). The lane's eight values are column c0 + j of those
// two groups of four rows, in order. p must lie in LDS and be 8-byte aligned.
__device__ __forceinline__ mf_bf16x8 mf_read_tr8(const bf16_t* p, int rows2_elems) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    typedef s16x4 __attribute__((address_space(3))) * lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p + rows2_elems));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(mf_bf16x8, v);
}

}  // namespace dsa3d
