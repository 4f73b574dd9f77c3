// dsa3d_device.h -- device helpers of libdsa3d (internal; gfx950 only).
//
// Element storage: float32 as `float`, bfloat16 as raw `uint16_t` bits.
// Widening bf16 -> f32 is exact (a shift); narrowing rounds to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa3d {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even, by gfx950's packed conversion (v_cvt_pk_bf16_f32);
// checked bit for bit against the integer rounding x + 0x7fff + lsb on ties,
// denormals, infinities and overflow (NaN stays NaN; its payload may differ).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// v_dot2_f32_bf16: c + a.lo*b.lo + a.hi*b.hi (products of bf16 are exact in f32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Eight consecutive elements of a row, the unit one lane owns.
template <typename T> struct Frag8;
template <> struct Frag8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<float4*>(p) = a;
        *reinterpret_cast<float4*>(p + 4) = b;
    }
    __device__ __forceinline__ void to_f32(float x[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    __device__ __forceinline__ void from_f32(const float x[8]) {
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(x[4], x[5], x[6], x[7]);
    }
    // partial dot product with another fragment
    __device__ __forceinline__ float dot(const Frag8& o, float c) const {
        c = fmaf(a.x, o.a.x, c); c = fmaf(a.y, o.a.y, c); c = fmaf(a.z, o.a.z, c); c = fmaf(a.w, o.a.w, c);
        c = fmaf(b.x, o.b.x, c); c = fmaf(b.y, o.b.y, c); c = fmaf(b.z, o.b.z, c); c = fmaf(b.w, o.b.w, c);
        return c;
    }
    // x[i] += s * this[i]
    __device__ __forceinline__ void axpy(float s, float x[8]) const {
        x[0] = fmaf(s, a.x, x[0]); x[1] = fmaf(s, a.y, x[1]); x[2] = fmaf(s, a.z, x[2]); x[3] = fmaf(s, a.w, x[3]);
        x[4] = fmaf(s, b.x, x[4]); x[5] = fmaf(s, b.y, x[5]); x[6] = fmaf(s, b.z, x[6]); x[7] = fmaf(s, b.w, x[7]);
    }
};
template <> struct Frag8<bf16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const bf16_t* p) { a = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = a; }
    __device__ __forceinline__ void to_f32(float x[8]) const {
        x[0] = bf16_lo(a.x); x[1] = bf16_hi(a.x); x[2] = bf16_lo(a.y); x[3] = bf16_hi(a.y);
        x[4] = bf16_lo(a.z); x[5] = bf16_hi(a.z); x[6] = bf16_lo(a.w); x[7] = bf16_hi(a.w);
    }
    __device__ __forceinline__ void from_f32(const float x[8]) {
        a = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7]));
    }
    __device__ __forceinline__ float dot(const Frag8& o, float c) const {
        c = dot2_bf16(a.x, o.a.x, c); c = dot2_bf16(a.y, o.a.y, c);
        c = dot2_bf16(a.z, o.a.z, c); c = dot2_bf16(a.w, o.a.w, c);
        return c;
    }
    __device__ __forceinline__ void axpy(float s, float x[8]) const {
        x[0] = fmaf(s, bf16_lo(a.x), x[0]); x[1] = fmaf(s, bf16_hi(a.x), x[1]);
        x[2] = fmaf(s, bf16_lo(a.y), x[2]); x[3] = fmaf(s, bf16_hi(a.y), x[3]);
        x[4] = fmaf(s, bf16_lo(a.z), x[4]); x[5] = fmaf(s, bf16_hi(a.z), x[5]);
        x[6] = fmaf(s, bf16_lo(a.w), x[6]); x[7] = fmaf(s, bf16_hi(a.w), x[7]);
    }
};

template <typename T> __device__ __forceinline__ float load_scalar(const T* p);
template <> __device__ __forceinline__ float load_scalar<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_scalar<bf16_t>(const bf16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);
}
template <typename T> __device__ __forceinline__ void store_scalar(T* p, float x);
template <> __device__ __forceinline__ void store_scalar<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_scalar<bf16_t>(bf16_t* p, float x) {
    *p = (bf16_t)f32_to_bf16_bits(x);
}

// Sum over the aligned group of L lanes that owns one (query, head); every
// lane of the group receives the total. Within a 16-lane DPP row the steps are
// DPP moves that read lanes of the same group only: swap neighbours (quad
// permutation 1,0,3,2), swap pairs (2,3,0,1), mirror each half row (lane i <->
// 7-i) and mirror the row (i <-> 15-i); after the first k steps every lane
// holds the sum of its aligned 2^k lanes. Wider groups finish with shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (L >= 2) x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
    if constexpr (L >= 16) x = dpp_add<0x140>(x); // row_mirror
#pragma unroll
    for (int m = 16; m < L; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Workgroups are dealt to the 8 XCDs round-robin (block i -> XCD i % 8). This
// maps the hardware block id to a logical one so that each XCD walks one
// contiguous range of logical blocks; neighbouring queries then share that
// XCD's L2 for their overlapping key/value neighbourhoods.
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t bid, uint32_t nblocks) {
    const uint32_t q8 = nblocks / 8u, r8 = nblocks % 8u;
    const uint32_t x = bid % 8u, j = bid / 8u;
    return x * q8 + (x < r8 ? x : r8) + j;
}

// Geometry of one window point of one query, in the operator's arithmetic:
// ref = x + dil*(i - (k-1)/2) in integers, pos = (float)ref + offset as one
// rounded float32 add, x0 = floorf(pos), f = pos - x0 (float32). Returns false
// when the sample lies entirely outside (NaN, infinite or |pos| >= 2^30).
struct Window {
    int32_t kt, kh, kw, khw;
    int32_t dil_t, dil_h, dil_w;
    int32_t rt, rh, rw;  // (k-1)/2
};

// The cell of a sample whose reference point (integers, converted exactly to
// float32) is (rt, rh, rw) and whose offset is (dt, dh, dw).
__device__ __forceinline__ bool sample_cell(float rt, float rh, float rw, float dt, float dh, float dw, int32_t& t0,
                                            int32_t& h0, int32_t& w0, float& ft, float& fh, float& fw) {
    const float pt = __fadd_rn(rt, dt);
    const float ph = __fadd_rn(rh, dh);
    const float pw = __fadd_rn(rw, dw);
    const float lim = 1073741824.0f;  // 2^30
    if (!(fabsf(pt) < lim) || !(fabsf(ph) < lim) || !(fabsf(pw) < lim)) return false;
    const float xt = floorf(pt), xh = floorf(ph), xw = floorf(pw);
    ft = __fsub_rn(pt, xt);
    fh = __fsub_rn(ph, xh);
    fw = __fsub_rn(pw, xw);
    t0 = (int32_t)xt;
    h0 = (int32_t)xh;
    w0 = (int32_t)xw;
    return true;
}

// Same, from the window point number p (row-major over the window).
__device__ __forceinline__ bool sample_geometry(const Window& win, int32_t t, int32_t h, int32_t w, int32_t p,
                                                float dt, float dh, float dw, int32_t& t0, int32_t& h0,
                                                int32_t& w0, float& ft, float& fh, float& fw) {
    const int32_t it = p / win.khw;
    const int32_t rem = p - it * win.khw;
    const int32_t ih = rem / win.kw;
    const int32_t iw = rem - ih * win.kw;
    return sample_cell((float)(t + win.dil_t * (it - win.rt)), (float)(h + win.dil_h * (ih - win.rh)),
                       (float)(w + win.dil_w * (iw - win.rw)), dt, dh, dw, t0, h0, w0, ft, fh, fw);
}

}  // namespace dsa3d
