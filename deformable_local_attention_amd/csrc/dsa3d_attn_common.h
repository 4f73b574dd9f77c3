// dsa3d_attn_common.h -- per-task helpers shared by the forward and backward
// attention kernels (internal; gfx950 only).
//
// A "task" is one (token, head) pair. Tasks of a launch cover the heads
// [head0, head0 + nheads) and are ordered (batch, head, t, h, w) with w
// fastest, so that the lanes of a workgroup hold neighbouring tokens of one
// head, whose sampled neighbourhoods overlap.
#pragma once

#include "dsa3d_device.h"

namespace dsa3d {

struct TaskGrid {
    int32_t T, H, W;
    int32_t heads;          // heads of the full tensors (row stride = heads * head_dim)
    int32_t head0, nheads;  // head range of this launch
    int64_t ntasks;         // B * T * H * W * nheads
};

// task -> batch b, absolute head eta, token coordinates (t,h,w) and the
// token's flat index in [B,T,H,W].
__device__ __forceinline__ void task_coords(const TaskGrid& g, int64_t task, int32_t& b, int32_t& eta, int32_t& t,
                                            int32_t& h, int32_t& w, int64_t& tok) {
    const int64_t HW = (int64_t)g.H * g.W;
    const int64_t THW = HW * g.T;
    const int64_t bh = task / THW;
    int64_t rem = task - bh * THW;
    b = (int32_t)(bh / g.nheads);
    eta = g.head0 + (int32_t)(bh - (int64_t)b * g.nheads);
    t = (int32_t)(rem / HW);
    rem -= (int64_t)t * HW;
    h = (int32_t)(rem / g.W);
    w = (int32_t)(rem - (int64_t)h * g.W);
    tok = (int64_t)b * THW + (int64_t)t * HW + (int64_t)h * g.W + w;
}

// Block order of the attention kernels. A workgroup owns G consecutive
// tokens of one row (t, h, w0 .. w0+G-1) of one (batch, head); blocks are
// dealt out in "supertiles" of ST x SH x SW blocks (t, h, block column), one
// supertile after another, so that the blocks running at the same time on an
// XCD cover a compact 3-D region: the neighbourhoods their samples read then
// overlap, and the key/value (or query/gradient) rows they gather stay in that
// XCD's L2 longer than with a row-by-row order.
struct BlockOrder {
    int32_t G;            // tokens per block along w
    int32_t BW;           // blocks per row: ceil(W / G)
    int32_t ST, SH, SW;   // supertile extent in (t, h, block column)
    int64_t nblk_bh;      // blocks per (batch, head): T * H * BW
};

// Logical block -> (batch*nheads + local head, t, h, first w).
__device__ __forceinline__ void block_coords(const TaskGrid& g, const BlockOrder& o, int64_t lb, int64_t& bh,
                                             int32_t& t, int32_t& h, int32_t& w0) {
    bh = lb / o.nblk_bh;
    int64_t r = lb - bh * o.nblk_bh;
    const int64_t slab = (int64_t)o.ST * g.H * o.BW;       // full t-slab of supertiles
    const int32_t i = (int32_t)(r / slab);
    r -= (int64_t)i * slab;
    const int32_t st = min(o.ST, g.T - i * o.ST);
    const int64_t hrow = (int64_t)st * o.SH * o.BW;        // one h-row of supertiles in this slab
    const int32_t j = (int32_t)(r / hrow);
    r -= (int64_t)j * hrow;
    const int32_t sh = min(o.SH, g.H - j * o.SH);
    const int64_t tile = (int64_t)st * sh * o.SW;          // one full supertile of this row
    const int32_t k = (int32_t)(r / tile);
    r -= (int64_t)k * tile;
    const int32_t sw = min(o.SW, o.BW - k * o.SW);
    const int32_t dt = (int32_t)(r / (sh * sw));
    const int32_t rr = (int32_t)(r - (int64_t)dt * sh * sw);
    const int32_t dh = rr / sw;
    const int32_t dw = rr - dh * sw;
    t = i * o.ST + dt;
    h = j * o.SH + dh;
    w0 = (k * o.SW + dw) * o.G;
}

// The eight trilinear corners x0 + {0,1}^3 of one sample: token index (or -1
// outside the grid) and weight prod_axis (c ? f : 1 - f). Corner i has offset
// (i>>2 & 1, i>>1 & 1, i & 1) in (t, h, w).
struct Corners {
    int64_t tok[8];
    float w[8];
};

__device__ __forceinline__ void make_corners(const TaskGrid& g, int32_t b, int32_t t0, int32_t h0, int32_t w0,
                                             float ft, float fh, float fw, bool inside, Corners& c) {
    const float at[2] = {1.0f - ft, ft}, ah[2] = {1.0f - fh, fh}, aw[2] = {1.0f - fw, fw};
    const int64_t base_b = (int64_t)b * g.T;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ct = (i >> 2) & 1, ch = (i >> 1) & 1, cw = i & 1;
        const int32_t tt = t0 + ct, hh = h0 + ch, ww = w0 + cw;
        const bool ok = inside && (uint32_t)tt < (uint32_t)g.T && (uint32_t)hh < (uint32_t)g.H &&
                        (uint32_t)ww < (uint32_t)g.W;
        c.tok[i] = ok ? ((base_b + tt) * g.H + hh) * (int64_t)g.W + ww : -1;
        c.w[i] = ok ? at[ct] * ah[ch] * aw[cw] : 0.0f;
    }
}

template <typename T>
__device__ __forceinline__ void load_offsets(const T* off, float& dt, float& dh, float& dw) {
    dt = load_scalar<T>(off + 0);
    dh = load_scalar<T>(off + 1);
    dw = load_scalar<T>(off + 2);
}

// Zero row read in place of a corner outside the grid (256 floats: the widest
// row); each code object holds its own copy.
static __device__ __attribute__((aligned(16))) const float g_zero_row[256] = {0.0f};

}  // namespace dsa3d
