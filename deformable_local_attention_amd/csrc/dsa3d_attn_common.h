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
    int32_t chunk;        // XCD placement: 0 = one contiguous range per XCD,
                          // else chunks of this many blocks dealt to the XCDs in turn
    int64_t nblk_bh;      // blocks per (batch, head): T * H * BW
};

// Hardware block id -> logical block. Workgroups are dealt to the 8 XCDs
// round-robin (block i -> XCD i % 8). With chunk = 0 each XCD walks one
// contiguous eighth of the logical blocks; with chunk = c the XCDs take
// consecutive c-block chunks in turn (chunk k on XCD k % 8), so that at any
// time the eight XCDs work on neighbouring chunks and share the rows they
// gather through the memory-side cache. Blocks past the last full round of
// chunks keep their id.
__device__ __forceinline__ uint32_t logical_block(uint32_t bid, uint32_t nblocks, int32_t chunk) {
    if (chunk <= 0) return xcd_logical_block(bid, nblocks);
    const uint32_t round = 8u * (uint32_t)chunk;
    if (bid >= nblocks / round * round) return bid;
    const uint32_t x = bid % 8u, j = bid / 8u;
    return ((j / chunk) * 8u + x) * (uint32_t)chunk + j % (uint32_t)chunk;
}

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

// The eight corners of a sample's cell, for the gathering kernels: weights
// with the grid bounds folded in (a corner outside the grid has weight 0 and
// must be read as a zero row), the token of corner 0 and whether all eight
// corners lie in the grid. Corner i is token tok0 + ct*H*W + ch*W + cw for
// (ct, ch, cw) = (i>>2 & 1, i>>1 & 1, i & 1).
struct CellCorners {
    float w[8];
    uint32_t tok0;  // meaningful for the corners that are in the grid
    uint32_t valid; // bit i: corner i is in the grid
    bool all_in;
};

__device__ __forceinline__ void cell_corners(const TaskGrid& g, uint32_t tok_b, bool inside, int32_t t0, int32_t h0,
                                             int32_t w0, float ft, float fh, float fw, CellCorners& cc) {
    const bool ta = inside && (uint32_t)t0 < (uint32_t)g.T, tb = inside && (uint32_t)(t0 + 1) < (uint32_t)g.T;
    const bool ha = inside && (uint32_t)h0 < (uint32_t)g.H, hb = inside && (uint32_t)(h0 + 1) < (uint32_t)g.H;
    const bool wa = inside && (uint32_t)w0 < (uint32_t)g.W, wb = inside && (uint32_t)(w0 + 1) < (uint32_t)g.W;
    const float at[2] = {ta ? 1.0f - ft : 0.0f, tb ? ft : 0.0f};
    const float ah[2] = {ha ? 1.0f - fh : 0.0f, hb ? fh : 0.0f};
    const float aw[2] = {wa ? 1.0f - fw : 0.0f, wb ? fw : 0.0f};
    const bool vt[2] = {ta, tb}, vh[2] = {ha, hb}, vw[2] = {wa, wb};
    uint32_t valid = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ct = (i >> 2) & 1, ch = (i >> 1) & 1, cw = i & 1;
        cc.w[i] = at[ct] * ah[ch] * aw[cw];
        valid |= (vt[ct] && vh[ch] && vw[cw]) ? (1u << i) : 0u;
    }
    cc.valid = valid;
    cc.all_in = valid == 0xffu;
    cc.tok0 = tok_b + ((uint32_t)t0 * (uint32_t)g.H + (uint32_t)h0) * (uint32_t)g.W + (uint32_t)w0;
}

// The offset (dt, dh, dw) of one sample, widened to float32.
template <typename T>
__device__ __forceinline__ void load_offsets(const T* off, float& dt, float& dh, float& dw) {
    dt = load_scalar<T>(off + 0);
    dh = load_scalar<T>(off + 1);
    dw = load_scalar<T>(off + 2);
}

// One sample's cell as computed by one lane and shared with its group through
// LDS: corner weights with the grid bounds folded in, the token of corner 0,
// the in-grid corner mask, the three fractions, and one spare word.
struct __attribute__((aligned(16))) SampleGeo {
    float w[8];
    uint32_t tok0;
    uint32_t valid;   // bit i: corner i in the grid; bit 8: all eight
    float ft, fh, fw;
    uint32_t extra;
};

// The geometry of window point p of query (t, h, w): reference point, cell
// and corner data.
template <typename T>
__device__ __forceinline__ void sample_geo(const TaskGrid& g, const Window& win, uint32_t tok_b, int32_t t, int32_t h,
                                           int32_t w, int32_t p, const T* off, SampleGeo& sg, int32_t& t0,
                                           int32_t& h0, int32_t& w0) {
    float dt, dh, dw;
    load_offsets<T>(off, dt, dh, dw);
    t0 = h0 = w0 = 0;
    float ft = 0.f, fh = 0.f, fw = 0.f;
    const bool inside = sample_geometry(win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw);
    CellCorners cc;
    cell_corners(g, tok_b, inside, t0, h0, w0, ft, fh, fw, cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) sg.w[i] = cc.w[i];
    sg.tok0 = cc.tok0;
    sg.valid = cc.valid | (cc.all_in ? 0x100u : 0u);
    sg.ft = ft;
    sg.fh = fh;
    sg.fw = fw;
    sg.extra = 0u;
}

// Ordering of LDS accesses between lanes of one wave: the wave executes in
// lockstep and its LDS operations complete in order, so only the compiler
// must be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Strides of the corner rows of one tensor: tokens per frame and per row,
// and the same in bytes (row_bytes = bytes per token).
struct CornerStrides {
    uint32_t hw_tok, w_tok;
    int64_t row_bytes, dh_bytes, dt_bytes;
};

__device__ __forceinline__ CornerStrides corner_strides(const TaskGrid& g, int64_t row_bytes) {
    CornerStrides s;
    s.hw_tok = (uint32_t)g.H * (uint32_t)g.W;
    s.w_tok = (uint32_t)g.W;
    s.row_bytes = row_bytes;
    s.dh_bytes = (int64_t)g.W * row_bytes;
    s.dt_bytes = (int64_t)s.hw_tok * row_bytes;
    return s;
}

// Byte addresses of the eight corner rows in two tensors of the same layout
// (keys and values, or queries and output gradients), starting at `base_a` /
// `base_b` (the lane's part of the head's row of token 0); corners outside the
// grid get `zero`. When every lane of the wave has its whole cell in the grid
// the selects are skipped.
struct CornerAddr {
    const char* a[8];
    const char* b[8];
};

__device__ __forceinline__ void corner_addresses(uint32_t tok0, uint32_t valid, const char* base_a,
                                                 const char* base_b, const CornerStrides& s, const char* zero,
                                                 bool wave_all_in, CornerAddr& ca) {
    const int64_t b_minus_a = base_b - base_a;
    if (wave_all_in) {
        const char* p0 = base_a + (int64_t)(int32_t)tok0 * s.row_bytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ca.a[i] = p0 + (((i >> 2) & 1) ? s.dt_bytes : 0) + (((i >> 1) & 1) ? s.dh_bytes : 0) +
                      ((i & 1) ? s.row_bytes : 0);
            ca.b[i] = ca.a[i] + b_minus_a;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t tok = tok0 + (((i >> 2) & 1) ? s.hw_tok : 0u) + (((i >> 1) & 1) ? s.w_tok : 0u) +
                                 (uint32_t)(i & 1);
            const bool ok = (valid >> i) & 1u;
            const int64_t off = (int64_t)(int32_t)tok * s.row_bytes;
            ca.a[i] = ok ? base_a + off : zero;
            ca.b[i] = ok ? base_b + off : zero;
        }
    }
}

// Zero row read in place of a corner outside the grid (256 floats: the widest
// row); each code object holds its own copy. It is never written; it is not
// declared const so that it lives in the global address space like the
// tensors, which keeps the row loads global rather than flat.
static __device__ __attribute__((aligned(16))) float g_zero_row[256] = {0.0f};

}  // namespace dsa3d
