// dsa3d_conv.hip -- depthwise 3x3x3 convolution of the offset network (gfx950).
//
// The offset network convolves the query tensor [B,T,H,W,C] channel by channel
// with a 3x3x3 kernel (stride 1, zero padding 1, bias) before its pointwise
// layer [MegaSlide-DiT, §5.3 Implementation considerations: nn.Conv3d with
// groups equal to the hidden size; the kernel size is not given there, 3x3x3
// is the reading taken]. Tap (i, j, k) of channel c multiplies the input at
// offset (i-1, j-1, k-1): a cross-correlation, as torch's Conv3d.
//
// The work is bound by memory traffic and plain ALU work, not by a contraction,
// so it runs on the vector units. A lane owns one channel of one row (b, t, h)
// of the grid and walks a run of tokens along w; the 9 input rows at
// (t+-1, h+-1) are read coalesced across the wave (64 consecutive channels)
// and a 3-column window of them, widened to float32 once, slides along w in
// registers, so each input element is loaded once per (row, run) and reused
// for the three outputs it touches along w. The rows a block's neighbours need
// are consecutive blocks (rows are the fastest grid axis), so they meet in L2.
//
//   forward:   y  = bias + conv(q, w)                       (one rounding)
//   dq:        dq += conv(dy, w mirrored through its centre)  (one rounding)
//   dw, db:    per tap, sums over tokens of dy * shifted q, split over groups
//              of rows and then summed over the groups in a fixed order.
#include "dsa3d_device.h"
#include "dsa3d_internal.h"

namespace dsa3d {

namespace {

struct ConvGrid {
    int32_t B, T, H, W;
    int64_t C;
};

// The 9 input rows (t+dt, h+dh), dt, dh in {-1, 0, 1}, of the lane's channel
// pair. A row outside the grid points at the lane's own row and is flagged in
// `outside` (bit r), so its loads stay in bounds and their values are replaced
// by zero (padding) before use.
template <typename T>
__device__ __forceinline__ uint32_t neighbour_rows(const T* x, const ConvGrid& g, int64_t row, int64_t c,
                                                   const T* rows[9]) {
    const int32_t h = (int32_t)(row % g.H);
    const int32_t t = (int32_t)((row / g.H) % g.T);
    uint32_t outside = 0;
#pragma unroll
    for (int dt = -1; dt <= 1; ++dt)
#pragma unroll
        for (int dh = -1; dh <= 1; ++dh) {
            const int r = (dt + 1) * 3 + (dh + 1);
            const bool in = (unsigned)(t + dt) < (unsigned)g.T && (unsigned)(h + dh) < (unsigned)g.H;
            rows[r] = x + ((in ? row + (int64_t)dt * g.H + dh : row) * g.W) * g.C + c;
            if (!in) outside |= 1u << r;
        }
    return outside;
}

// Column w (clamped into the grid; zero for a column outside it) of the 9 rows.
template <typename T, bool EDGE>
__device__ __forceinline__ void load_column(const T* const rows[9], uint32_t outside, const ConvGrid& g, int32_t w,
                                            float col[9]) {
    const bool win = (unsigned)w < (unsigned)g.W;
    const int64_t off = (int64_t)min(max(w, 0), g.W - 1) * g.C;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
        const float v = load_scalar<T>(rows[r] + off);
        const bool keep = win && (!EDGE || !((outside >> r) & 1u));
        col[r] = keep ? v : 0.0f;
    }
}

// The same rows through buffer resources, when a row of the grid spans less
// than 2 GiB: a row outside the grid gets no records and a column outside a
// row lies past its records, so the hardware's range check returns zero for
// both (the padding) and no load needs a clamp or a select. One 32-bit offset,
// (w * C + c) * sizeof(T), serves all nine rows.
struct RowRsrc {
    __amdgpu_buffer_rsrc_t r[9];
};

constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer resource: untyped 32-bit data format

template <typename T>
__device__ __forceinline__ void neighbour_rsrc(const T* x, const ConvGrid& g, int64_t row, RowRsrc& rs) {
    // rows number fewer than 2^31 (B*T*H*W < 2^31): 32-bit division
    const uint32_t r32 = (uint32_t)row;
    const int32_t h = (int32_t)(r32 % (uint32_t)g.H);
    const int32_t t = (int32_t)((r32 / (uint32_t)g.H) % (uint32_t)g.T);
    const int32_t nrec = (int32_t)((int64_t)g.W * g.C * (int64_t)sizeof(T));
#pragma unroll
    for (int dt = -1; dt <= 1; ++dt)
#pragma unroll
        for (int dh = -1; dh <= 1; ++dh) {
            const int r = (dt + 1) * 3 + (dh + 1);
            const bool in = (unsigned)(t + dt) < (unsigned)g.T && (unsigned)(h + dh) < (unsigned)g.H;
            const T* base = x + (in ? (row + (int64_t)dt * g.H + dh) * g.W * g.C : 0);
            rs.r[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, in ? nrec : 0, kBufferWord3);
        }
}

template <typename T> __device__ __forceinline__ float load_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t voff);
template <> __device__ __forceinline__ float load_rsrc<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
template <> __device__ __forceinline__ float load_rsrc<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0) << 16);
}

// Column w of the 9 rows (zero outside the grid) for channel c.
template <typename T>
__device__ __forceinline__ void load_column_rsrc(const RowRsrc& rs, const ConvGrid& g, int32_t w, int64_t c,
                                                 float col[9]) {
    const uint32_t voff = (uint32_t)(((int64_t)w * g.C + c) * (int64_t)sizeof(T));  // w = -1 wraps past the records
#pragma unroll
    for (int r = 0; r < 9; ++r) col[r] = load_rsrc<T>(rs.r[r], voff);
}

// The lane's weights of channel c (MIRROR: tap 26 - tap), float32.
template <typename T, bool MIRROR>
__device__ __forceinline__ void load_weights(const T* wt, int64_t c, float wa[27]) {
#pragma unroll
    for (int tap = 0; tap < 27; ++tap) wa[tap] = load_scalar<T>(wt + c * 27 + (MIRROR ? 26 - tap : tap));
}

// One row run [w0, w1) of outputs; `column(w, col)` loads column w of the 9 rows.
template <typename T, bool ACCUM, typename Column>
__device__ __forceinline__ void conv_run(Column column, const ConvGrid& g, int32_t w0, int32_t w1, const float wa[27],
                                         float bb, T* orow) {
    float cm[9], c0[9], cp[9];  // columns w-1, w, w+1
    column(w0 - 1, cm);
    column(w0, c0);
    for (int32_t w = w0; w < w1; ++w) {
        column(w + 1, cp);
        float acc = bb;
#pragma unroll
        for (int r = 0; r < 9; ++r) {
            acc = fmaf(wa[r * 3 + 0], cm[r], acc);
            acc = fmaf(wa[r * 3 + 1], c0[r], acc);
            acc = fmaf(wa[r * 3 + 2], cp[r], acc);
        }
        T* o = orow + (int64_t)w * g.C;
        if (ACCUM) acc += load_scalar<T>(o);
        store_scalar<T>(o, acc);
#pragma unroll
        for (int r = 0; r < 9; ++r) {
            cm[r] = c0[r];
            c0[r] = cp[r];
        }
    }
}

}  // namespace

// y[row, w, c] = bias[c] + sum_tap wt[c, tap] * x[row + (dt, dh), w + dk, c] (MIRROR: tap 26 - tap),
// or (ACCUM) out[...] += the sum without bias. One block per (row (b,t,h), group of 256 channels,
// run of `run` tokens along w). BUF: the input rows are read through buffer resources.
template <typename T, bool MIRROR, bool ACCUM, bool BUF>
__global__ void __launch_bounds__(256) dsa3d_dwconv_kernel(const T* x, const T* wt, const T* bias, T* out, ConvGrid g,
                                                           int32_t run, int64_t ngroups) {
    // 1-D grid, XCD-contiguous: each XCD walks a range of (run, channel group, row) with the row
    // fastest, so the blocks of neighbouring rows, which read the same input rows, share its L2
    const int64_t nrows = (int64_t)g.B * g.T * g.H;
    const int64_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t row = lb % nrows;
    const int64_t cg = (lb / nrows) % ngroups;
    const int32_t ri = (int32_t)(lb / nrows / ngroups);
    const int64_t c = cg * 256 + threadIdx.x;
    if (c >= g.C) return;
    const int32_t w0 = ri * run;
    const int32_t w1 = min(g.W, w0 + run);
    float wa[27];
    load_weights<T, MIRROR>(wt, c, wa);
    const float bb = (!ACCUM && bias) ? load_scalar<T>(bias + c) : 0.0f;
    T* orow = out + row * g.W * g.C + c;
    if constexpr (BUF) {
        RowRsrc rs;
        neighbour_rsrc(x, g, row, rs);
        conv_run<T, ACCUM>([&](int32_t w, float col[9]) { load_column_rsrc<T>(rs, g, w, c, col); }, g, w0, w1, wa,
                           bb, orow);
    } else {
        const T* rows[9];
        const uint32_t outside = neighbour_rows(x, g, row, c, rows);
        if (outside)
            conv_run<T, ACCUM>([&](int32_t w, float col[9]) { load_column<T, true>(rows, outside, g, w, col); }, g,
                               w0, w1, wa, bb, orow);
        else
            conv_run<T, ACCUM>([&](int32_t w, float col[9]) { load_column<T, false>(rows, outside, g, w, col); }, g,
                               w0, w1, wa, bb, orow);
    }
}

namespace {

// bf16 rows, two channels per lane, on v_dot2_f32_bf16: each lane owns the
// channel pair (c, c+1), loaded as one 32-bit word per input row and column.
// The nine rows of a column are paired ((0,1), (2,3), (4,5), (6,7), (8,zero))
// into words that hold one channel of two rows, so one dot2 multiplies two taps
// of a channel by their (bf16, exact) weights and adds both products into the
// float32 sum: 15 dot2 per output element instead of 27 multiply-adds, and no
// widening of the inputs. A column's pairs are formed once (byte permutes)
// and serve the three outputs along w that read it. Rows come through buffer
// resources (a row outside the grid has no records and a column outside a
// row lies past them: the hardware's range check supplies the zero padding).
// MIRROR: the kernel mirrored through its centre (the input gradient);
// ACCUM: added to the output (one rounding), without bias.
struct ColPairs {
    uint32_t p[5][2];  // [row pair][channel of the lane's pair]
};

__device__ __forceinline__ void pair_column(const uint32_t x[9], ColPairs& cp) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        cp.p[j][0] = __builtin_amdgcn_perm(x[2 * j + 1], x[2 * j], 0x05040100u);  // channel c of rows 2j, 2j+1
        cp.p[j][1] = __builtin_amdgcn_perm(x[2 * j + 1], x[2 * j], 0x07060302u);  // channel c+1
    }
    cp.p[4][0] = x[8] & 0xffffu;
    cp.p[4][1] = x[8] >> 16;
}

template <bool MIRROR, bool ACCUM>
__global__ void __launch_bounds__(256) dsa3d_dwconv_pair_kernel(const bf16_t* x, const bf16_t* wt, const bf16_t* bias,
                                                                bf16_t* out, ConvGrid g, int32_t run, int64_t ngroups) {
    const uint32_t nrows = (uint32_t)g.B * (uint32_t)g.T * (uint32_t)g.H;  // < 2^31
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t row = lb % nrows;
    const uint32_t cg = (lb / nrows) % (uint32_t)ngroups;
    const int32_t ri = (int32_t)(lb / nrows / (uint32_t)ngroups);
    const int64_t c = (int64_t)cg * 512 + 2 * (int64_t)threadIdx.x;  // the lane's channel pair (c, c+1)
    if (c >= g.C) return;  // C is even: a pair is whole or absent
    const int32_t w0 = ri * run;
    const int32_t w1 = min(g.W, w0 + run);
    // weight words: [column k][row pair j][channel], each (row 2j, row 2j+1) as bf16 (lo, hi)
    uint32_t wp[3][5][2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const bf16_t* wc = wt + (c + ch) * 27;
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int r0 = 2 * j, r1 = 2 * j + 1;
                const int t0 = MIRROR ? 26 - (r0 * 3 + k) : r0 * 3 + k;
                const int t1 = MIRROR ? 26 - (r1 * 3 + k) : r1 * 3 + k;
                const uint32_t lo = wc[t0];
                const uint32_t hi = r1 < 9 ? (uint32_t)wc[t1] : 0u;
                wp[k][j][ch] = lo | (hi << 16);
            }
    }
    float bb[2] = {0.0f, 0.0f};
    if (!ACCUM && bias) {
        bb[0] = load_scalar<bf16_t>(bias + c);
        bb[1] = load_scalar<bf16_t>(bias + c + 1);
    }
    RowRsrc rs;
    neighbour_rsrc(x, g, row, rs);
    const int64_t C2 = g.C * 2;  // bytes per token
    auto load_column = [&](int32_t w, uint32_t v[9]) {
        const uint32_t voff = (uint32_t)((int64_t)w * C2 + c * 2);  // w = -1 wraps past the records
#pragma unroll
        for (int r = 0; r < 9; ++r) v[r] = __builtin_amdgcn_raw_buffer_load_b32(rs.r[r], voff, 0, 0);
    };
    ColPairs ca, cb, cc;
    uint32_t raw[9];
    load_column(w0 - 1, raw);
    pair_column(raw, ca);
    load_column(w0, raw);
    pair_column(raw, cb);
    load_column(w0 + 1, raw);  // a column past the row reads zeros
    bf16_t* orow = out + row * g.W * g.C + c;
    // One output: columns (l, m, r) = (w-1, w, w+1); column w+1 arrived during
    // the previous output and is paired now, column w+2 is requested now. The
    // loop is unrolled by three so that the three column buffers rotate by
    // name instead of being copied.
    auto step = [&](int32_t w, const ColPairs& l, const ColPairs& m, ColPairs& r) {
        pair_column(raw, r);
        load_column(w + 2, raw);
        float acc[2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            float s = bb[ch];
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                s = dot2_bf16(l.p[j][ch], wp[0][j][ch], s);
                s = dot2_bf16(m.p[j][ch], wp[1][j][ch], s);
                s = dot2_bf16(r.p[j][ch], wp[2][j][ch], s);
            }
            acc[ch] = s;
        }
        uint32_t* o = reinterpret_cast<uint32_t*>(orow + (int64_t)w * g.C);
        if (ACCUM) {
            const uint32_t old = *o;
            acc[0] = bf16_lo(old) + acc[0];
            acc[1] = bf16_hi(old) + acc[1];
        }
        *o = pack_bf16x2(acc[0], acc[1]);
    };
    for (int32_t w = w0; w < w1; w += 3) {
        step(w, ca, cb, cc);
        if (w + 1 >= w1) break;
        step(w + 1, cb, cc, ca);
        if (w + 2 >= w1) break;
        step(w + 2, cc, ca, cb);
    }
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// bf16 rows whose channel count is a multiple of 64, through LDS. A block owns
// 64 channels of an 8-row x 16-token tile of the (h, w) plane and walks a run
// of frames. The input slab that one frame contributes (the tile and a
// one-token halo: 10 rows x 18 tokens x 64 channels, one 128-byte piece per
// token) is loaded once into one of three LDS slots, which hold the frames
// f-1, f and f+1 of the output frame f; the slabs of frames f+2 and f+3 are in
// flight in registers while frame f is computed. Each input element thus
// passes the texture path about 1.4 times per frame run (plus two halo frames
// per run) instead of nine times, the stencil's reuse across rows and frames
// coming from LDS rather than from L2.
//
// A thread owns one output row of the tile and one channel pair and walks the
// tile's 16 tokens along w with the column pairs and dot2 products of the pair
// kernel above (forward and input gradient), or, for the weight gradient,
// sums dy * input per tap in float32 and the block then adds its eight rows'
// sums in a fixed order into one partial per tile.
// ---------------------------------------------------------------------------
constexpr int CT_TH = 8, CT_TW = 16;                 // output rows and tokens of a tile
constexpr int CT_SR = CT_TH + 2, CT_SC = CT_TW + 2;  // slab rows and tokens (one-token halo)
constexpr int CT_ROWB = CT_SC * 128 + 128;           // bytes per slab row, padded so that rows r and
                                                     // r+1 start 32 banks apart
constexpr int CT_SLOT = CT_SR * CT_ROWB;             // one frame's slab: 24,320 bytes
constexpr int CT_PIECES = CT_SR * CT_SC * 8;         // 16-byte pieces per slab: 1,440
constexpr int CT_THREADS = 32 * CT_TH;               // a thread per output row and channel pair
constexpr int CT_LOADS = (CT_PIECES + CT_THREADS - 1) / CT_THREADS;  // per thread: 6

enum { CT_FWD = 0, CT_DQ = 1, CT_WGRAD = 2 };
// the weight gradient's row sums ([row][channel][27 taps + bias] floats) reuse the three slots
static_assert(CT_TH * 64 * 28 * 4 <= 3 * CT_SLOT, "the row sums must fit in the slab slots");

struct TileCoords {
    int32_t b, ta, tb, h0, w0;
    int64_t c0;
    int64_t group;  // the tile's index among the (batch, frame run, row tile, token tile) tiles
};

__device__ __forceinline__ TileCoords tile_coords(const ConvGrid& g, int32_t tc, int32_t ntc, int32_t nht,
                                                  int32_t nwt, uint32_t ncg) {
    // channel groups fastest: the blocks of one tile read the same tokens' rows side by side
    uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    TileCoords tc_;
    tc_.c0 = (int64_t)(lb % ncg) * 64;
    lb /= ncg;
    const int32_t wi = (int32_t)(lb % (uint32_t)nwt);
    lb /= (uint32_t)nwt;
    const int32_t hi = (int32_t)(lb % (uint32_t)nht);
    lb /= (uint32_t)nht;
    const int32_t ti = (int32_t)(lb % (uint32_t)ntc);
    tc_.b = (int32_t)(lb / (uint32_t)ntc);
    tc_.group = (((int64_t)tc_.b * ntc + ti) * nht + hi) * nwt + wi;
    tc_.ta = ti * tc;
    tc_.tb = min(g.T, tc_.ta + tc);
    tc_.h0 = hi * CT_TH;
    tc_.w0 = wi * CT_TW;
    return tc_;
}

// The pieces this thread moves for every frame: the byte offset of its piece
// within one frame of the input (from the frame's first token), or an offset
// past the frame for a piece outside the grid's (h, w) plane, and its LDS
// offset within a slot.
constexpr uint32_t CT_OUTSIDE = 0x80000000u;  // past every frame's records: the load returns zero

struct SlabPieces {
    uint32_t goff[CT_LOADS];
    uint32_t soff[CT_LOADS];
};

__device__ __forceinline__ void slab_pieces(const ConvGrid& g, const TileCoords& tc, SlabPieces& sp) {
#pragma unroll
    for (int i = 0; i < CT_LOADS; ++i) {
        const int k = (int)threadIdx.x + CT_THREADS * i;
        const int piece = k >> 3, part = k & 7;
        const int srow = piece / CT_SC, scol = piece % CT_SC;
        const int32_t h = tc.h0 - 1 + srow, w = tc.w0 - 1 + scol;
        const bool in = k < CT_PIECES && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
        sp.goff[i] = in ? (uint32_t)((((int64_t)h * g.W + w) * g.C + tc.c0 + 8 * part) * 2) : CT_OUTSIDE;
        sp.soff[i] = (uint32_t)(srow * CT_ROWB + scol * 128 + part * 16);
    }
}

// One frame of one batch item as a buffer resource: no records for a frame
// outside [0, T), so that its loads return zero (the padding) without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t frame_rsrc(const bf16_t* x, const ConvGrid& g, int32_t b,
                                                             int32_t f) {
    const bool fin = (unsigned)f < (unsigned)g.T;
    const int64_t fsize = (int64_t)g.H * g.W * g.C;
    const bf16_t* base = x + (fin ? ((int64_t)b * g.T + f) * fsize : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), (short)0, fin ? (int)(fsize * 2) : 0,
                                             kBufferWord3);
}

typedef __attribute__((ext_vector_type(4))) uint32_t ct_u32x4;

// Frame f's slab into registers (zero outside the grid).
__device__ __forceinline__ void slab_load(const bf16_t* x, const ConvGrid& g, const TileCoords& tc,
                                          const SlabPieces& sp, int32_t f, ct_u32x4 v[CT_LOADS]) {
    const __amdgpu_buffer_rsrc_t rs = frame_rsrc(x, g, tc.b, f);
#pragma unroll
    for (int i = 0; i < CT_LOADS; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, sp.goff[i], 0, 0);
}

__device__ __forceinline__ void slab_store(char* slot, const SlabPieces& sp, const ct_u32x4 v[CT_LOADS]) {
#pragma unroll
    for (int i = 0; i < CT_LOADS; ++i)
        if (CT_THREADS * (i + 1) <= CT_PIECES || (int)threadIdx.x + CT_THREADS * i < CT_PIECES)
            *reinterpret_cast<ct_u32x4*>(slot + sp.soff[i]) = v[i];
}

template <int MODE>
__global__ void __launch_bounds__(CT_THREADS) dsa3d_dwconv_tile_kernel(const bf16_t* x, const bf16_t* wt,
                                                                const bf16_t* bias, bf16_t* out, const bf16_t* dy,
                                                                float* part, float* partb, ConvGrid g, int32_t tc,
                                                                int32_t ntc, int32_t nht, int32_t nwt) {
    __shared__ __attribute__((aligned(16))) char lds[3 * CT_SLOT];
    const uint32_t ncg = (uint32_t)(g.C / 64);
    const TileCoords tcd = tile_coords(g, tc, ntc, nht, nwt, ncg);
    const int r = (int)threadIdx.x >> 5, p = (int)threadIdx.x & 31;
    const int64_t c = tcd.c0 + 2 * p;  // the thread's channel pair (c, c+1)
    const int32_t h = tcd.h0 + r;
    const bool hin = h < g.H;

    SlabPieces sp;
    slab_pieces(g, tcd, sp);
    // the thread's first output of a frame row, in bytes from the frame's first token (or outside)
    const uint32_t row_off = hin ? (uint32_t)((((int64_t)h * g.W + tcd.w0) * g.C + c) * 2) : CT_OUTSIDE;
    // slot of frame f (f >= ta - 1)
    auto slot = [&](int32_t f) -> uint32_t { return (uint32_t)((f - tcd.ta + 1) % 3) * CT_SLOT; };

    // forward / input gradient: weight words [column k][row pair j][channel], rows (2j, 2j+1) as (lo, hi)
    uint32_t wp[3][5][2];
    float bb[2] = {0.0f, 0.0f};
    // weight gradient: sums [tap][channel] and the bias sums
    float aa[27][2];
    float sb[2] = {0.0f, 0.0f};
    if constexpr (MODE != CT_WGRAD) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const bf16_t* wc = wt + (c + ch) * 27;
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int j = 0; j < 5; ++j) {
                    const int r0 = 2 * j, r1 = 2 * j + 1;
                    const int t0 = MODE == CT_DQ ? 26 - (r0 * 3 + k) : r0 * 3 + k;
                    const int t1 = MODE == CT_DQ ? 26 - (r1 * 3 + k) : r1 * 3 + k;
                    const uint32_t lo = wc[t0];
                    const uint32_t hi = r1 < 9 ? (uint32_t)wc[t1] : 0u;
                    wp[k][j][ch] = lo | (hi << 16);
                }
        }
        if (MODE == CT_FWD && bias) {
            bb[0] = load_scalar<bf16_t>(bias + c);
            bb[1] = load_scalar<bf16_t>(bias + c + 1);
        }
    } else {
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) aa[tap][0] = aa[tap][1] = 0.0f;
    }

    // the input gradient's existing values (dq) or the output gradient (weight gradient) of the
    // thread's 16 outputs of a frame, requested a frame ahead
    constexpr bool ROWVALS = MODE != CT_FWD;
    const bf16_t* rv_src = MODE == CT_DQ ? out : dy;
    uint32_t rv_cur[CT_TW], rv_nxt[CT_TW];
    auto rowvals = [&](int32_t f, uint32_t dst[CT_TW]) {
        const __amdgpu_buffer_rsrc_t rs = frame_rsrc(rv_src, g, tcd.b, f);
#pragma unroll
        for (int j = 0; j < CT_TW; ++j) {
            const bool ok = tcd.w0 + j < g.W;  // (a row outside the grid has row_off outside)
            dst[j] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, ok ? row_off + (uint32_t)(j * g.C * 2) : CT_OUTSIDE, 0, 0);
        }
    };
    if constexpr (ROWVALS) rowvals(tcd.ta, rv_nxt);

    // Two frames' slabs are in flight in registers, va and vb alternating. Every
    // frame step issues the same memory operations in the same order, with no
    // branch around them: a frame outside the run reads and writes through a
    // resource without records (loads return zero, stores are dropped), so the
    // compiler's count of the operations in flight after each load is exact and
    // the wait for one slab does not also wait for the next.
    ct_u32x4 va[CT_LOADS], vb[CT_LOADS];
    slab_load(x, g, tcd, sp, tcd.ta - 1, va);
    slab_store(lds + slot(tcd.ta - 1), sp, va);
    slab_load(x, g, tcd, sp, tcd.ta, va);
    slab_store(lds + slot(tcd.ta), sp, va);
    slab_load(x, g, tcd, sp, tcd.ta + 1, va);
    slab_load(x, g, tcd, sp, tcd.ta + 2 <= tcd.tb ? tcd.ta + 2 : -1, vb);
    // output frame t (dropped past the run); v holds frame t+1's slab and then takes frame t+3's
    auto frame = [&](int32_t t, ct_u32x4 v[CT_LOADS]) {
        const bool live = t < tcd.tb;
        slab_store(lds + slot(t + 1), sp, v);  // the slot of frame t-2, free since the last barrier
        __syncthreads();
        slab_load(x, g, tcd, sp, t + 3 <= tcd.tb ? t + 3 : -1, v);  // in flight during frames t and t+1
        if constexpr (ROWVALS) {
#pragma unroll
            for (int j = 0; j < CT_TW; ++j) rv_cur[j] = rv_nxt[j];
            rowvals(t + 1 < tcd.tb ? t + 1 : -1, rv_nxt);
        }
        // the nine rows (t+dt, h+dh) of the thread's channel pair, row index (dt+1)*3 + (dh+1)
        uint32_t rb[9];
#pragma unroll
        for (int dt = -1; dt <= 1; ++dt)
#pragma unroll
            for (int dh = -1; dh <= 1; ++dh)
                rb[(dt + 1) * 3 + (dh + 1)] = slot(t + dt) + (uint32_t)((r + 1 + dh) * CT_ROWB + 4 * p);
        auto column = [&](int col, uint32_t raw[9]) {
#pragma unroll
            for (int i = 0; i < 9; ++i) raw[i] = *reinterpret_cast<const uint32_t*>(lds + rb[i] + col * 128);
        };
        if constexpr (MODE != CT_WGRAD) {
            const __amdgpu_buffer_rsrc_t ors = frame_rsrc(out, g, tcd.b, live ? t : -1);
            ColPairs ca, cb, cc;
            uint32_t raw[9];
            column(0, raw);
            pair_column(raw, ca);
            column(1, raw);
            pair_column(raw, cb);
            column(2, raw);
            // output j (token w0 + j) reads slab columns j, j+1, j+2
            auto step = [&](int j, const ColPairs& l, const ColPairs& m, ColPairs& rr) {
                pair_column(raw, rr);
                if (j + 3 < CT_SC) column(j + 3, raw);
                float acc[2];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    float s = bb[ch];
#pragma unroll
                    for (int jj = 0; jj < 5; ++jj) {
                        s = dot2_bf16(l.p[jj][ch], wp[0][jj][ch], s);
                        s = dot2_bf16(m.p[jj][ch], wp[1][jj][ch], s);
                        s = dot2_bf16(rr.p[jj][ch], wp[2][jj][ch], s);
                    }
                    acc[ch] = s;
                }
                if (MODE == CT_DQ) {
                    acc[0] = bf16_lo(rv_cur[j]) + acc[0];
                    acc[1] = bf16_hi(rv_cur[j]) + acc[1];
                }
                // a token past the row or a row outside the grid: an offset past the records
                const bool ok = tcd.w0 + j < g.W;
                __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(acc[0], acc[1]), ors,
                                                      ok ? row_off + (uint32_t)(j * g.C * 2) : CT_OUTSIDE, 0, 0);
            };
#pragma unroll
            for (int j = 0; j < CT_TW; j += 3) {
                step(j, ca, cb, cc);
                if (j + 1 < CT_TW) step(j + 1, cb, cc, ca);
                if (j + 2 < CT_TW) step(j + 2, cc, ca, cb);
            }
        } else if (live) {  // (no memory operation inside: the branch leaves the counts alone)
            // columns j, j+1, j+2 widened to float32: [row][channel]
            float cm[9][2], c0[9][2], cp[9][2];
            uint32_t raw[9];
            auto widen = [&](const uint32_t rw[9], float col[9][2]) {
#pragma unroll
                for (int i = 0; i < 9; ++i) {
                    col[i][0] = bf16_lo(rw[i]);
                    col[i][1] = bf16_hi(rw[i]);
                }
            };
            column(0, raw);
            widen(raw, cm);
            column(1, raw);
            widen(raw, c0);
#pragma unroll
            for (int j = 0; j < CT_TW; ++j) {
                column(j + 2, raw);
                widen(raw, cp);
                const int32_t w = tcd.w0 + j;
                if (hin && w < g.W) {
                    const uint32_t d = rv_cur[j];
                    const float d0 = bf16_lo(d), d1 = bf16_hi(d);
                    sb[0] += d0;
                    sb[1] += d1;
#pragma unroll
                    for (int i = 0; i < 9; ++i) {
                        aa[i * 3 + 0][0] = fmaf(d0, cm[i][0], aa[i * 3 + 0][0]);
                        aa[i * 3 + 0][1] = fmaf(d1, cm[i][1], aa[i * 3 + 0][1]);
                        aa[i * 3 + 1][0] = fmaf(d0, c0[i][0], aa[i * 3 + 1][0]);
                        aa[i * 3 + 1][1] = fmaf(d1, c0[i][1], aa[i * 3 + 1][1]);
                        aa[i * 3 + 2][0] = fmaf(d0, cp[i][0], aa[i * 3 + 2][0]);
                        aa[i * 3 + 2][1] = fmaf(d1, cp[i][1], aa[i * 3 + 2][1]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 9; ++i) {
                    cm[i][0] = c0[i][0]; cm[i][1] = c0[i][1];
                    c0[i][0] = cp[i][0]; c0[i][1] = cp[i][1];
                }
            }
        }
        __syncthreads();  // every thread is done with frame t-1's slot
    };
    // the first pair of frames outside the loop, so that the loop starts from the
    // same operations in flight as every later pair
    frame(tcd.ta, va);
    frame(tcd.ta + 1, vb);
    for (int32_t t = tcd.ta + 2; t < tcd.tb; t += 2) {
        frame(t, va);
        frame(t + 1, vb);
    }
    if constexpr (MODE == CT_WGRAD) {
        // the eight rows' sums of each (channel, tap), added in row order: [row][channel][28] floats
        // (27 taps and the bias sum) in the slab slots, which no thread reads any more
        float* red = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            float* dst = red + ((size_t)r * 64 + 2 * p + ch) * 28;
#pragma unroll
            for (int tap = 0; tap < 27; ++tap) dst[tap] = aa[tap][ch];
            dst[27] = sb[ch];
        }
        __syncthreads();
        for (int i = (int)threadIdx.x; i < 64 * 28; i += CT_THREADS) {
            float s = 0.0f;
#pragma unroll
            for (int rr = 0; rr < CT_TH; ++rr) s += red[rr * 64 * 28 + i];
            const int ch = i / 28, tap = i % 28;
            if (tap < 27)
                part[(tcd.group * g.C + tcd.c0 + ch) * 27 + tap] = s;
            else
                partb[tcd.group * g.C + tcd.c0 + ch] = s;
        }
    }
}

}  // namespace

namespace {

// The weight-gradient sums of one row: acc[tap] += dy[w] * x[row + (dt, dh), w + dk];
// `column(w, col)` loads column w of the 9 input rows.
template <typename T, typename Column>
__device__ __forceinline__ void wgrad_row(Column column, const T* grow, const ConvGrid& g, float aa[27], float& sb) {
    float cm[9], c0[9], cp[9];
    column(-1, cm);
    column(0, c0);
    for (int32_t w = 0; w < g.W; ++w) {
        column(w + 1, cp);
        const float d = load_scalar<T>(grow + (int64_t)w * g.C);
        sb += d;
#pragma unroll
        for (int r = 0; r < 9; ++r) {
            aa[r * 3 + 0] = fmaf(d, cm[r], aa[r * 3 + 0]);
            aa[r * 3 + 1] = fmaf(d, c0[r], aa[r * 3 + 1]);
            aa[r * 3 + 2] = fmaf(d, cp[r], aa[r * 3 + 2]);
        }
#pragma unroll
        for (int r = 0; r < 9; ++r) {
            cm[r] = c0[r];
            c0[r] = cp[r];
        }
    }
}

}  // namespace

// Per group of `rows_per_group` rows: part[group][c][tap] = sum over the
// group's tokens of dy[tok, c] * x[tok + tap offset, c], partb[group][c] =
// sum of dy[tok, c]; rows in increasing order, w in increasing order.
// One block per (group of rows, group of 256 channels).
template <typename T>
__global__ void __launch_bounds__(256) dsa3d_dwconv_wgrad_kernel(const T* x, const T* dy, float* part, float* partb,
                                                                 ConvGrid g, int64_t rows_per_group) {
    // 1-D grid, XCD-contiguous, row groups fastest (neighbouring groups share input rows)
    const int64_t nrows = (int64_t)g.B * g.T * g.H;
    const int64_t ngrp = (nrows + rows_per_group - 1) / rows_per_group;
    const int64_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t grp = lb % ngrp;
    const int64_t c = (lb / ngrp) * 256 + threadIdx.x;
    if (c >= g.C) return;
    const int64_t r0 = grp * rows_per_group;
    const int64_t r1 = min(nrows, r0 + rows_per_group);
    float aa[27];
#pragma unroll
    for (int tap = 0; tap < 27; ++tap) aa[tap] = 0.f;
    float sb = 0.f;
    for (int64_t row = r0; row < r1; ++row) {
        const T* grow = dy + row * g.W * g.C + c;
        const T* rows[9];
        const uint32_t outside = neighbour_rows(x, g, row, c, rows);
        if (outside)
            wgrad_row<T>([&](int32_t w, float col[9]) { load_column<T, true>(rows, outside, g, w, col); }, grow, g,
                         aa, sb);
        else
            wgrad_row<T>([&](int32_t w, float col[9]) { load_column<T, false>(rows, outside, g, w, col); }, grow, g,
                         aa, sb);
    }
    float* pa = part + (grp * g.C + c) * 27;
#pragma unroll
    for (int tap = 0; tap < 27; ++tap) pa[tap] = aa[tap];
    partb[grp * g.C + c] = sb;
}

// out[i] = sum_{z < nsplit} part[z*n + i], z in increasing order.
__global__ void __launch_bounds__(256) dsa3d_conv_split_sum_kernel(const float* part, float* out, int64_t n,
                                                                   int64_t nsplit) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.0f;
        for (int64_t z = 0; z < nsplit; ++z) s += part[z * n + i];
        out[i] = s;
    }
}

namespace {

ConvGrid conv_grid(const dsa3d_desc& d) {
    return ConvGrid{(int32_t)d.B, (int32_t)d.T, (int32_t)d.H, (int32_t)d.W, (int64_t)d.heads * d.head_dim};
}

// Rows per group of the weight gradient: enough groups for about 8192 waves,
// at most 512 (each output of the split sum adds the groups one by one).
int64_t wgrad_rows_per_group(const dsa3d_desc& d) {
    const int64_t rows = d.B * d.T * d.H;
    const int64_t C = (int64_t)d.heads * d.head_dim;
    const int64_t waves_per_group = (C + 63) / 64;
    const int64_t groups = std::max<int64_t>(
        1, std::min<int64_t>({rows, (int64_t)512, 8192 / std::max<int64_t>(1, waves_per_group)}));
    return (rows + groups - 1) / groups;
}

// The LDS-tiled kernels take bf16 rows whose channel count is a multiple of 64
// from an input whose base is 16-byte aligned (the slabs move in 16-byte
// pieces), with frames of less than 2 GiB.
struct ConvTiles {
    int32_t tc, ntc, nht, nwt;
    int64_t groups;  // B * ntc * nht * nwt
};

bool conv_tiled(const dsa3d_desc& d, const void* x) {
    const int64_t C = (int64_t)d.heads * d.head_dim;
    // one frame (H * W * C bf16) is addressed by 32-bit buffer offsets below 2^31
    return d.dtype != DSA3D_F32 && C % 64 == 0 && ((uintptr_t)x & 15u) == 0 && d.H * d.W * C * 2 < (1ll << 31);
}

// Frame runs of 16 frames; for the weight gradient, longer runs when the tiles
// would otherwise number more than 512 (each output of the split sum adds the
// tiles' partials one by one).
ConvTiles conv_tiles(const dsa3d_desc& d, bool wgrad) {
    ConvTiles t;
    t.nht = (int32_t)((d.H + CT_TH - 1) / CT_TH);
    t.nwt = (int32_t)((d.W + CT_TW - 1) / CT_TW);
    int64_t runs = (d.T + 15) / 16;
    if (wgrad) {
        const int64_t per = std::max<int64_t>(1, d.B * t.nht * t.nwt);
        runs = std::max<int64_t>(1, std::min<int64_t>(runs, 512 / per));
    }
    t.tc = (int32_t)((d.T + runs - 1) / runs);
    t.ntc = (int32_t)((d.T + t.tc - 1) / t.tc);
    t.groups = d.B * t.ntc * (int64_t)t.nht * t.nwt;
    return t;
}

// The forward reads a grid row of less than 2 GiB (W * C * sizeof(T)) through buffer resources:
// at 720p (64x45x80 tokens, 1024 channels, bf16) 0.50 ms against 0.61 ms. The dq and weight
// kernels measured 5% and 38% slower that way and keep the clamped loads.
bool conv_rows_buffered(const ConvGrid& g, size_t elem) { return (uint64_t)g.W * (uint64_t)g.C * elem < (1ull << 31); }

template <typename T, bool MIRROR, bool ACCUM>
hipError_t conv_launch(const dsa3d_desc& d, const void* x, const void* w, const void* bias, void* out, int kernel_id,
                       hipStream_t s) {
    const ConvGrid g = conv_grid(d);
    const int64_t rows = (int64_t)g.B * g.T * g.H;
    if (rows == 0 || g.W == 0) return hipSuccess;
    // runs of at most 64 tokens along w, of equal length
    const int32_t nrun = (g.W + 63) / 64;
    const int32_t run = (g.W + nrun - 1) / nrun;
    const int64_t ngroups = (g.C + 255) / 256;
    const int64_t nblocks = rows * ngroups * nrun;
    LaunchScope ls(kernel_id, s);
    if constexpr (sizeof(T) == 2) {
        if (conv_tiled(d, x)) {
            const ConvTiles ct = conv_tiles(d, false);
            const int64_t nb = ct.groups * (g.C / 64);
            hipLaunchKernelGGL((dsa3d_dwconv_tile_kernel<MIRROR ? CT_DQ : CT_FWD>), dim3((unsigned)nb), dim3(CT_THREADS), 0, s,
                               reinterpret_cast<const bf16_t*>(x), reinterpret_cast<const bf16_t*>(w),
                               reinterpret_cast<const bf16_t*>(bias), reinterpret_cast<bf16_t*>(out), nullptr, nullptr,
                               nullptr, g, ct.tc, ct.ntc, ct.nht, ct.nwt);
            return hipGetLastError();
        }
        if (conv_rows_buffered(g, sizeof(T))) {
            const int64_t ngroups2 = (g.C + 511) / 512;
            hipLaunchKernelGGL((dsa3d_dwconv_pair_kernel<MIRROR, ACCUM>), dim3((unsigned)(rows * ngroups2 * nrun)),
                               dim3(256), 0, s, reinterpret_cast<const bf16_t*>(x), reinterpret_cast<const bf16_t*>(w),
                               reinterpret_cast<const bf16_t*>(bias), reinterpret_cast<bf16_t*>(out), g, run, ngroups2);
            return hipGetLastError();
        }
    }
    bool buffered = false;
    if constexpr (!ACCUM) buffered = conv_rows_buffered(g, sizeof(T));
    if constexpr (!ACCUM) {
        if (buffered) {
            hipLaunchKernelGGL((dsa3d_dwconv_kernel<T, MIRROR, ACCUM, true>), dim3((unsigned)nblocks), dim3(256), 0,
                               s, reinterpret_cast<const T*>(x), reinterpret_cast<const T*>(w),
                               reinterpret_cast<const T*>(bias), reinterpret_cast<T*>(out), g, run, ngroups);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((dsa3d_dwconv_kernel<T, MIRROR, ACCUM, false>), dim3((unsigned)nblocks), dim3(256), 0, s,
                       reinterpret_cast<const T*>(x), reinterpret_cast<const T*>(w), reinterpret_cast<const T*>(bias),
                       reinterpret_cast<T*>(out), g, run, ngroups);
    return hipGetLastError();
}

}  // namespace

namespace {

// The number of partials of the weight-gradient sums (tiles, or groups of rows).
int64_t wgrad_groups(const dsa3d_desc& d, bool tiled) {
    if (tiled) return conv_tiles(d, true).groups;
    const int64_t rows = d.B * d.T * d.H;
    const int64_t rpg = wgrad_rows_per_group(d);
    return (rows + rpg - 1) / rpg;
}

}  // namespace

size_t dwconv_bwd_workspace_bytes(const dsa3d_desc& d) {
    const int64_t C = (int64_t)d.heads * d.head_dim;
    // sized for either path: which one runs depends on the input's alignment too
    const int64_t groups = std::max(wgrad_groups(d, false), conv_tiled(d, nullptr) ? wgrad_groups(d, true) : 0);
    return (size_t)groups * C * 27 * 4 + 256 + (size_t)groups * C * 4 + 256;
}

hipError_t launch_dwconv_forward(const dsa3d_desc& d, const void* q, const void* w, const void* bias, void* y,
                                 hipStream_t s) {
    if (d.dtype == DSA3D_F32) return conv_launch<float, false, false>(d, q, w, bias, y, DSA3D_K_DWCONV, s);
    return conv_launch<bf16_t, false, false>(d, q, w, bias, y, DSA3D_K_DWCONV, s);
}

hipError_t launch_dwconv_backward(const dsa3d_desc& d, const void* q, const void* w, const void* dy, void* dq,
                                  float* dw, float* db, void* ws, hipStream_t s) {
    const ConvGrid g = conv_grid(d);
    const int64_t rows = (int64_t)g.B * g.T * g.H;
    if (rows == 0 || g.W == 0) return hipSuccess;
    const bool f32 = d.dtype == DSA3D_F32;
    hipError_t e = f32 ? conv_launch<float, true, true>(d, dy, w, nullptr, dq, DSA3D_K_DWCONV_DQ, s)
                       : conv_launch<bf16_t, true, true>(d, dy, w, nullptr, dq, DSA3D_K_DWCONV_DQ, s);
    if (e != hipSuccess) return e;
    const bool tiled = conv_tiled(d, q);
    const int64_t groups = wgrad_groups(d, tiled);
    float* part = reinterpret_cast<float*>(ws);
    float* partb = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                            (((size_t)groups * g.C * 27 * 4 + 255) & ~size_t(255)));
    if (tiled) {
        LaunchScope ls(DSA3D_K_DWCONV_WGRAD, s);
        const ConvTiles ct = conv_tiles(d, true);
        hipLaunchKernelGGL((dsa3d_dwconv_tile_kernel<CT_WGRAD>), dim3((unsigned)(ct.groups * (g.C / 64))), dim3(CT_THREADS),
                           0, s, reinterpret_cast<const bf16_t*>(q), nullptr, nullptr, nullptr,
                           reinterpret_cast<const bf16_t*>(dy), part, partb, g, ct.tc, ct.ntc, ct.nht, ct.nwt);
    } else {
        const int64_t rpg = wgrad_rows_per_group(d);
        LaunchScope ls(DSA3D_K_DWCONV_WGRAD, s);
        dim3 grid((unsigned)(groups * ((g.C + 255) / 256)));
        if (f32)
            hipLaunchKernelGGL((dsa3d_dwconv_wgrad_kernel<float>), grid, dim3(256), 0, s,
                               reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(dy), part, partb, g,
                               rpg);
        else
            hipLaunchKernelGGL((dsa3d_dwconv_wgrad_kernel<bf16_t>), grid, dim3(256), 0, s,
                               reinterpret_cast<const bf16_t*>(q), reinterpret_cast<const bf16_t*>(dy), part, partb, g,
                               rpg);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
    const int64_t nw = g.C * 27;
    hipLaunchKernelGGL(dsa3d_conv_split_sum_kernel, dim3((unsigned)std::min<int64_t>((nw + 255) / 256, 65536)),
                       dim3(256), 0, s, part, dw, nw, groups);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (db) {
        hipLaunchKernelGGL(dsa3d_conv_split_sum_kernel, dim3((unsigned)std::min<int64_t>((g.C + 255) / 256, 65536)),
                           dim3(256), 0, s, partb, db, g.C, groups);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsa3d
