// dsa3d_fixed.hip -- the fixed-window path of 3D-DSA (every offset zero) for gfx950.
//
// With all offsets zero the operator is fixed local attention over the
// dilated k_t x k_h x k_w window around each token [MegaSlide-DiT, §9.1: the
// offset network frozen and every offset set to zero, a fixed (3,7,7)
// window]: each sample lands exactly on its reference token, so its one
// corner has weight 1 and the other seven weight 0. These kernels take that
// case without reading offsets or interpolating: one key row and one value row
// per sample. A reference token outside the grid reads zero rows (logit 0,
// value 0), as in the general path.
//
// The backward needs no sample index: key y is sampled by the queries
// x = y - dil*(i - (k-1)/2) of the window points i, so each key walks its own
// window in reverse and sums its dk, dv terms in the window's fixed order
// (deterministic by construction). The query kernel leaves <dO, o> per task
// in the workspace for the key kernel.
//
// Lane groups (L = head_dim/8 lanes, 8 channels each) and the block order are
// those of the general kernels; a task owns a few neighbouring tokens along w.
// For bf16 rows with an undilated w axis and k_w <= 17 the kernels run on the
// matrix cores instead (the forward for rows of 32-256 channels, the backward
// for 32-128): the queries of a row and their keys form banded dense
// products there.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"
#include "dsa3d_mfma.h"

#include <type_traits>

namespace dsa3d {

struct FixedArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    void* out;
    float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;  // <dO, o> per task, [B,T,H,W,heads]; the matrix-core kernels keep (lse, <dO, o>)
                  // pairs in head-major order, [B,heads,T,H,W], so a row of queries is contiguous
    int32_t group;  // tokens per task along w: kFixedGroup, or 1 with a dilated w axis
    TaskGrid g;
    BlockOrder ord;
    int32_t P;
    float scale;
    Window win;
};

namespace {

struct FixedTask {
    int32_t b, eta, t, h, w;
    int64_t tok;      // flat token index in [B,T,H,W]
    int64_t row_off;  // element offset of the lane's 8 channels in a token's row
    uint32_t tok_b;   // first token of the batch item
};

template <int D>
__device__ __forceinline__ bool fixed_task(const FixedArgs& a, int li, int grp, FixedTask& k) {
    int64_t bh;
    int32_t t, h, w0;
    block_coords(a.g, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, h, w0);
    k.w = w0 + grp;
    if (k.w >= a.g.W) return false;
    k.b = (int32_t)(bh / a.g.nheads);
    k.eta = a.g.head0 + (int32_t)(bh - (int64_t)k.b * a.g.nheads);
    k.t = t;
    k.h = h;
    k.tok_b = (uint32_t)k.b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    k.tok = (int64_t)k.tok_b + ((int64_t)t * a.g.H + h) * a.g.W + k.w;
    k.row_off = (int64_t)k.eta * D + li * 8;
    return true;
}

// Token of window point (it, ih, iw) seen from (t, h, w) with sign +1 (the
// query's samples) or -1 (the queries that sample a key); false outside the grid.
__device__ __forceinline__ bool window_token(const TaskGrid& g, const Window& win, int32_t t, int32_t h, int32_t w,
                                             int it, int ih, int iw, int sign, uint32_t tok_b, uint32_t& tok) {
    const int32_t tt = t + sign * win.dil_t * (it - win.rt);
    const int32_t hh = h + sign * win.dil_h * (ih - win.rh);
    const int32_t ww = w + sign * win.dil_w * (iw - win.rw);
    const bool in = (uint32_t)tt < (uint32_t)g.T && (uint32_t)hh < (uint32_t)g.H && (uint32_t)ww < (uint32_t)g.W;
    tok = tok_b + ((uint32_t)tt * (uint32_t)g.H + (uint32_t)hh) * (uint32_t)g.W + (uint32_t)ww;
    return in;
}

}  // namespace

// A task owns Q neighbouring tokens along w (Q = 4 when the window is not
// dilated along w, else 1). The Q queries' windows overlap in all but Q - 1
// of their columns: for each (frame, row) of the window the task walks the
// Q + k_w - 1 columns once, loads each column token's rows once and updates
// every query whose window holds that column. Each query still takes its
// window points in the window's order (columns left to right), so its
// arithmetic is that of a task of one token.
constexpr int kFixedGroup = 4;

// Forward: one pass over the window with an online softmax per query (as the
// general forward, with one key and one value row per sample).
template <typename T, int D, int Q>
__global__ void __launch_bounds__(256) dsa3d_fixed_fwd_kernel(FixedArgs a) {
    constexpr int L = D / 8;
    const int li = threadIdx.x % L;
    FixedTask k;
    if (!fixed_task<D>(a, li, (threadIdx.x / L) * Q, k)) return;
    const int64_t C = (int64_t)a.g.heads * D;
    const uint64_t row_bytes = (uint64_t)C * sizeof(T);
    const char* Kb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + k.row_off);
    const char* Vb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + k.row_off);
    const char* zero = reinterpret_cast<const char*>(g_zero_row);
    const int nq = min(Q, a.g.W - k.w);  // queries of the task inside the grid
    Frag8<T> qf[Q];
    float m[Q], z[Q], o[Q][8];
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        qf[j].load(reinterpret_cast<const T*>(j < nq ? reinterpret_cast<const char*>(
                                                            reinterpret_cast<const T*>(a.q) + (k.tok + j) * C + k.row_off)
                                                      : zero));
        m[j] = -INFINITY;
        z[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }
    const int ncol = Q + a.win.kw - 1;
    for (int it = 0; it < a.win.kt; ++it)
        for (int ih = 0; ih < a.win.kh; ++ih)
            for (int u = 0; u < ncol; ++u) {
                // column u: window point iw = u - j of query j
                uint32_t tk;
                const bool in = window_token(a.g, a.win, k.t, k.h, k.w, it, ih, u, 1, k.tok_b, tk);
                const uint64_t off = (uint64_t)tk * row_bytes;
                Frag8<T> kf, vf;
                kf.load(reinterpret_cast<const T*>(in ? Kb + off : zero));
                vf.load(reinterpret_cast<const T*>(in ? Vb + off : zero));
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    if (u - j < 0 || u - j >= a.win.kw) continue;
                    const float s = a.scale * group_sum<L>(kf.dot(qf[j], 0.0f));
                    const float m_new = fmaxf(m[j], s);
                    const float alpha = __expf(m[j] - m_new);
                    const float beta = __expf(s - m_new);
                    z[j] = fmaf(z[j], alpha, beta);
                    if (!__all(m_new == m[j])) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
                    }
                    vf.axpy(beta, o[j]);
                    m[j] = m_new;
                }
            }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        if (j >= nq) continue;
        const float inv_z = 1.0f / z[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] *= inv_z;
        Frag8<T> of;
        of.from_f32(o[j]);
        of.store(reinterpret_cast<T*>(a.out) + (k.tok + j) * C + k.row_off);
        if (li == 0) a.lse[(k.tok + j) * a.g.heads + k.eta] = m[j] + __logf(z[j]);
    }
}

// ---------------------------------------------------------------------------
// Forward on the matrix cores: bf16, head_dim a multiple of 32 (up to 256),
// no dilation along w and k_w <= 17.
//
// The 16 tokens w0 .. w0+15 of one row (t, h) of one head share, for each
// (frame, row) of the window, one segment of 15 + k_w consecutive key tokens
// (columns w0 - r_w ...): query c uses segment keys c .. c + k_w - 1, a band.
// A wave takes these 16 queries through the window segment by segment:
//   S^T = K_seg Q^T         two 16-key tiles, head_dim/32 steps of
//                           v_mfma_f32_16x16x32_bf16,
//   logits outside the band -> -inf, online softmax per query,
//   O^T += V_seg^T P^T      one 16-channel tile per product; the weights are
//                           split into a bf16 part and a bf16 remainder (two
//                           products), so they enter at about 2^-17 relative
//                           precision, and everything accumulates in f32.
// The product layouts: lane l holds row l%16 and k-slice 8*(l/16) .. +7 of
// each operand, and D[4*(l/16) + r][l%16] of the result. The k-slice of lane
// group g in the second product is the key set {4g..4g+3, 16+4g..16+4g+3},
// which is where the first product left group g's logits, so the weights
// need no data movement; the segment's value rows pass through LDS, from
// which each lane reads its eight (key, channel) elements. Keys outside the
// grid are zero rows (logit 0, value 0), as in the gathering kernels; keys past
// the segment lie outside every band.
constexpr int kMfmaTokens = 16;  // queries per wave
constexpr int kMfmaMaxKw = 17;   // 15 + k_w keys fit two 16-key tiles
constexpr int kMfmaPairMaxD = 128;  // rows of up to this many channels go two to a wave
constexpr int kMfmaKeyPairMaxD = 64;  // the same for the backward per key (more accumulators)

// One window segment's operands: the two 16-key tiles of keys for the first
// product (key 16*T + l%16, channels 32j + 8*(l/16) .. +7) and this lane's
// part of the value rows on their way to LDS.
template <int D>
struct MfmaSeg {
    mf_bf16x8 k[2][D / 32];
    uint4 v[D / 16];
};

// Staging of a segment's 32 rows (tokens w_first .. w_first + 31 of one
// (frame, row)) into LDS: load i takes rows i*(512/D) + l/(D/8), lane l
// reading the 16 bytes at channel 8*(l%(D/8)), so the lanes of one row read it
// whole and in order and a load touches only full cache lines. The loads go
// through a buffer resource spanning the grid row (no records when the row lies
// outside the grid), and a row outside the segment or the grid gets an offset
// past the records: either way the hardware returns zeros. Which rows lie in
// the segment and the grid does not change along the window, so a lane's
// offsets are fixed. (A grid row of the head-interleaved tensor must stay
// below 2 GiB, the records limit.)
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 buffer resource: untyped 32-bit data format
constexpr uint32_t kPastRecords = 0x80000000u;

template <int D>
struct SegStage {
    static constexpr int kLanes = D / 8;       // lanes per row
    static constexpr int kRows = 64 / kLanes;  // rows per load
    static constexpr int kLoads = D / 16;      // loads per segment
    static constexpr bool kTable = kLoads <= 8;  // offsets kept in registers (else formed per load)
    int lds;                            // LDS element offset of this lane's 16 bytes in load 0
    uint32_t off[kTable ? kLoads : 1];  // byte offset of load i from the segment row's first token
    uint32_t off0, step, ok;            // the same formed per load: load 0's row (mod 2^32), step, bit i = in
    int32_t nrec;                       // bytes of a grid row
    __device__ SegStage(int lane, int32_t w_first, int span, int32_t W, int64_t C, int RS) {
        const int row = lane / kLanes, ch = 8 * (lane % kLanes);
        lds = row * RS + ch;
        off0 = (uint32_t)(((int64_t)(w_first + row) * C + ch) * 2);
        step = (uint32_t)(kRows * C * 2);
        nrec = (int32_t)((int64_t)W * C * 2);
        ok = 0;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = i * kRows + row;
            const bool in = r < span && (uint32_t)(w_first + r) < (uint32_t)W;
            ok |= (uint32_t)in << i;
            if constexpr (kTable) off[i] = in ? off0 + (uint32_t)i * step : kPastRecords;
        }
    }
    // the resource of the grid row starting at `rowp` (its first token, this head)
    __device__ __amdgpu_buffer_rsrc_t rsrc(const bf16_t* rowp, bool in_grid) const {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(rowp), (short)0, in_grid ? nrec : 0,
                                                 kRawBufferWord3);
    }
    __device__ uint4 load(__amdgpu_buffer_rsrc_t r, int i) const {
        uint32_t o;
        if constexpr (kTable) o = off[i];
        else o = ((ok >> i) & 1u) ? off0 + (uint32_t)i * step : kPastRecords;
        const mf_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
        return uint4{v[0], v[1], v[2], v[3]};
    }
    __device__ void put(bf16_t* s, int RS, int i, const uint4& x) const {
        *reinterpret_cast<uint4*>(s + lds + i * kRows * RS) = x;
    }
};

// A wave takes R rows h .. h+R-1 of 16 tokens (R = 2 when the window is not
// dilated along h and rows have at most 128 channels, else 1). The rows' windows share all but R - 1 of their
// (frame, row) segments, so the wave walks the union once: each segment's
// keys and values are loaded once, and the value fragments read from LDS once,
// for every row whose window holds the segment.
template <int D, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
dsa3d_fixed_fwd_mfma_kernel(FixedArgs a) {
    constexpr int RS = D + 8;  // LDS row stride (elements): the four lane groups' rows fall in distinct banks
    __shared__ __attribute__((aligned(16))) bf16_t s_v[4][32 * RS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    int64_t bh;
    int32_t t, hr, bw0;
    TaskGrid gr = a.g;
    gr.H = (a.g.H + R - 1) / R;  // the block order walks groups of R rows
    block_coords(gr, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, hr, bw0);
    const int32_t h = R * hr;
    const int32_t w0 = bw0 + wv * kMfmaTokens;
    if (w0 >= a.g.W) return;  // no block-wide barrier below
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int64_t C = (int64_t)a.g.heads * D;
    const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + (int64_t)eta * D;
    const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + (int64_t)eta * D;
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);  // 512 zero elements
    bf16_t* vs = s_v[wv];
    bool qin[R];
    int64_t qtok[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        qin[rho] = w0 + c < a.g.W && h + rho < a.g.H;
        qtok[rho] = (int64_t)tok_b + ((int64_t)t * a.g.H + h + rho) * a.g.W + (w0 + c);
    }

    // This lane's key columns (the same in every segment) and whether they lie
    // in the grid and the segment: keys c and 16 + c of the first product; the
    // value rows are staged whole.
    const int span = kMfmaTokens - 1 + a.win.kw;
    const int32_t wk0 = w0 - a.win.rw + c, wk1 = wk0 + 16;
    const bool ok0 = c < span && (uint32_t)wk0 < (uint32_t)a.g.W;
    const bool ok1 = 16 + c < span && (uint32_t)wk1 < (uint32_t)a.g.W;
    const int64_t ko0 = (int64_t)wk0 * C + 8 * g, ko1 = (int64_t)wk1 * C + 8 * g;
    const SegStage<D> vst(lane, w0 - a.win.rw, span, a.g.W, C, RS);
    const int nu = a.win.kh + R - 1;  // segment rows of the union per frame

    // Q as the second operand of the first product: query c, channels 32j + 8g .. +7
    mf_bf16x8 qb[R][D / 32];
    mf_f32x4 oacc[R][D / 32][2];  // O^T rows 4g + r of tile (tau, par): channel 32*tau + 8g + 2r + par, query c
    float m[R], lsum[R];          // maximum in use (query c) and this lane's share of the denominator
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
            qb[rho][j] = *reinterpret_cast<const mf_bf16x8*>(
                qin[rho] ? reinterpret_cast<const bf16_t*>(a.q) + qtok[rho] * C + (int64_t)eta * D + 32 * j + 8 * g
                         : zero);
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau) oacc[rho][tau][0] = oacc[rho][tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
        m[rho] = -INFINITY;
        lsum[rho] = 0.0f;
    }

    for (int it = 0; it < a.win.kt; ++it) {
        const int32_t tt = t + a.win.dil_t * (it - a.win.rt);
        for (int u = 0; u < nu; ++u) {
            // segment row: window row u - rho of row rho
            const int32_t hh = R == 1 ? h + a.win.dil_h * (u - a.win.rh) : h - a.win.rh + u;
            const bool rin = (uint32_t)tt < (uint32_t)a.g.T && (uint32_t)hh < (uint32_t)a.g.H;
            const int64_t rb = rin ? ((int64_t)tok_b + ((int64_t)tt * a.g.H + hh) * a.g.W) * C : 0;
            // a key outside the grid reads the zero row (offsets below stay within its 512 elements)
            const bf16_t* p0 = rin && ok0 ? K + rb + ko0 : zero;
            const bf16_t* p1 = rin && ok1 ? K + rb + ko1 : zero;
            MfmaSeg<D> cur;
#pragma unroll
            for (int j = 0; j < D / 32; ++j) {
                cur.k[0][j] = *reinterpret_cast<const mf_bf16x8*>(p0 + 32 * j);
                cur.k[1][j] = *reinterpret_cast<const mf_bf16x8*>(p1 + 32 * j);
            }
            const __amdgpu_buffer_rsrc_t vr = vst.rsrc(V + rb, rin);
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc) cur.v[pc] = vst.load(vr, pc);
            wave_lds_sync();  // the previous segment's values have been read
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc)
                vst.put(vs, RS, pc, cur.v[pc]);
            bool use[R];
            mf_bf16x8 pb_hi[R], pb_lo[R];
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                use[rho] = u - rho >= 0 && u - rho < a.win.kh;  // wave-uniform
                if (!use[rho]) continue;
                // S^T for keys 16*T + 4g + r of the segment, query c of row rho
                mf_f32x4 sacc[2];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    sacc[T] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < D / 32; ++j)
                        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[T][j], qb[rho][j], sacc[T], 0, 0, 0);
                }
                // softmax of query c over its band: keys c .. c + k_w - 1
                float sv[8];
                float mloc = -INFINITY;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kc = 16 * (i >> 2) + 4 * g + (i & 3);
                    sv[i] = (uint32_t)(kc - c) < (uint32_t)a.win.kw ? a.scale * sacc[i >> 2][i & 3] : -INFINITY;
                    mloc = fmaxf(mloc, sv[i]);
                }
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
                if (!__all(mloc <= m[rho] + kMfmaLazyMax)) {  // always on the row's first segment (m = -inf)
                    const float m_new = fmaxf(m[rho], mloc);
                    const float alpha = __expf(m[rho] - m_new);
#pragma unroll
                    for (int tau = 0; tau < D / 32; ++tau) {
                        oacc[rho][tau][0] *= alpha;
                        oacc[rho][tau][1] *= alpha;
                    }
                    lsum[rho] *= alpha;
                    m[rho] = m_new;
                }
                // weights as a bf16 part and a bf16 remainder, in the second product's k order
                mf_u32x4 phi, plo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float q0 = __expf(sv[2 * i] - m[rho]), q1 = __expf(sv[2 * i + 1] - m[rho]);
                    lsum[rho] += q0 + q1;
                    const uint32_t hw = mf_pack(q0, q1);
                    phi[i] = hw;
                    plo[i] = mf_pack(q0 - bf16_lo(hw), q1 - bf16_hi(hw));
                }
                pb_hi[rho] = __builtin_bit_cast(mf_bf16x8, phi);
                pb_lo[rho] = __builtin_bit_cast(mf_bf16x8, plo);
            }
            wave_lds_sync();  // the segment's values are in LDS
            // O^T += V^T P^T over tiles of 16 channels 32*tau + 2m + par (m = 0..15):
            // one 32-bit LDS read gives a key's channel pair for the tiles
            // (tau, 0) and (tau, 1). Element 8g + i of the k-slice is key 4g + i
            // (i < 4) or 16 + 4g + i - 4.
#pragma unroll
            for (int tau = 0; tau < D / 32; ++tau) {
                const bf16_t* col = vs + 32 * tau + 2 * c;
                uint32_t d[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = i < 4 ? 4 * g + i : 12 + 4 * g + i;
                    d[i] = *reinterpret_cast<const uint32_t*>(col + key * RS);
                }
                mf_u32x4 ve, vo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ve[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x05040100u);  // even channels of keys 2i, 2i+1
                    vo[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07060302u);  // odd channels
                }
                const mf_bf16x8 vE = __builtin_bit_cast(mf_bf16x8, ve), vO = __builtin_bit_cast(mf_bf16x8, vo);
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    if (!use[rho]) continue;
                    oacc[rho][tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vE, pb_hi[rho], oacc[rho][tau][0], 0, 0, 0);
                    oacc[rho][tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vE, pb_lo[rho], oacc[rho][tau][0], 0, 0, 0);
                    oacc[rho][tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vO, pb_hi[rho], oacc[rho][tau][1], 0, 0, 0);
                    oacc[rho][tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vO, pb_lo[rho], oacc[rho][tau][1], 0, 0, 0);
                }
            }
        }
    }

#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        float l = lsum[rho];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (!qin[rho]) continue;
        const float inv = 1.0f / l;
        bf16_t* orow = reinterpret_cast<bf16_t*>(a.out) + qtok[rho] * C + (int64_t)eta * D;
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau) {  // channels 32*tau + 8g .. +7 of query c
            const mf_f32x4& e = oacc[rho][tau][0];
            const mf_f32x4& o = oacc[rho][tau][1];
            uint4 w;
            w.x = mf_pack(e[0] * inv, o[0] * inv);
            w.y = mf_pack(e[1] * inv, o[1] * inv);
            w.z = mf_pack(e[2] * inv, o[2] * inv);
            w.w = mf_pack(e[3] * inv, o[3] * inv);
            *reinterpret_cast<uint4*>(orow + 32 * tau + 8 * g) = w;
        }
        if (g == 0) a.lse[qtok[rho] * a.g.heads + eta] = m[rho] + __logf(l);
    }
}

// Backward per query on the matrix cores (same shapes and layout as the
// forward above): for each segment of the union of the R rows' windows,
//   S^T  = K_seg Q^T,  dP^T = V_seg dO^T      (keys x queries, as in the forward)
//   P    = exp(scale*S - lse),  dS = P (dP - <dO, o>)   (band keys only)
//   dq^T += K_seg^T (scale*dS)^T              (weights split into a bf16 part
//                                              and a bf16 remainder)
// The segment's keys pass through LDS once and serve both as the first
// product's operand (16-byte reads) and, read a channel pair at a time, as
// the third's; the values are the second product's operand, loaded directly.
// <dO, o> is left in the workspace for the key kernel, as by the vector kernel.
template <int D, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
dsa3d_fixed_bwd_query_mfma_kernel(FixedArgs a) {
    constexpr int RS = D + 8;  // LDS row stride (elements), as in the forward
    __shared__ __attribute__((aligned(16))) bf16_t s_k[4][32 * RS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    int64_t bh;
    int32_t t, hr, bw0;
    TaskGrid gr = a.g;
    gr.H = (a.g.H + R - 1) / R;
    block_coords(gr, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, hr, bw0);
    const int32_t h = R * hr;
    const int32_t w0 = bw0 + wv * kMfmaTokens;
    if (w0 >= a.g.W) return;  // no block-wide barrier below
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int64_t thw = (int64_t)a.g.T * a.g.H * a.g.W;
    const int64_t C = (int64_t)a.g.heads * D;
    const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + (int64_t)eta * D;
    const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + (int64_t)eta * D;
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);  // 512 zero elements
    bf16_t* ks = s_k[wv];

    const int span = kMfmaTokens - 1 + a.win.kw;
    const int32_t wk0 = w0 - a.win.rw + c, wk1 = wk0 + 16;
    const bool ok0 = c < span && (uint32_t)wk0 < (uint32_t)a.g.W;
    const bool ok1 = 16 + c < span && (uint32_t)wk1 < (uint32_t)a.g.W;
    const int64_t ko0 = (int64_t)wk0 * C + 8 * g, ko1 = (int64_t)wk1 * C + 8 * g;
    const SegStage<D> kst_map(lane, w0 - a.win.rw, span, a.g.W, C, RS);
    const int nu = a.win.kh + R - 1;

    bool qin[R];
    int64_t qtok[R];
    mf_bf16x8 qb[R][D / 32], gb[R][D / 32];  // Q and dO as second operands: query c, channels 32j + 8g .. +7
    mf_f32x4 dacc[R][D / 32][2];             // dq^T rows 4g + r of tile (tau, par): channel 32*tau + 8g + 2r + par
    float lse[R], dsum[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        qin[rho] = w0 + c < a.g.W && h + rho < a.g.H;
        qtok[rho] = (int64_t)tok_b + ((int64_t)t * a.g.H + h + rho) * a.g.W + (w0 + c);
        const int64_t ro = qtok[rho] * C + (int64_t)eta * D + 8 * g;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
            const bf16_t* qp = qin[rho] ? reinterpret_cast<const bf16_t*>(a.q) + ro + 32 * j : zero;
            const bf16_t* gp = qin[rho] ? reinterpret_cast<const bf16_t*>(a.dout) + ro + 32 * j : zero;
            const bf16_t* op = qin[rho] ? reinterpret_cast<const bf16_t*>(a.o) + ro + 32 * j : zero;
            qb[rho][j] = *reinterpret_cast<const mf_bf16x8*>(qp);
            gb[rho][j] = *reinterpret_cast<const mf_bf16x8*>(gp);
            const uint4 gw = *reinterpret_cast<const uint4*>(gp), ow = *reinterpret_cast<const uint4*>(op);
            part = dot2_bf16(gw.x, ow.x, part);
            part = dot2_bf16(gw.y, ow.y, part);
            part = dot2_bf16(gw.z, ow.z, part);
            part = dot2_bf16(gw.w, ow.w, part);
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        dsum[rho] = part;
        lse[rho] = qin[rho] ? a.lse[qtok[rho] * a.g.heads + eta] : 0.0f;
        if (qin[rho] && g == 0)
            reinterpret_cast<float2*>(a.dsum)[((int64_t)b * a.g.heads + eta) * thw + (qtok[rho] - tok_b)] =
                make_float2(lse[rho], part);
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau) dacc[rho][tau][0] = dacc[rho][tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int it = 0; it < a.win.kt; ++it) {
        const int32_t tt = t + a.win.dil_t * (it - a.win.rt);
        for (int u = 0; u < nu; ++u) {
            const int32_t hh = R == 1 ? h + a.win.dil_h * (u - a.win.rh) : h - a.win.rh + u;
            const bool rin = (uint32_t)tt < (uint32_t)a.g.T && (uint32_t)hh < (uint32_t)a.g.H;
            const int64_t rb = rin ? ((int64_t)tok_b + ((int64_t)tt * a.g.H + hh) * a.g.W) * C : 0;
            const bf16_t* p0 = rin && ok0 ? V + rb + ko0 : zero;
            const bf16_t* p1 = rin && ok1 ? V + rb + ko1 : zero;
            mf_bf16x8 va[2][D / 32];  // values as the second product's first operand
            uint4 kst[D / 16];        // this lane's part of the key rows, on their way to LDS
#pragma unroll
            for (int j = 0; j < D / 32; ++j) {
                va[0][j] = *reinterpret_cast<const mf_bf16x8*>(p0 + 32 * j);
                va[1][j] = *reinterpret_cast<const mf_bf16x8*>(p1 + 32 * j);
            }
            const __amdgpu_buffer_rsrc_t kr = kst_map.rsrc(K + rb, rin);
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc) kst[pc] = kst_map.load(kr, pc);
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc)
                kst_map.put(ks, RS, pc, kst[pc]);
            wave_lds_sync();  // the segment's keys are in LDS
            mf_bf16x8 ka[2][D / 32];  // keys as the first product's first operand: key 16T + c, channels 32j + 8g
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int j = 0; j < D / 32; ++j)
                    ka[T][j] = *reinterpret_cast<const mf_bf16x8*>(ks + (16 * T + c) * RS + 32 * j + 8 * g);
            bool use[R];
            mf_bf16x8 ds_hi[R], ds_lo[R];
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                use[rho] = u - rho >= 0 && u - rho < a.win.kh;  // wave-uniform
                if (!use[rho]) continue;
                mf_f32x4 sacc[2], pacc[2];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    sacc[T] = pacc[T] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < D / 32; ++j) {
                        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[T][j], qb[rho][j], sacc[T], 0, 0, 0);
                        pacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[T][j], gb[rho][j], pacc[T], 0, 0, 0);
                    }
                }
                mf_u32x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int ii = 2 * i + e;
                        const int kc = 16 * (ii >> 2) + 4 * g + (ii & 3);
                        const bool band = (uint32_t)(kc - c) < (uint32_t)a.win.kw;
                        const float p = __expf(a.scale * sacc[ii >> 2][ii & 3] - lse[rho]);
                        x[e] = band ? a.scale * p * (pacc[ii >> 2][ii & 3] - dsum[rho]) : 0.0f;
                    }
                    const uint32_t hw = mf_pack(x[0], x[1]);
                    hi[i] = hw;
                    lo[i] = mf_pack(x[0] - bf16_lo(hw), x[1] - bf16_hi(hw));
                }
                ds_hi[rho] = __builtin_bit_cast(mf_bf16x8, hi);
                ds_lo[rho] = __builtin_bit_cast(mf_bf16x8, lo);
            }
            // dq^T += K^T (scale dS)^T, the keys read a channel pair at a time (as the forward's values)
#pragma unroll
            for (int tau = 0; tau < D / 32; ++tau) {
                const bf16_t* col = ks + 32 * tau + 2 * c;
                uint32_t d[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = i < 4 ? 4 * g + i : 12 + 4 * g + i;
                    d[i] = *reinterpret_cast<const uint32_t*>(col + key * RS);
                }
                mf_u32x4 ke, ko;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ke[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x05040100u);
                    ko[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07060302u);
                }
                const mf_bf16x8 kE = __builtin_bit_cast(mf_bf16x8, ke), kO = __builtin_bit_cast(mf_bf16x8, ko);
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    if (!use[rho]) continue;
                    dacc[rho][tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kE, ds_hi[rho], dacc[rho][tau][0], 0, 0, 0);
                    dacc[rho][tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kE, ds_lo[rho], dacc[rho][tau][0], 0, 0, 0);
                    dacc[rho][tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kO, ds_hi[rho], dacc[rho][tau][1], 0, 0, 0);
                    dacc[rho][tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kO, ds_lo[rho], dacc[rho][tau][1], 0, 0, 0);
                }
            }
            wave_lds_sync();  // the segment's keys have been read before the next segment writes them
        }
    }

#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        if (!qin[rho]) continue;
        bf16_t* drow = reinterpret_cast<bf16_t*>(a.dq) + qtok[rho] * C + (int64_t)eta * D;
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau) {  // channels 32*tau + 8g .. +7 of query c
            const mf_f32x4& e = dacc[rho][tau][0];
            const mf_f32x4& o = dacc[rho][tau][1];
            uint4 w;
            w.x = mf_pack(e[0], o[0]);
            w.y = mf_pack(e[1], o[1]);
            w.z = mf_pack(e[2], o[2]);
            w.w = mf_pack(e[3], o[3]);
            *reinterpret_cast<uint4*>(drow + 32 * tau + 8 * g) = w;
        }
    }
}

// Backward per key on the matrix cores (bf16 rows of 32-128 channels, an
// undilated w axis, k_w <= 17). The window is symmetric, so the queries
// that sample the 16 keys w0 .. w0+15 of a row lie, frame by frame and row by
// row, in the same segments of 15 + k_w tokens as the forward's keys, with
// the same band: query slot j of a segment samples key c when 0 <= j - c < k_w.
// A wave takes R rows of 16 keys (R = 2 when h is not dilated) and walks the
// union of their segments; with the segment's queries and output gradients
// staged in LDS:
//   S^T  = Q_seg K^T,  dP^T = dO_seg V^T     (queries x keys)
//   P    = exp(scale*S - lse_q),  dS = P (dP - <dO, o>_q)  (band, queries in the grid)
//   dv^T += dO_seg^T P^T,  dk^T += Q_seg^T (scale*dS)^T   (weights split into a
//                                                          bf16 part and remainder)
// A query outside the grid does not exist, so it contributes nothing (its
// weights are zero); a key's sums run over its window in a fixed order.
template <int D, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
dsa3d_fixed_bwd_key_mfma_kernel(FixedArgs a) {
    constexpr int RS = D + 8;  // LDS row stride (elements), as in the forward
    __shared__ __attribute__((aligned(16))) bf16_t s_q[4][32 * RS];
    __shared__ __attribute__((aligned(16))) bf16_t s_g[4][32 * RS];
    __shared__ float s_st[4][2][32];  // lse and <dO, o> of the segment's queries (0 outside the grid)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    int64_t bh;
    int32_t t, hr, bw0;
    TaskGrid gr = a.g;
    gr.H = (a.g.H + R - 1) / R;
    block_coords(gr, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, hr, bw0);
    const int32_t h = R * hr;
    const int32_t w0 = bw0 + wv * kMfmaTokens;
    if (w0 >= a.g.W) return;  // no block-wide barrier below
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int64_t thw = (int64_t)a.g.T * a.g.H * a.g.W;
    const float2* stats = reinterpret_cast<const float2*>(a.dsum) + ((int64_t)b * a.g.heads + eta) * thw;
    const int64_t C = (int64_t)a.g.heads * D;
    const bf16_t* Qp = reinterpret_cast<const bf16_t*>(a.q) + (int64_t)eta * D;
    const bf16_t* Gp = reinterpret_cast<const bf16_t*>(a.dout) + (int64_t)eta * D;
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);  // 512 zero elements
    bf16_t* qs = s_q[wv];
    bf16_t* gs = s_g[wv];
    float* st_lse = s_st[wv][0];
    float* st_ds = s_st[wv][1];

    const int span = kMfmaTokens - 1 + a.win.kw;
    const SegStage<D> qst_map(lane, w0 - a.win.rw, span, a.g.W, C, RS);  // the segment's queries
    const int32_t wst = w0 - a.win.rw + (lane & 31);  // query column whose statistics this lane stages
    const bool okst = (lane & 31) < span && (uint32_t)wst < (uint32_t)a.g.W;
    const int nu = a.win.kh + R - 1;

    bool kin[R];
    int64_t ktok[R];
    mf_bf16x8 kb[R][D / 32], vb[R][D / 32];  // own keys and values as second operands: key c, channels 32j + 8g
    mf_f32x4 dk[R][D / 32][2], dv[R][D / 32][2];  // rows 4g + r of tile (tau, par): channel 32*tau + 16*par + 4g + r
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        kin[rho] = w0 + c < a.g.W && h + rho < a.g.H;
        ktok[rho] = (int64_t)tok_b + ((int64_t)t * a.g.H + h + rho) * a.g.W + (w0 + c);
        const int64_t ro = ktok[rho] * C + (int64_t)eta * D + 8 * g;
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
            kb[rho][j] = *reinterpret_cast<const mf_bf16x8*>(
                kin[rho] ? reinterpret_cast<const bf16_t*>(a.k) + ro + 32 * j : zero);
            vb[rho][j] = *reinterpret_cast<const mf_bf16x8*>(
                kin[rho] ? reinterpret_cast<const bf16_t*>(a.v) + ro + 32 * j : zero);
        }
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau)
            dk[rho][tau][0] = dk[rho][tau][1] = dv[rho][tau][0] = dv[rho][tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int it = 0; it < a.win.kt; ++it) {
        const int32_t tt = t + a.win.dil_t * (it - a.win.rt);
        for (int u = 0; u < nu; ++u) {
            const int32_t hh = R == 1 ? h + a.win.dil_h * (u - a.win.rh) : h - a.win.rh + u;
            const bool rin = (uint32_t)tt < (uint32_t)a.g.T && (uint32_t)hh < (uint32_t)a.g.H;
            const int64_t rtok = (int64_t)tok_b + ((int64_t)tt * a.g.H + hh) * a.g.W;
            const int64_t rb = rin ? rtok * C : 0;
            const __amdgpu_buffer_rsrc_t qr = qst_map.rsrc(Qp + rb, rin), gres = qst_map.rsrc(Gp + rb, rin);
            uint4 qst[D / 16], gst[D / 16];
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc) {
                qst[pc] = qst_map.load(qr, pc);
                gst[pc] = qst_map.load(gres, pc);
            }
            const bool sin = rin && okst;
            const float2 sq = sin ? stats[rtok - tok_b + wst] : make_float2(0.0f, 0.0f);  // (lse, <dO, o>)
#pragma unroll
            for (int pc = 0; pc < D / 16; ++pc) {
                qst_map.put(qs, RS, pc, qst[pc]);
                qst_map.put(gs, RS, pc, gst[pc]);
            }
            if (lane < 32) {
                st_lse[lane] = sq.x;
                st_ds[lane] = sq.y;
            }
            wave_lds_sync();  // the segment's queries are in LDS
            // first operands: query 16T + c, channels 32j + 8g
            mf_bf16x8 qa[2][D / 32], ga[2][D / 32];
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int j = 0; j < D / 32; ++j) {
                    qa[T][j] = *reinterpret_cast<const mf_bf16x8*>(qs + (16 * T + c) * RS + 32 * j + 8 * g);
                    ga[T][j] = *reinterpret_cast<const mf_bf16x8*>(gs + (16 * T + c) * RS + 32 * j + 8 * g);
                }
            // statistics of this lane's queries 16T + 4g + r, and whether they lie in the grid
            float ql[8], qd[8];
            bool qok[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int qc = 16 * (i >> 2) + 4 * g + (i & 3);
                ql[i] = st_lse[qc];
                qd[i] = st_ds[qc];
                qok[i] = rin && qc < span && (uint32_t)(w0 - a.win.rw + qc) < (uint32_t)a.g.W;
            }
            bool use[R];
            mf_bf16x8 p_hi[R], p_lo[R], s_hi[R], s_lo[R];
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                use[rho] = u - rho >= 0 && u - rho < a.win.kh;  // wave-uniform
                if (!use[rho]) continue;
                mf_f32x4 sacc[2], pacc[2];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    sacc[T] = pacc[T] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < D / 32; ++j) {
                        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[T][j], kb[rho][j], sacc[T], 0, 0, 0);
                        pacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[T][j], vb[rho][j], pacc[T], 0, 0, 0);
                    }
                }
                mf_u32x4 ph, pl, sh, sl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float pw[2], dw[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int ii = 2 * i + e;
                        const int qc = 16 * (ii >> 2) + 4 * g + (ii & 3);
                        const bool band = qok[ii] && (uint32_t)(qc - c) < (uint32_t)a.win.kw;
                        const float p = band ? __expf(a.scale * sacc[ii >> 2][ii & 3] - ql[ii]) : 0.0f;
                        pw[e] = p;
                        dw[e] = a.scale * p * (pacc[ii >> 2][ii & 3] - qd[ii]);
                    }
                    const uint32_t hp = mf_pack(pw[0], pw[1]), hs = mf_pack(dw[0], dw[1]);
                    ph[i] = hp;
                    pl[i] = mf_pack(pw[0] - bf16_lo(hp), pw[1] - bf16_hi(hp));
                    sh[i] = hs;
                    sl[i] = mf_pack(dw[0] - bf16_lo(hs), dw[1] - bf16_hi(hs));
                }
                p_hi[rho] = __builtin_bit_cast(mf_bf16x8, ph);
                p_lo[rho] = __builtin_bit_cast(mf_bf16x8, pl);
                s_hi[rho] = __builtin_bit_cast(mf_bf16x8, sh);
                s_lo[rho] = __builtin_bit_cast(mf_bf16x8, sl);
            }
            // dv^T += dO^T P^T and dk^T += Q^T (scale dS)^T on tiles of 16 channels (tile (tau, par):
            // channels 32*tau + 16*par ..), the first operands read with the transposing LDS read: lane
            // c of block g receives channel c of the four queries 4g .. 4g+3, then of 16+4g .. 16+4g+3
#pragma unroll
            for (int tau = 0; tau < D / 32; ++tau) {
#pragma unroll
                for (int par = 0; par < 2; ++par) {
                    const int toff = (4 * g + (c >> 2)) * RS + 32 * tau + 16 * par + 4 * (c & 3);
                    const mf_bf16x8 qA = mf_read_tr8(qs + toff, 16 * RS), gA = mf_read_tr8(gs + toff, 16 * RS);
#pragma unroll
                    for (int rho = 0; rho < R; ++rho) {
                        if (!use[rho]) continue;
                        dv[rho][tau][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gA, p_hi[rho], dv[rho][tau][par], 0, 0, 0);
                        dv[rho][tau][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gA, p_lo[rho], dv[rho][tau][par], 0, 0, 0);
                        dk[rho][tau][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qA, s_hi[rho], dk[rho][tau][par], 0, 0, 0);
                        dk[rho][tau][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qA, s_lo[rho], dk[rho][tau][par], 0, 0, 0);
                    }
                }
            }
            wave_lds_sync();  // the segment's queries have been read before the next segment writes them
        }
    }

#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        if (!kin[rho]) continue;
        bf16_t* krow = reinterpret_cast<bf16_t*>(a.dk) + ktok[rho] * C + (int64_t)eta * D;
        bf16_t* vrow = reinterpret_cast<bf16_t*>(a.dv) + ktok[rho] * C + (int64_t)eta * D;
#pragma unroll
        for (int tau = 0; tau < D / 32; ++tau)
#pragma unroll
            for (int par = 0; par < 2; ++par) {  // channels 32*tau + 16*par + 4g .. +3 of key c
                const mf_f32x4& k4 = dk[rho][tau][par];
                const mf_f32x4& v4 = dv[rho][tau][par];
                *reinterpret_cast<uint2*>(krow + 32 * tau + 16 * par + 4 * g) =
                    make_uint2(mf_pack(k4[0], k4[1]), mf_pack(k4[2], k4[3]));
                *reinterpret_cast<uint2*>(vrow + 32 * tau + 16 * par + 4 * g) =
                    make_uint2(mf_pack(v4[0], v4[1]), mf_pack(v4[2], v4[3]));
            }
    }
}

// Backward per query: a_p = exp(s_p - lse), ds_p = a_p (<dO, V[p]> - <dO, o>),
// dq = scale * sum_p ds_p K[p]; <dO, o> is kept for the key kernel.
template <typename T, int D, int Q>
__global__ void __launch_bounds__(256) dsa3d_fixed_bwd_query_kernel(FixedArgs a) {
    constexpr int L = D / 8;
    const int li = threadIdx.x % L;
    FixedTask k;
    if (!fixed_task<D>(a, li, (threadIdx.x / L) * Q, k)) return;
    const int64_t C = (int64_t)a.g.heads * D;
    const uint64_t row_bytes = (uint64_t)C * sizeof(T);
    const char* Kb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + k.row_off);
    const char* Vb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + k.row_off);
    const char* zero = reinterpret_cast<const char*>(g_zero_row);
    const int nq = min(Q, a.g.W - k.w);
    Frag8<T> qf[Q], gf[Q];
    float Dsum[Q], lse[Q], dq[Q][8];
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const bool ok = j < nq;
        const int64_t rj = (k.tok + j) * C + k.row_off;
        Frag8<T> of;
        qf[j].load(reinterpret_cast<const T*>(ok ? reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + rj) : zero));
        gf[j].load(reinterpret_cast<const T*>(ok ? reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + rj) : zero));
        of.load(reinterpret_cast<const T*>(ok ? reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.o) + rj) : zero));
        Dsum[j] = group_sum<L>(gf[j].dot(of, 0.0f));
        const int64_t ti = (k.tok + (ok ? j : 0)) * a.g.heads + k.eta;
        lse[j] = ok ? a.lse[ti] : 0.0f;
        if (ok && li == 0) a.dsum[ti] = Dsum[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) dq[j][e] = 0.f;
    }
    const int ncol = Q + a.win.kw - 1;
    for (int it = 0; it < a.win.kt; ++it)
        for (int ih = 0; ih < a.win.kh; ++ih)
            for (int u = 0; u < ncol; ++u) {
                uint32_t tk;
                const bool in = window_token(a.g, a.win, k.t, k.h, k.w, it, ih, u, 1, k.tok_b, tk);
                const uint64_t off = (uint64_t)tk * row_bytes;
                Frag8<T> kf, vf;
                kf.load(reinterpret_cast<const T*>(in ? Kb + off : zero));
                vf.load(reinterpret_cast<const T*>(in ? Vb + off : zero));
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    if (u - j < 0 || u - j >= a.win.kw) continue;
                    const float qk = group_sum<L>(kf.dot(qf[j], 0.0f));
                    const float da = group_sum<L>(vf.dot(gf[j], 0.0f));
                    const float ap = __expf(a.scale * qk - lse[j]);
                    const float ds = ap * (da - Dsum[j]);
                    kf.axpy(a.scale * ds, dq[j]);  // the general path's arithmetic at zero offsets
                }
            }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        if (j >= nq) continue;
        Frag8<T> dqf;
        dqf.from_f32(dq[j]);
        dqf.store(reinterpret_cast<T*>(a.dq) + (k.tok + j) * C + k.row_off);
    }
}

// Backward per key y: the queries x = y - dil*(i - r) of the window points i
// (in the window's order) add scale*ds_{x,i} q_x to dk and a_{x,i} dO_x to dv.
// A query outside the grid reads zero rows and lse = <dO,o> = 0, so its terms
// are exactly zero. The Q keys of a task share the query columns; columns are
// walked right to left, so that each key takes its window points in order.
template <typename T, int D, int Q>
__global__ void __launch_bounds__(256) dsa3d_fixed_bwd_key_kernel(FixedArgs a) {
    constexpr int L = D / 8;
    const int li = threadIdx.x % L;
    FixedTask k;
    if (!fixed_task<D>(a, li, (threadIdx.x / L) * Q, k)) return;
    const int64_t C = (int64_t)a.g.heads * D;
    const uint64_t row_bytes = (uint64_t)C * sizeof(T);
    const char* Qb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + k.row_off);
    const char* Gb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + k.row_off);
    const char* zero = reinterpret_cast<const char*>(g_zero_row);
    const int nq = min(Q, a.g.W - k.w);
    Frag8<T> kf[Q], vf[Q];
    float ak[Q][8], av[Q][8];
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const bool ok = j < nq;
        const int64_t rj = (k.tok + j) * C + k.row_off;
        kf[j].load(reinterpret_cast<const T*>(ok ? reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + rj) : zero));
        vf[j].load(reinterpret_cast<const T*>(ok ? reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + rj) : zero));
#pragma unroll
        for (int e = 0; e < 8; ++e) { ak[j][e] = 0.f; av[j][e] = 0.f; }
    }
    const int ncol = Q + a.win.kw - 1;
    for (int it = 0; it < a.win.kt; ++it)
        for (int ih = 0; ih < a.win.kh; ++ih)
            for (int u = 0; u < ncol; ++u) {
                // query column k.w + Q - 1 - (u - r_w), right to left: window point
                // iw = u - (Q - 1) + j of key j (ascending for every key)
                uint32_t tx;
                const bool in = window_token(a.g, a.win, k.t, k.h, k.w + Q - 1, it, ih, u, -1, k.tok_b, tx);
                const uint64_t off = (uint64_t)tx * row_bytes;
                Frag8<T> qx, gx;
                qx.load(reinterpret_cast<const T*>(in ? Qb + off : zero));
                gx.load(reinterpret_cast<const T*>(in ? Gb + off : zero));
                const int64_t xi = in ? (int64_t)tx * a.g.heads + k.eta : 0;  // in bounds either way
                const float lse = in ? a.lse[xi] : 0.0f;
                const float Dsum = in ? a.dsum[xi] : 0.0f;
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    const int iw = u - (Q - 1) + j;
                    if (iw < 0 || iw >= a.win.kw) continue;
                    const float s = a.scale * group_sum<L>(qx.dot(kf[j], 0.0f));
                    const float da = group_sum<L>(gx.dot(vf[j], 0.0f));
                    const float ap = __expf(s - lse);
                    const float ds = ap * (da - Dsum);
                    qx.axpy(a.scale * ds, ak[j]);
                    gx.axpy(ap, av[j]);
                }
            }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        if (j >= nq) continue;
        Frag8<T> dkf, dvf;
        dkf.from_f32(ak[j]);
        dvf.from_f32(av[j]);
        dkf.store(reinterpret_cast<T*>(a.dk) + (k.tok + j) * C + k.row_off);
        dvf.store(reinterpret_cast<T*>(a.dv) + (k.tok + j) * C + k.row_off);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

FixedArgs fixed_args(const dsa3d_desc& d) {
    FixedArgs a{};
    a.g = make_task_grid(d, 0, d.heads);
    a.P = d.P;
    a.scale = logit_scale(d);
    a.win = make_window(d);
    a.group = d.dil_w == 1 ? kFixedGroup : 1;
    a.ord = make_block_order(d, attn_tokens_per_block(d.head_dim) * a.group, kGatherSupertile, "DSA3D_ORDER_FIXED");
    return a;
}

template <typename T, int D>
hipError_t fixed_fwd_t(const FixedArgs& a, int64_t nb, hipStream_t s) {
    LaunchScope ls(DSA3D_K_FORWARD, s);
    if (a.group == kFixedGroup)
        hipLaunchKernelGGL((dsa3d_fixed_fwd_kernel<T, D, kFixedGroup>), dim3((unsigned)nb), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((dsa3d_fixed_fwd_kernel<T, D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D> hipError_t fixed_fwd_f32(const FixedArgs& a, int64_t nb, hipStream_t s) { return fixed_fwd_t<float, D>(a, nb, s); }
template <int D> hipError_t fixed_fwd_bf16(const FixedArgs& a, int64_t nb, hipStream_t s) { return fixed_fwd_t<bf16_t, D>(a, nb, s); }

// am and ak (the matrix-core query and key kernels' arguments and block
// counts) are null where those kernels do not apply; rows of 256 channels
// keep the vector kernels (the matrix-core ones would not fit their registers).
template <typename T, int D>
hipError_t fixed_bwd_t(const FixedArgs& a, int64_t nb, const FixedArgs* am, int64_t nbm, const FixedArgs* ak,
                       int64_t nbk, hipStream_t s) {
    {
        LaunchScope ls(DSA3D_K_BWD_QUERY, s);
        bool done = false;
        if constexpr (std::is_same<T, bf16_t>::value && D >= 32 && D <= kMfmaPairMaxD) {
            if (am != nullptr) {
                if constexpr (D <= kMfmaPairMaxD) {
                    if (am->win.dil_h == 1) {
                        hipLaunchKernelGGL((dsa3d_fixed_bwd_query_mfma_kernel<D, 2>), dim3((unsigned)nbm), dim3(256), 0,
                                           s, *am);
                        done = true;
                    }
                }
                if (!done) {
                    hipLaunchKernelGGL((dsa3d_fixed_bwd_query_mfma_kernel<D, 1>), dim3((unsigned)nbm), dim3(256), 0, s,
                                       *am);
                    done = true;
                }
            }
        }
        if (!done) {
            if (a.group == kFixedGroup)
                hipLaunchKernelGGL((dsa3d_fixed_bwd_query_kernel<T, D, kFixedGroup>), dim3((unsigned)nb), dim3(256), 0,
                                   s, a);
            else
                hipLaunchKernelGGL((dsa3d_fixed_bwd_query_kernel<T, D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    LaunchScope ls(DSA3D_K_BWD_KEY, s);
    if constexpr (std::is_same<T, bf16_t>::value && D >= 32 && D <= kMfmaPairMaxD) {
        if (ak != nullptr) {
            if constexpr (D <= kMfmaKeyPairMaxD) {
                if (ak->win.dil_h == 1) {
                    hipLaunchKernelGGL((dsa3d_fixed_bwd_key_mfma_kernel<D, 2>), dim3((unsigned)nbk), dim3(256), 0, s,
                                       *ak);
                    return hipGetLastError();
                }
            }
            hipLaunchKernelGGL((dsa3d_fixed_bwd_key_mfma_kernel<D, 1>), dim3((unsigned)nbk), dim3(256), 0, s, *ak);
            return hipGetLastError();
        }
    }
    if (a.group == kFixedGroup)
        hipLaunchKernelGGL((dsa3d_fixed_bwd_key_kernel<T, D, kFixedGroup>), dim3((unsigned)nb), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((dsa3d_fixed_bwd_key_kernel<T, D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t fixed_bwd_f32(const FixedArgs& a, int64_t nb, const FixedArgs* am, int64_t nbm, const FixedArgs* ak,
                         int64_t nbk, hipStream_t s) {
    return fixed_bwd_t<float, D>(a, nb, am, nbm, ak, nbk, s);
}
template <int D>
hipError_t fixed_bwd_bf16(const FixedArgs& a, int64_t nb, const FixedArgs* am, int64_t nbm, const FixedArgs* ak,
                          int64_t nbk, hipStream_t s) {
    return fixed_bwd_t<bf16_t, D>(a, nb, am, nbm, ak, nbk, s);
}

}  // namespace

size_t fixed_bwd_workspace_bytes(const dsa3d_desc& d) {  // room for a float pair per task
    return (size_t)(d.B * d.T * d.H * d.W) * (size_t)d.heads * 2 * sizeof(float) + 256;
}

bool fixed_fwd_on_mfma(const dsa3d_desc& d) {
    return d.dtype == DSA3D_BF16 && (d.head_dim == 32 || d.head_dim == 64 || d.head_dim == 128 || d.head_dim == 256) &&
           d.dil_w == 1 && d.kw <= kMfmaMaxKw && (int64_t)d.W * d.heads * d.head_dim * 2 <= (int64_t)INT32_MAX;
}

template <int D>
hipError_t fixed_fwd_mfma(const FixedArgs& a, int64_t nb, hipStream_t s) {
    LaunchScope ls(DSA3D_K_FORWARD, s);
    if constexpr (D <= kMfmaPairMaxD) {
        if (a.win.dil_h == 1) {
            hipLaunchKernelGGL((dsa3d_fixed_fwd_mfma_kernel<D, 2>), dim3((unsigned)nb), dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((dsa3d_fixed_fwd_mfma_kernel<D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Block order of the matrix-core kernels: four waves of 16 tokens along w per
// block, each on R rows (2 when the h axis is not dilated and rows have at
// most pair_max_d channels).
BlockOrder fixed_mfma_order(const dsa3d_desc& d, int pair_max_d) {
    dsa3d_desc dr = d;
    dr.H = d.dil_h == 1 && d.head_dim <= pair_max_d ? (d.H + 1) / 2 : d.H;
    return make_block_order(dr, 4 * kMfmaTokens, kGatherSupertile, "DSA3D_ORDER_FIXED_MFMA");
}

hipError_t launch_fixed_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, void* out,
                                float* lse, hipStream_t s) {
    FixedArgs a = fixed_args(d);
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    if (fixed_fwd_on_mfma(d)) {
        a.ord = fixed_mfma_order(d, kMfmaPairMaxD);
        const int64_t nb = a.ord.nblk_bh * d.B * d.heads;
        if (nb == 0) return hipSuccess;
        switch (d.head_dim) {
            case 32: return fixed_fwd_mfma<32>(a, nb, s);
            case 64: return fixed_fwd_mfma<64>(a, nb, s);
            case 128: return fixed_fwd_mfma<128>(a, nb, s);
            default: return fixed_fwd_mfma<256>(a, nb, s);
        }
    }
    const int64_t nb = a.ord.nblk_bh * d.B * d.heads;
    if (nb == 0) return hipSuccess;
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fixed_fwd_f32, a, nb, s); }
    DSA3D_DISPATCH_D(d.head_dim, fixed_fwd_bf16, a, nb, s);
}

hipError_t launch_fixed_backward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                                 hipStream_t s) {
    FixedArgs a = fixed_args(d);
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = const_cast<float*>(lse);
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dsum = reinterpret_cast<float*>(ws);
    const int64_t nb = a.ord.nblk_bh * d.B * d.heads;
    if (nb == 0) return hipSuccess;
    FixedArgs am = a, ak = a;
    am.ord = fixed_mfma_order(d, kMfmaPairMaxD);
    ak.ord = fixed_mfma_order(d, kMfmaKeyPairMaxD);
    const int64_t nbm = am.ord.nblk_bh * d.B * d.heads, nbk = ak.ord.nblk_bh * d.B * d.heads;
    const bool mf = fixed_fwd_on_mfma(d);
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fixed_bwd_f32, a, nb, nullptr, 0, nullptr, 0, s); }
    DSA3D_DISPATCH_D(d.head_dim, fixed_bwd_bf16, a, nb, mf ? &am : nullptr, nbm, mf ? &ak : nullptr, nbk, s);
}

}  // namespace dsa3d
