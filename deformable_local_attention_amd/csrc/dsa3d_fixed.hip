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
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"

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
    float* dsum;  // <dO, o> per task, [B,T,H,W,heads]
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

template <typename T, int D>
hipError_t fixed_bwd_t(const FixedArgs& a, int64_t nb, hipStream_t s) {
    {
        LaunchScope ls(DSA3D_K_BWD_QUERY, s);
        if (a.group == kFixedGroup)
            hipLaunchKernelGGL((dsa3d_fixed_bwd_query_kernel<T, D, kFixedGroup>), dim3((unsigned)nb), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((dsa3d_fixed_bwd_query_kernel<T, D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    LaunchScope ls(DSA3D_K_BWD_KEY, s);
    if (a.group == kFixedGroup)
        hipLaunchKernelGGL((dsa3d_fixed_bwd_key_kernel<T, D, kFixedGroup>), dim3((unsigned)nb), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((dsa3d_fixed_bwd_key_kernel<T, D, 1>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D> hipError_t fixed_bwd_f32(const FixedArgs& a, int64_t nb, hipStream_t s) { return fixed_bwd_t<float, D>(a, nb, s); }
template <int D> hipError_t fixed_bwd_bf16(const FixedArgs& a, int64_t nb, hipStream_t s) { return fixed_bwd_t<bf16_t, D>(a, nb, s); }

}  // namespace

size_t fixed_bwd_workspace_bytes(const dsa3d_desc& d) {
    return (size_t)(d.B * d.T * d.H * d.W) * (size_t)d.heads * sizeof(float) + 256;
}

hipError_t launch_fixed_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, void* out,
                                float* lse, hipStream_t s) {
    FixedArgs a = fixed_args(d);
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
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
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fixed_bwd_f32, a, nb, s); }
    DSA3D_DISPATCH_D(d.head_dim, fixed_bwd_bf16, a, nb, s);
}

}  // namespace dsa3d
