// dsa3d_attn.hip -- fused 3D-DSA forward kernel for gfx950, plus the geometry
// test hook and a zero-fill kernel.
//
// One (query token, head) -- a "task" -- is owned by an aligned group of
// L = head_dim/8 lanes of a wave64; each lane owns 8 consecutive channels, so
// one key/value row of a head (head_dim elements) is read by the group as one
// coalesced L*16-byte (bf16) or L*32-byte (f32) access. Tasks are ordered
// (batch, head, t, h, w) with w fastest, so the groups of a workgroup are
// neighbouring queries of one head whose sampled neighbourhoods overlap; the
// block id is remapped so that each XCD walks one contiguous range of them.
//
// Per task, one pass over the P samples with an online softmax: the logit
// s_p = scale * sum_c w_c <q, K[c]> weights the 8 corner dot products (keys are
// never interpolated into a row), then the running maximum m, denominator z
// and output o = sum_p exp(s_p - m) sum_c w_c V[c] are updated, o being
// rescaled by exp(m_old - m_new) when m grows; o/z and lse = m + log z are
// written at the end. Corners outside the grid read a shared zero row, so no
// lane diverges on the border.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"

#ifdef DSA3D_TUNING
#include <cstdio>
#include <cstdlib>
#endif

namespace dsa3d {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* off;
    void* out;
    float* lse;
    TaskGrid g;
    BlockOrder ord;
    int32_t P;
    float scale;
    Window win;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_fwd_kernel(FwdArgs a) {
    constexpr int L = D / 8;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    int64_t bh;
    int32_t t, h, w0;
    block_coords(a.g, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, h, w0);
    const int32_t w = w0 + g;
    if (w >= a.g.W) return;  // no block-wide barrier below
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int64_t tok = (int64_t)tok_b + ((int64_t)t * a.g.H + h) * a.g.W + w;
    const int64_t C = (int64_t)a.g.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const CornerStrides cs = corner_strides(a.g, C * (int64_t)sizeof(T));
    const char* Kb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + row_off);
    const char* Vb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + row_off);
    const char* zero = reinterpret_cast<const char*>(g_zero_row);
    const T* offq = reinterpret_cast<const T*>(a.off) + (tok * a.g.heads + eta) * (int64_t)a.P * 3;

    Frag8<T> qf;
    qf.load(reinterpret_cast<const T*>(a.q) + tok * C + row_off);

    // The group walks the samples in chunks of L: each lane computes the cell
    // of one sample of the chunk and leaves it in LDS, then every lane reads
    // each sample's cell from there (a broadcast read).
    __shared__ SampleGeo s_geo[256];
    SampleGeo* geo = s_geo + (threadIdx.x - li);

    float m = -INFINITY, z = 0.0f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < a.P; p0 += L) {
        const int n = min(L, a.P - p0);
        wave_lds_sync();  // the previous chunk has been read
        if (li < n) {
            SampleGeo sg;
            int32_t t0, h0, w0c;
            sample_geo<T>(a.g, a.win, tok_b, t, h, w, p0 + li, offq + (p0 + li) * 3, sg, t0, h0, w0c);
            geo[li] = sg;
        }
        wave_lds_sync();
        for (int j = 0; j < n; ++j) {
            const SampleGeo& sg = geo[j];
            const uint32_t valid = sg.valid;
            CornerAddr ca;
            corner_addresses(sg.tok0, valid, Kb, Vb, cs, zero, __all((valid >> 8) & 1u), ca);
            Frag8<T> kf[8], vf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kf[i].load(reinterpret_cast<const T*>(ca.a[i]));
                vf[i].load(reinterpret_cast<const T*>(ca.b[i]));
            }
            float wgt[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wgt[i] = sg.w[i];
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf(wgt[i], kf[i].dot(qf, 0.0f), acc);
            const float s = a.scale * group_sum<L>(acc);
            const float m_new = fmaxf(m, s);
            const float alpha = __expf(m - m_new);  // 0 for the first sample (m = -inf)
            const float beta = __expf(s - m_new);
            z = fmaf(z, alpha, beta);
            if (!__all(m_new == m)) {  // the running max rarely moves after the first samples
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) vf[i].axpy(beta * wgt[i], o);
            m = m_new;
        }
    }
    const float inv_z = 1.0f / z;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv_z;
    Frag8<T> of;
    of.from_f32(o);
    of.store(reinterpret_cast<T*>(a.out) + tok * C + row_off);
    if (li == 0) a.lse[tok * a.g.heads + eta] = m + __logf(z);
}

__global__ void __launch_bounds__(256) dsa3d_fill_zero_kernel(uint32_t* p, int64_t nwords) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <typename T>
__global__ void __launch_bounds__(256) dsa3d_geometry_kernel(TaskGrid g, Window win, int32_t P, const void* off,
                                                             int32_t* base, float* frac) {
    const int64_t n = g.ntasks * P;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t task = i / P;
        const int32_t p = (int32_t)(i - task * P);
        int32_t b, eta, t, h, w;
        int64_t tok;
        task_coords(g, task, b, eta, t, h, w, tok);
        const int64_t j = ((tok * g.heads + eta) * (int64_t)P + p) * 3;
        float dt, dh, dw;
        load_offsets<T>(reinterpret_cast<const T*>(off) + j, dt, dh, dw);
        int32_t t0 = INT32_MIN, h0 = INT32_MIN, w0 = INT32_MIN;
        float ft = 0.f, fh = 0.f, fw = 0.f;
        if (!sample_geometry(win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw)) {
            t0 = h0 = w0 = INT32_MIN;
            ft = fh = fw = 0.f;
        }
        base[j] = t0; base[j + 1] = h0; base[j + 2] = w0;
        frac[j] = ft; frac[j + 1] = fh; frac[j + 2] = fw;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
Window make_window(const dsa3d_desc& d) {
    Window w;
    w.kt = d.kt; w.kh = d.kh; w.kw = d.kw; w.khw = d.kh * d.kw;
    w.dil_t = d.dil_t; w.dil_h = d.dil_h; w.dil_w = d.dil_w;
    w.rt = (d.kt - 1) / 2; w.rh = (d.kh - 1) / 2; w.rw = (d.kw - 1) / 2;
    return w;
}

TaskGrid make_task_grid(const dsa3d_desc& d, int32_t head0, int32_t nheads) {
    TaskGrid g;
    g.T = (int32_t)d.T; g.H = (int32_t)d.H; g.W = (int32_t)d.W;
    g.heads = d.heads;
    g.head0 = head0; g.nheads = nheads;
    g.ntasks = d.B * d.T * d.H * d.W * nheads;
    return g;
}

float logit_scale(const dsa3d_desc& d) { return d.scale != 0.0f ? d.scale : 1.0f / sqrtf((float)d.head_dim); }

unsigned grid_for(int64_t n, int threads, int64_t cap) {
    int64_t b = (n + threads - 1) / threads;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

BlockOrder make_block_order(const dsa3d_desc& d, int G, Supertile st, const char* tuning_env) {
    BlockOrder o;
    o.G = G;
    o.BW = (int32_t)((d.W + G - 1) / G);
    int frames = st.frames, rows = st.rows, tokens = st.tokens, chunk = -1;
#ifdef DSA3D_TUNING
    // tuning builds only: <tuning_env>="frames,rows,tokens,chunk"
    if (const char* e = getenv(tuning_env)) sscanf(e, "%d,%d,%d,%d", &frames, &rows, &tokens, &chunk);
#else
    (void)tuning_env;
#endif
    if (rows < 0) {  // bands of about -rows rows, of equal height
        const int64_t bands = std::max<int64_t>(1, (d.H + (-rows) / 2) / (-rows));
        rows = (int)((d.H + bands - 1) / bands);
    }
    o.ST = std::max(1, frames);
    o.SH = std::max(1, rows);
    o.SW = std::max(1, tokens / G);
    o.chunk = chunk < 0 ? o.ST * o.SH * o.SW : chunk;
    o.nblk_bh = d.T * d.H * (int64_t)o.BW;
    return o;
}

int attn_tokens_per_block(int head_dim) { return 256 / (head_dim / 8); }

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, int64_t nblocks, hipStream_t s) {
    LaunchScope ls(DSA3D_K_FORWARD, s);
    hipLaunchKernelGGL((dsa3d_fwd_kernel<T, D>), dim3((unsigned)nblocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t fwd_f32(const FwdArgs& a, int64_t nb, hipStream_t s) { return launch_fwd_t<float, D>(a, nb, s); }
template <int D>
static hipError_t fwd_bf16(const FwdArgs& a, int64_t nb, hipStream_t s) { return launch_fwd_t<bf16_t, D>(a, nb, s); }

hipError_t launch_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                          void* out, float* lse, hipStream_t s) {
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.off = off; a.out = out; a.lse = lse;
    a.g = make_task_grid(d, 0, d.heads);
    a.P = d.P;
    a.scale = logit_scale(d);
    a.win = make_window(d);
    a.ord = make_block_order(d, attn_tokens_per_block(d.head_dim), kForwardSupertile, "DSA3D_ORDER");
    const int64_t nb = a.ord.nblk_bh * d.B * d.heads;
    if (nb == 0) return hipSuccess;
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fwd_f32, a, nb, s); }
    DSA3D_DISPATCH_D(d.head_dim, fwd_bf16, a, nb, s);
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
    const int64_t words = (int64_t)(bytes / 4);
    if (words == 0) return hipSuccess;
    LaunchScope ls(DSA3D_K_FILL, s);
    hipLaunchKernelGGL(dsa3d_fill_zero_kernel, dim3(grid_for(words, 256, 65536)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

hipError_t launch_geometry(const dsa3d_desc& d, const void* off, int32_t* base, float* frac, hipStream_t s) {
    const TaskGrid g = make_task_grid(d, 0, d.heads);
    const Window win = make_window(d);
    const int64_t n = g.ntasks * d.P;
    if (n == 0) return hipSuccess;
    LaunchScope ls(DSA3D_K_GEOMETRY, s);
    if (d.dtype == DSA3D_F32)
        hipLaunchKernelGGL((dsa3d_geometry_kernel<float>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, g, win,
                           d.P, off, base, frac);
    else
        hipLaunchKernelGGL((dsa3d_geometry_kernel<bf16_t>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, g, win,
                           d.P, off, base, frac);
    return hipGetLastError();
}

}  // namespace dsa3d
