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
// Per task: pass 1 computes the P logits s_p = scale * sum_c w_c <q, K[c]>
// over the 8 trilinear corners c of each sample (keys are never interpolated
// into a row: the corner dot products are weighted instead), keeping them in
// LDS; the exact softmax follows; pass 2 accumulates
// o = sum_p a_p sum_c w_c V[c] in float32 registers. Corners outside the grid
// read a shared zero row, so no lane diverges on the border.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"

namespace dsa3d {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* off;
    void* out;
    float* lse;
    TaskGrid g;
    int32_t P;
    float scale;
    Window win;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_fwd_kernel(FwdArgs a) {
    constexpr int L = D / 8;
    extern __shared__ float s_logit[];  // [groups_per_block][P]
    const int groups = blockDim.x / L;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t task = (int64_t)lb * groups + g;
    const bool active = task < a.g.ntasks;
    const int64_t task_c = active ? task : a.g.ntasks - 1;  // inactive groups shadow the last task

    int32_t b, eta, t, h, w;
    int64_t tok;
    task_coords(a.g, task_c, b, eta, t, h, w, tok);
    const int64_t C = (int64_t)a.g.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const T* Kb = reinterpret_cast<const T*>(a.k) + row_off;
    const T* Vb = reinterpret_cast<const T*>(a.v) + row_off;
    const T* zero = reinterpret_cast<const T*>(g_zero_row);
    const T* offq = reinterpret_cast<const T*>(a.off) + (tok * a.g.heads + eta) * (int64_t)a.P * 3;

    Frag8<T> qf;
    qf.load(reinterpret_cast<const T*>(a.q) + tok * C + row_off);

    float* sl = s_logit + g * a.P;
    float m = -INFINITY;
    for (int p = 0; p < a.P; ++p) {
        float dt, dh, dw;
        load_offsets<T>(offq + p * 3, dt, dh, dw);
        int32_t t0 = 0, h0 = 0, w0 = 0;
        float ft = 0.f, fh = 0.f, fw = 0.f;
        const bool inside = sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw);
        Corners c;
        make_corners(a.g, b, t0, h0, w0, ft, fh, fw, inside, c);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            Frag8<T> kf;
            kf.load(c.tok[i] >= 0 ? Kb + c.tok[i] * C : zero);
            acc = fmaf(c.w[i], kf.dot(qf, 0.0f), acc);
        }
        const float s = a.scale * group_sum<L>(acc);
        if (li == 0) sl[p] = s;
        m = fmaxf(m, s);
    }
    __syncthreads();
    float z = 0.0f;
    for (int p = li; p < a.P; p += L) z += __expf(sl[p] - m);
    z = group_sum<L>(z);
    const float inv_z = 1.0f / z;

    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.P; ++p) {
        float dt, dh, dw;
        load_offsets<T>(offq + p * 3, dt, dh, dw);
        int32_t t0 = 0, h0 = 0, w0 = 0;
        float ft = 0.f, fh = 0.f, fw = 0.f;
        const bool inside = sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw);
        Corners c;
        make_corners(a.g, b, t0, h0, w0, ft, fh, fw, inside, c);
        const float ap = __expf(sl[p] - m) * inv_z;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            Frag8<T> vf;
            vf.load(c.tok[i] >= 0 ? Vb + c.tok[i] * C : zero);
            vf.axpy(ap * c.w[i], o);
        }
    }
    if (active) {
        Frag8<T> of;
        of.from_f32(o);
        of.store(reinterpret_cast<T*>(a.out) + tok * C + row_off);
        if (li == 0) a.lse[tok * a.g.heads + eta] = m + __logf(z);
    }
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

int fwd_groups_per_block(int head_dim, int P) {
    const int L = head_dim / 8;
    int groups = 256 / L;
    const int per_wave = 64 / L;
    while (groups > per_wave && (size_t)groups * P * sizeof(float) > 65536) groups -= per_wave;
    if ((size_t)groups * P * sizeof(float) > 65536) return 0;
    return groups;
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
    const int groups = fwd_groups_per_block(D, a.P);
    const int threads = groups * (D / 8);
    const int64_t nb = (a.g.ntasks + groups - 1) / groups;
    LaunchScope ls(DSA3D_K_FORWARD, s);
    hipLaunchKernelGGL((dsa3d_fwd_kernel<T, D>), dim3((unsigned)nb), dim3(threads), groups * a.P * sizeof(float), s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t fwd_f32(const FwdArgs& a, hipStream_t s) { return launch_fwd_t<float, D>(a, s); }
template <int D>
static hipError_t fwd_bf16(const FwdArgs& a, hipStream_t s) { return launch_fwd_t<bf16_t, D>(a, s); }

hipError_t launch_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                          void* out, float* lse, hipStream_t s) {
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.off = off; a.out = out; a.lse = lse;
    a.g = make_task_grid(d, 0, d.heads);
    a.P = d.P;
    a.scale = logit_scale(d);
    a.win = make_window(d);
    if (a.g.ntasks == 0) return hipSuccess;
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fwd_f32, a, s); }
    DSA3D_DISPATCH_D(d.head_dim, fwd_bf16, a, s);
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
