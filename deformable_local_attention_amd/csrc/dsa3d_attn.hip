// dsa3d_attn.hip -- fused 3D-DSA attention kernels for gfx950.
//
// One (query token, head) -- a "task" -- is owned by an aligned group of
// L = head_dim/8 lanes of a wave64; each lane owns 8 consecutive channels, so
// one key/value row of a head (head_dim elements) is read by the group as one
// coalesced L*16-byte (bf16) or L*32-byte (f32) access. Tasks are ordered
// (batch, head, t, h, w) with w fastest, so the groups of a workgroup are
// neighbouring queries of one head whose sampled neighbourhoods overlap; the
// block id is remapped so that each XCD walks one contiguous range of them.
//
// Forward (per task): pass 1 computes the P logits s_p = scale * sum_c w_c
// <q, K[c]> over the 8 trilinear corners c of each sample (keys are never
// interpolated into a row: the corner dot products are weighted instead),
// keeping them in LDS; the exact softmax follows; pass 2 accumulates
// o = sum_p a_p sum_c w_c V[c] in float32 registers. Corners outside the grid
// read a shared zero row, so no lane diverges on the border.
//
// Backward (per task, one pass over P): recompute s_p, a_p = exp(s_p - lse),
// da_p = sum_c w_c <dO, V[c]>, ds_p = a_p (da_p - <dO, o>); accumulate
// dq = scale sum_p ds_p sum_c w_c K[c] in registers; write
// doffsets_p = scale ds_p G_p + a_p H_p, where G and H are the corner dot
// products weighted by the derivative of the trilinear weights; and add
// w_c scale ds_p q and w_c a_p dO into the dk/dv accumulators of every
// in-grid corner with global atomics (float32, or 64-bit fixed point in
// deterministic mode).
#include "dsa3d_device.h"
#include "dsa3d_internal.h"

namespace dsa3d {

// Zero row read in place of a corner outside the grid (256 floats: the widest row).
__device__ __attribute__((aligned(16))) const float g_zero_row[256] = {0.0f};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* off;
    void* out;
    float* lse;
    // backward only
    const void* o;
    const void* dout;
    void* dq;
    void* doff;
    void* acc_k;  // float32 or fixed-point accumulators, or dk/dv themselves
    void* acc_v;
    int32_t T, H, W;
    int32_t heads;
    int32_t head0, nheads;  // head range of this launch
    int32_t P;
    float scale;
    Window win;
    int64_t ntasks;         // B*T*H*W*nheads
    int64_t acc_row;        // accumulator elements per token (nheads*D or C)
    int32_t acc_head0;      // head index of the accumulator's first head slot
};

template <typename T, int D>
__device__ __forceinline__ void task_coords(const AttnArgs& a, int64_t task, int32_t& b, int32_t& eta, int32_t& t,
                                            int32_t& h, int32_t& w, int64_t& tok) {
    const int64_t HW = (int64_t)a.H * a.W;
    const int64_t THW = HW * a.T;
    const int64_t bh = task / THW;
    int64_t rem = task - bh * THW;
    b = (int32_t)(bh / a.nheads);
    eta = a.head0 + (int32_t)(bh - (int64_t)b * a.nheads);
    t = (int32_t)(rem / HW);
    rem -= (int64_t)t * HW;
    h = (int32_t)(rem / a.W);
    w = (int32_t)(rem - (int64_t)h * a.W);
    tok = (int64_t)b * THW + (int64_t)t * HW + (int64_t)h * a.W + w;
}

// Eight corner rows of one sample: element offsets (or -1 for a zero row) and
// trilinear weights; derivative factors on request.
struct Corners {
    int64_t tok[8];  // token index, or -1 outside the grid
    float w[8];
};

__device__ __forceinline__ void make_corners(const AttnArgs& a, int32_t b, int32_t t0, int32_t h0, int32_t w0,
                                             float ft, float fh, float fw, bool inside, Corners& c) {
    const float at[2] = {1.0f - ft, ft}, ah[2] = {1.0f - fh, fh}, aw[2] = {1.0f - fw, fw};
    const int64_t base_b = (int64_t)b * a.T;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ct = (i >> 2) & 1, ch = (i >> 1) & 1, cw = i & 1;
        const int32_t tt = t0 + ct, hh = h0 + ch, ww = w0 + cw;
        const bool ok = inside && (uint32_t)tt < (uint32_t)a.T && (uint32_t)hh < (uint32_t)a.H &&
                        (uint32_t)ww < (uint32_t)a.W;
        c.tok[i] = ok ? ((base_b + tt) * a.H + hh) * (int64_t)a.W + ww : -1;
        c.w[i] = ok ? at[ct] * ah[ch] * aw[cw] : 0.0f;
    }
}

template <typename T>
__device__ __forceinline__ void load_offsets(const T* off, float& dt, float& dh, float& dw) {
    dt = load_scalar<T>(off + 0);
    dh = load_scalar<T>(off + 1);
    dw = load_scalar<T>(off + 2);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_fwd_kernel(AttnArgs a) {
    constexpr int L = D / 8;
    extern __shared__ float s_logit[];  // [groups_per_block][P]
    const int groups = blockDim.x / L;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t task = (int64_t)lb * groups + g;
    const bool active = task < a.ntasks;
    const int64_t task_c = active ? task : a.ntasks - 1;  // inactive groups shadow the last task

    int32_t b, eta, t, h, w;
    int64_t tok;
    task_coords<T, D>(a, task_c, b, eta, t, h, w, tok);
    const int64_t C = (int64_t)a.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const T* Kb = reinterpret_cast<const T*>(a.k) + row_off;
    const T* Vb = reinterpret_cast<const T*>(a.v) + row_off;
    const T* zero = reinterpret_cast<const T*>(g_zero_row);
    const T* offq = reinterpret_cast<const T*>(a.off) + (tok * a.heads + eta) * (int64_t)a.P * 3;

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
        make_corners(a, b, t0, h0, w0, ft, fh, fw, inside, c);
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
        make_corners(a, b, t0, h0, w0, ft, fh, fw, inside, c);
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
        if (li == 0) a.lse[tok * a.heads + eta] = m + __logf(z);
    }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
template <bool DET>
__device__ __forceinline__ void acc_add(void* base, int64_t idx, float x) {
    if (DET) {
        atomicAdd(reinterpret_cast<unsigned long long*>(base) + idx, to_fixed(x));
    } else {
        unsafeAtomicAdd(reinterpret_cast<float*>(base) + idx, x);
    }
}

template <typename T, int D, bool DET>
__global__ void __launch_bounds__(256) dsa3d_bwd_kernel(AttnArgs a) {
    constexpr int L = D / 8;
    const int groups = blockDim.x / L;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t task = (int64_t)lb * groups + g;
    if (task >= a.ntasks) return;  // no block-wide barrier below

    int32_t b, eta, t, h, w;
    int64_t tok;
    task_coords<T, D>(a, task, b, eta, t, h, w, tok);
    const int64_t C = (int64_t)a.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const T* Kb = reinterpret_cast<const T*>(a.k) + row_off;
    const T* Vb = reinterpret_cast<const T*>(a.v) + row_off;
    const T* zero = reinterpret_cast<const T*>(g_zero_row);
    const int64_t offrow = (tok * a.heads + eta) * (int64_t)a.P * 3;
    const T* offq = reinterpret_cast<const T*>(a.off) + offrow;
    T* doffq = reinterpret_cast<T*>(a.doff) + offrow;
    const int64_t acc_off = (int64_t)(eta - a.acc_head0) * D + li * 8;

    Frag8<T> qf, gf, of;
    qf.load(reinterpret_cast<const T*>(a.q) + tok * C + row_off);
    gf.load(reinterpret_cast<const T*>(a.dout) + tok * C + row_off);
    of.load(reinterpret_cast<const T*>(a.o) + tok * C + row_off);
    float qv[8], gv[8];
    qf.to_f32(qv);
    gf.to_f32(gv);
    const float Dsum = group_sum<L>(gf.dot(of, 0.0f));
    const float lse = a.lse[tok * a.heads + eta];

    float dq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.P; ++p) {
        float dt, dh, dw;
        load_offsets<T>(offq + p * 3, dt, dh, dw);
        int32_t t0 = 0, h0 = 0, w0 = 0;
        float ft = 0.f, fh = 0.f, fw = 0.f;
        const bool inside = sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw);
        Corners c;
        make_corners(a, b, t0, h0, w0, ft, fh, fw, inside, c);
        Frag8<T> kf[8], vf[8];
        float qk[8], dv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kf[i].load(c.tok[i] >= 0 ? Kb + c.tok[i] * C : zero);
            vf[i].load(c.tok[i] >= 0 ? Vb + c.tok[i] * C : zero);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qk[i] = kf[i].dot(qf, 0.0f);
            dv[i] = vf[i].dot(gf, 0.0f);
        }
        // weighted sums: logit, dL/da, and the offset-derivative sums per axis
        const float at[2] = {1.0f - ft, ft}, ah[2] = {1.0f - fh, fh}, aw[2] = {1.0f - fw, fw};
        float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ct = (i >> 2) & 1, ch = (i >> 1) & 1, cw = i & 1;
            const float st = ct ? 1.f : -1.f, sh = ch ? 1.f : -1.f, sw = cw ? 1.f : -1.f;
            const float gt = st * ah[ch] * aw[cw], gh = at[ct] * sh * aw[cw], gw = at[ct] * ah[ch] * sw;
            // zero rows give zero dot products, so no validity test is needed here
            r[0] = fmaf(c.w[i], qk[i], r[0]);
            r[1] = fmaf(c.w[i], dv[i], r[1]);
            r[2] = fmaf(gt, qk[i], r[2]);
            r[3] = fmaf(gh, qk[i], r[3]);
            r[4] = fmaf(gw, qk[i], r[4]);
            r[5] = fmaf(gt, dv[i], r[5]);
            r[6] = fmaf(gh, dv[i], r[6]);
            r[7] = fmaf(gw, dv[i], r[7]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = group_sum<L>(r[j]);
        const float s = a.scale * r[0];
        const float ap = __expf(s - lse);
        const float ds = ap * (r[1] - Dsum);
        const float ck = a.scale * ds;
        if (li == 0) {
            store_scalar<T>(doffq + p * 3 + 0, fmaf(ck, r[2], ap * r[5]));
            store_scalar<T>(doffq + p * 3 + 1, fmaf(ck, r[3], ap * r[6]));
            store_scalar<T>(doffq + p * 3 + 2, fmaf(ck, r[4], ap * r[7]));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kf[i].axpy(ck * c.w[i], dq);
            if (c.tok[i] >= 0) {
                const int64_t base = c.tok[i] * a.acc_row + acc_off;
                const float sk = ck * c.w[i], sv = ap * c.w[i];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc_add<DET>(a.acc_k, base + e, sk * qv[e]);
                    acc_add<DET>(a.acc_v, base + e, sv * gv[e]);
                }
            }
        }
    }
    Frag8<T> dqf;
    dqf.from_f32(dq);
    dqf.store(reinterpret_cast<T*>(a.dq) + tok * C + row_off);
}

// acc_k/acc_v [ntok, nheads, D] (float32 or fixed point) -> dk/dv[tok, head0 + j, :]
// in the output dtype; the accumulators are cleared for the next pass.
template <typename T, bool DET>
__global__ void __launch_bounds__(256) dsa3d_finalize_kernel(void* acc_k, void* acc_v, T* dk, T* dv, int64_t ntok,
                                                             int32_t nheads, int32_t head0, int32_t heads, int32_t D) {
    const int64_t row = (int64_t)nheads * D;
    const int64_t n = ntok * row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n; i += (int64_t)gridDim.x * blockDim.x) {
        const bool second = i >= n;
        const int64_t ii = second ? i - n : i;
        void* acc = second ? acc_v : acc_k;
        T* out = second ? dv : dk;
        const int64_t tk = ii / row;
        const int64_t j = ii - tk * row;
        float x;
        if (DET) {
            unsigned long long* p = reinterpret_cast<unsigned long long*>(acc) + ii;
            x = from_fixed(*p);
            *p = 0ull;
        } else {
            float* p = reinterpret_cast<float*>(acc) + ii;
            x = *p;
            *p = 0.0f;
        }
        store_scalar<T>(out + tk * (int64_t)heads * D + (int64_t)head0 * D + j, x);
    }
}

__global__ void __launch_bounds__(256) dsa3d_fill_zero_kernel(uint32_t* p, int64_t nwords) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <typename T>
__global__ void __launch_bounds__(256) dsa3d_geometry_kernel(AttnArgs a, int32_t* base, float* frac) {
    const int64_t n = a.ntasks * a.P;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t task = i / a.P;
        const int32_t p = (int32_t)(i - task * a.P);
        int32_t b, eta, t, h, w;
        int64_t tok;
        task_coords<T, 8>(a, task, b, eta, t, h, w, tok);
        const T* o = reinterpret_cast<const T*>(a.off) + ((tok * a.heads + eta) * (int64_t)a.P + p) * 3;
        float dt, dh, dw;
        load_offsets<T>(o, dt, dh, dw);
        int32_t t0 = INT32_MIN, h0 = INT32_MIN, w0 = INT32_MIN;
        float ft = 0.f, fh = 0.f, fw = 0.f;
        if (!sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw)) {
            t0 = h0 = w0 = INT32_MIN;
            ft = fh = fw = 0.f;
        }
        const int64_t j = ((tok * a.heads + eta) * (int64_t)a.P + p) * 3;
        base[j] = t0; base[j + 1] = h0; base[j + 2] = w0;
        frac[j] = ft; frac[j + 1] = fh; frac[j + 2] = fw;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
static Window make_window(const dsa3d_desc& d) {
    Window w;
    w.kt = d.kt; w.kh = d.kh; w.kw = d.kw; w.khw = d.kh * d.kw;
    w.dil_t = d.dil_t; w.dil_h = d.dil_h; w.dil_w = d.dil_w;
    w.rt = (d.kt - 1) / 2; w.rh = (d.kh - 1) / 2; w.rw = (d.kw - 1) / 2;
    return w;
}

static AttnArgs base_args(const dsa3d_desc& d) {
    AttnArgs a{};
    a.T = (int32_t)d.T; a.H = (int32_t)d.H; a.W = (int32_t)d.W;
    a.heads = d.heads;
    a.head0 = 0; a.nheads = d.heads;
    a.P = d.P;
    a.scale = d.scale != 0.0f ? d.scale : 1.0f / sqrtf((float)d.head_dim);
    a.win = make_window(d);
    a.ntasks = d.B * d.T * d.H * d.W * d.heads;
    return a;
}

static inline unsigned grid_for(int64_t n, int threads, int64_t cap = 1 << 20) {
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
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t s) {
    const int groups = fwd_groups_per_block(D, a.P);
    const int threads = groups * (D / 8);
    const int64_t nb = (a.ntasks + groups - 1) / groups;
    LaunchScope ls(DSA3D_K_FORWARD, s);
    hipLaunchKernelGGL((dsa3d_fwd_kernel<T, D>), dim3((unsigned)nb), dim3(threads), groups * a.P * sizeof(float), s, a);
    return hipGetLastError();
}

template <typename T, int D, bool DET>
static hipError_t launch_bwd_t(const AttnArgs& a, hipStream_t s) {
    const int groups = 256 / (D / 8);
    const int64_t nb = (a.ntasks + groups - 1) / groups;
    LaunchScope ls(DSA3D_K_BACKWARD, s);
    hipLaunchKernelGGL((dsa3d_bwd_kernel<T, D, DET>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}

#define DSA3D_DISPATCH_D(D_, FN, ...)                 \
    switch (D_) {                                    \
        case 8: return FN<8>(__VA_ARGS__);           \
        case 16: return FN<16>(__VA_ARGS__);         \
        case 32: return FN<32>(__VA_ARGS__);         \
        case 64: return FN<64>(__VA_ARGS__);         \
        case 128: return FN<128>(__VA_ARGS__);       \
        case 256: return FN<256>(__VA_ARGS__);       \
        default: return hipErrorInvalidValue;        \
    }

template <int D>
static hipError_t fwd_f32(const AttnArgs& a, hipStream_t s) { return launch_fwd_t<float, D>(a, s); }
template <int D>
static hipError_t fwd_bf16(const AttnArgs& a, hipStream_t s) { return launch_fwd_t<bf16_t, D>(a, s); }

hipError_t launch_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                          void* out, float* lse, hipStream_t s) {
    AttnArgs a = base_args(d);
    a.q = q; a.k = k; a.v = v; a.off = off; a.out = out; a.lse = lse;
    if (a.ntasks == 0) return hipSuccess;
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, fwd_f32, a, s); }
    DSA3D_DISPATCH_D(d.head_dim, fwd_bf16, a, s);
}

template <int D>
static hipError_t bwd_f32_fast(const AttnArgs& a, hipStream_t s) { return launch_bwd_t<float, D, false>(a, s); }
template <int D>
static hipError_t bwd_f32_det(const AttnArgs& a, hipStream_t s) { return launch_bwd_t<float, D, true>(a, s); }
template <int D>
static hipError_t bwd_bf16_fast(const AttnArgs& a, hipStream_t s) { return launch_bwd_t<bf16_t, D, false>(a, s); }
template <int D>
static hipError_t bwd_bf16_det(const AttnArgs& a, hipStream_t s) { return launch_bwd_t<bf16_t, D, true>(a, s); }

static hipError_t bwd_dispatch(const dsa3d_desc& d, const AttnArgs& a, hipStream_t s) {
    const bool det = d.deterministic != 0;
    if (d.dtype == DSA3D_F32) {
        if (det) { DSA3D_DISPATCH_D(d.head_dim, bwd_f32_det, a, s); }
        DSA3D_DISPATCH_D(d.head_dim, bwd_f32_fast, a, s);
    }
    if (det) { DSA3D_DISPATCH_D(d.head_dim, bwd_bf16_det, a, s); }
    DSA3D_DISPATCH_D(d.head_dim, bwd_bf16_fast, a, s);
}

static hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
    const int64_t words = (int64_t)(bytes / 4);
    if (words == 0) return hipSuccess;
    LaunchScope ls(DSA3D_K_FILL, s);
    hipLaunchKernelGGL(dsa3d_fill_zero_kernel, dim3(grid_for(words, 256, 65536)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

size_t bwd_accumulator_bytes_per_head(const dsa3d_desc& d) {
    const int64_t ntok = d.B * d.T * d.H * d.W;
    const bool direct = d.dtype == DSA3D_F32 && !d.deterministic;
    if (direct) return 0;
    const size_t esize = d.deterministic ? 8 : 4;
    return 2 * (size_t)ntok * d.head_dim * esize;
}

hipError_t launch_backward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* doff, void* ws, size_t ws_bytes, hipStream_t s) {
    AttnArgs a = base_args(d);
    a.q = q; a.k = k; a.v = v; a.off = off; a.o = o; a.lse = const_cast<float*>(lse); a.dout = dout;
    a.dq = dq; a.doff = doff;
    const int64_t ntok = d.B * d.T * d.H * d.W;
    const int64_t C = (int64_t)d.heads * d.head_dim;
    const size_t esz = d.dtype == DSA3D_F32 ? 4 : 2;
    if (ntok == 0) return hipSuccess;
    hipError_t e;
    const size_t per_head = bwd_accumulator_bytes_per_head(d);
    if (per_head == 0) {
        // float32 fast mode: accumulate straight into dk/dv.
        if ((e = fill_zero(dk, (size_t)ntok * C * esz, s)) != hipSuccess) return e;
        if ((e = fill_zero(dv, (size_t)ntok * C * esz, s)) != hipSuccess) return e;
        a.acc_k = dk; a.acc_v = dv; a.acc_row = C; a.acc_head0 = 0;
        return bwd_dispatch(d, a, s);
    }
    const int64_t chunk = std::min<int64_t>(d.heads, (int64_t)(ws_bytes / per_head));
    const size_t half = (size_t)ntok * chunk * d.head_dim * (d.deterministic ? 8 : 4);
    if ((e = fill_zero(ws, 2 * half, s)) != hipSuccess) return e;
    for (int32_t h0 = 0; h0 < d.heads; h0 += (int32_t)chunk) {
        const int32_t nh = (int32_t)std::min<int64_t>(chunk, d.heads - h0);
        a.head0 = h0; a.nheads = nh;
        a.ntasks = ntok * nh;
        a.acc_k = ws;
        a.acc_v = reinterpret_cast<char*>(ws) + half;
        a.acc_row = (int64_t)nh * d.head_dim;
        a.acc_head0 = h0;
        if ((e = bwd_dispatch(d, a, s)) != hipSuccess) return e;
        const int64_t n = 2 * ntok * nh * d.head_dim;
        const unsigned gb = grid_for(n, 256, 65536);
        LaunchScope ls(DSA3D_K_BWD_FINALIZE, s);
        if (d.dtype == DSA3D_F32) {
            hipLaunchKernelGGL((dsa3d_finalize_kernel<float, true>), dim3(gb), dim3(256), 0, s, a.acc_k, a.acc_v,
                               (float*)dk, (float*)dv, ntok, nh, h0, d.heads, d.head_dim);
        } else if (d.deterministic) {
            hipLaunchKernelGGL((dsa3d_finalize_kernel<bf16_t, true>), dim3(gb), dim3(256), 0, s, a.acc_k, a.acc_v,
                               (bf16_t*)dk, (bf16_t*)dv, ntok, nh, h0, d.heads, d.head_dim);
        } else {
            hipLaunchKernelGGL((dsa3d_finalize_kernel<bf16_t, false>), dim3(gb), dim3(256), 0, s, a.acc_k, a.acc_v,
                               (bf16_t*)dk, (bf16_t*)dv, ntok, nh, h0, d.heads, d.head_dim);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_geometry(const dsa3d_desc& d, const void* off, int32_t* base, float* frac, hipStream_t s) {
    AttnArgs a = base_args(d);
    a.off = off;
    const int64_t n = a.ntasks * a.P;
    if (n == 0) return hipSuccess;
    LaunchScope ls(DSA3D_K_GEOMETRY, s);
    if (d.dtype == DSA3D_F32)
        hipLaunchKernelGGL((dsa3d_geometry_kernel<float>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, a, base,
                           frac);
    else
        hipLaunchKernelGGL((dsa3d_geometry_kernel<bf16_t>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, a, base,
                           frac);
    return hipGetLastError();
}

}  // namespace dsa3d
