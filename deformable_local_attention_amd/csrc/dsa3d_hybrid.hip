// dsa3d_hybrid.hip -- hybrid attention for gfx950: G global tokens per
// (batch, head) join every query's softmax over its P deformable samples
// [MegaSlide-DiT, §11 Limitations and Discussion, future work (i): sparse
// global tokens combined with local 3D-DSA].
//
// For query x of head eta, with the local logits s_p (p < P) and the global
// ones s_g = scale <q, GK[g]>, one softmax over all P + G logits:
//   o = sum_p a_p v_p + sum_g a_g GV[g],  lse = log(sum_p e^{s_p} + sum_g e^{s_g}).
// The local part is the operator's own forward, giving (o_l, lse_l); the
// global part is then folded in exactly: with (m, z, acc) the running max, sum
// and weighted sum of the global logits,
//   lse = log(e^{lse_l} + z e^m),  o = e^{lse_l - lse} o_l + e^{m - lse} acc.
// The backward needs nothing else from the local kernels: given the merged o
// and lse they compute a_p = e^{s_p - lse} and ds_p = a_p (da_p - <dO, o>) of
// the joint softmax. The global rows add
//   dq += scale sum_g ds_g GK[g],  dGK[g] = scale sum_x ds_g q_x,  dGV[g] = sum_x a_g dO_x,
// the last two reduced over every query of the (batch, head) in a fixed order
// (per-slab float32 partials, then an ordered sum).
//
// All three kernels run on the vector units: a global row is read by every
// query of a block from LDS, where the block stages GK and GV once.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"

namespace dsa3d {

namespace {

constexpr int kHybLds = 64 * 1024;  // bytes of staged global rows per block (keys and values)
constexpr int kHybRounds = 4;       // query groups per lane group in the per-query kernels

struct HybArgs {
    const void* q;
    const void* dout;
    const void* gk;     // [B, G, heads, D]
    const void* gv;
    void* out;          // forward: local output, merged in place; backward: merged output (read)
    float* lse;         // forward: local lse, merged in place; backward: merged lse (read)
    void* dq;           // backward: the local dq, the global share added in place
    float* dsum;        // backward: <dO, o> per (token, head), [B*T*H*W*heads]
    float* part;        // backward: float32 partials [B*heads][nslab][G][D] of dGK, then of dGV
    int64_t ntok_b;     // tokens per batch item (T*H*W)
    int32_t B, heads, G;
    int32_t nslab;      // query slabs per (batch, head) in the partial sums
    int32_t gchunk;     // global rows staged per round
    float scale;
};

// Stage global rows [g0, g0 + n) of (b, eta) of GK and GV into LDS as
// [n][D] each (cooperative 16-byte copies).
template <typename T, int D>
__device__ __forceinline__ void stage_rows(const HybArgs& a, int32_t b, int32_t eta, int32_t g0, int32_t n, T* sk,
                                           T* sv) {
    constexpr int PIECES = D / 8;  // 8 elements per piece
    const T* gk = reinterpret_cast<const T*>(a.gk);
    const T* gv = reinterpret_cast<const T*>(a.gv);
    for (int i = threadIdx.x; i < n * PIECES; i += blockDim.x) {
        const int r = i / PIECES, c = (i - r * PIECES) * 8;
        const int64_t src = (((int64_t)b * a.G + g0 + r) * a.heads + eta) * D + c;
        Frag8<T> fk, fv;
        fk.load(gk + src);
        fv.load(gv + src);
        fk.store(sk + r * D + c);
        fv.store(sv + r * D + c);
    }
}

}  // namespace

// Forward: per query (L = D/8 lanes, 8 channels each), the global logits in an
// online softmax over the staged rows, then the exact merge with the local
// (o, lse). A block takes kHybRounds groups of 256/L consecutive tokens of
// one (batch, head); every thread reaches every barrier.
template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_fwd_kernel(HybArgs a) {
    constexpr int L = D / 8;
    constexpr int QPB = 256 / L;
    __shared__ __attribute__((aligned(16))) char lds[kHybLds];
    T* sk = reinterpret_cast<T*>(lds);
    T* sv = sk + a.gchunk * D;
    const int grp = threadIdx.x / L, li = threadIdx.x % L;
    const int64_t blocks_bh = (a.ntok_b + QPB * kHybRounds - 1) / (QPB * kHybRounds);
    const int64_t bh = blockIdx.x / blocks_bh;
    const int64_t t0 = (blockIdx.x - bh * blocks_bh) * (QPB * kHybRounds);
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int64_t C = (int64_t)a.heads * D;
    float m[kHybRounds], z[kHybRounds], acc[kHybRounds][8];
    Frag8<T> qf[kHybRounds];
    bool valid[kHybRounds];
    int64_t tok[kHybRounds];
#pragma unroll
    for (int r = 0; r < kHybRounds; ++r) {
        const int64_t tl = t0 + r * QPB + grp;
        valid[r] = tl < a.ntok_b;
        tok[r] = (int64_t)b * a.ntok_b + (valid[r] ? tl : 0);  // an invalid group reads token 0, stores nothing
        qf[r].load(reinterpret_cast<const T*>(a.q) + tok[r] * C + (int64_t)eta * D + li * 8);
        m[r] = -INFINITY;
        z[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
    }
    for (int32_t g0 = 0; g0 < a.G; g0 += a.gchunk) {
        const int32_t n = min(a.gchunk, a.G - g0);
        __syncthreads();  // the previous chunk has been read
        stage_rows<T, D>(a, b, eta, g0, n, sk, sv);
        __syncthreads();
        for (int32_t g = 0; g < n; ++g) {
            Frag8<T> kf, vf;
            kf.load(sk + g * D + li * 8);
            vf.load(sv + g * D + li * 8);
#pragma unroll
            for (int r = 0; r < kHybRounds; ++r) {
                const float s = a.scale * group_sum<L>(kf.dot(qf[r], 0.0f));
                const float m_new = fmaxf(m[r], s);
                const float alpha = __expf(m[r] - m_new);
                const float beta = __expf(s - m_new);
                z[r] = fmaf(z[r], alpha, beta);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
                vf.axpy(beta, acc[r]);
                m[r] = m_new;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kHybRounds; ++r) {
        if (!valid[r]) continue;
        T* orow = reinterpret_cast<T*>(a.out) + tok[r] * C + (int64_t)eta * D + li * 8;
        float* lp = a.lse + tok[r] * a.heads + eta;
        const float l1 = *lp;
        const float l2 = m[r] + __logf(z[r]);
        const float mx = fmaxf(l1, l2);
        const float lse = mx + __logf(__expf(l1 - mx) + __expf(l2 - mx));
        const float w1 = __expf(l1 - lse), w2 = __expf(m[r] - lse);
        Frag8<T> of;
        of.load(orow);
        float o[8];
        of.to_f32(o);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w1, o[e], w2 * acc[r][e]);
        of.from_f32(o);
        of.store(orow);
        if (li == 0) *lp = lse;
    }
}

// Backward, query side: a_g = e^{s_g - lse}, da_g = <dO, GV[g]>,
// ds_g = a_g (da_g - <dO, o>), dq += scale sum_g ds_g GK[g] (added to the local
// dq, one rounding); <dO, o> is left in `dsum` for the global rows' kernel.
template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_bwd_query_kernel(HybArgs a) {
    constexpr int L = D / 8;
    constexpr int QPB = 256 / L;
    __shared__ __attribute__((aligned(16))) char lds[kHybLds];
    T* sk = reinterpret_cast<T*>(lds);
    T* sv = sk + a.gchunk * D;
    const int grp = threadIdx.x / L, li = threadIdx.x % L;
    const int64_t blocks_bh = (a.ntok_b + QPB * kHybRounds - 1) / (QPB * kHybRounds);
    const int64_t bh = blockIdx.x / blocks_bh;
    const int64_t t0 = (blockIdx.x - bh * blocks_bh) * (QPB * kHybRounds);
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int64_t C = (int64_t)a.heads * D;
    Frag8<T> qf[kHybRounds], gf[kHybRounds];
    float lse[kHybRounds], dsum[kHybRounds], dq[kHybRounds][8];
    bool valid[kHybRounds];
    int64_t tok[kHybRounds];
#pragma unroll
    for (int r = 0; r < kHybRounds; ++r) {
        const int64_t tl = t0 + r * QPB + grp;
        valid[r] = tl < a.ntok_b;
        tok[r] = (int64_t)b * a.ntok_b + (valid[r] ? tl : 0);
        const int64_t off = tok[r] * C + (int64_t)eta * D + li * 8;
        // an invalid group reads the (in-range) row of token 0 and stores nothing
        qf[r].load(reinterpret_cast<const T*>(a.q) + off);
        gf[r].load(reinterpret_cast<const T*>(a.dout) + off);
        Frag8<T> of;
        of.load(reinterpret_cast<const T*>(a.out) + off);
        dsum[r] = group_sum<L>(gf[r].dot(of, 0.0f));
        lse[r] = a.lse[tok[r] * a.heads + eta];
#pragma unroll
        for (int e = 0; e < 8; ++e) dq[r][e] = 0.0f;
    }
    for (int32_t g0 = 0; g0 < a.G; g0 += a.gchunk) {
        const int32_t n = min(a.gchunk, a.G - g0);
        __syncthreads();
        stage_rows<T, D>(a, b, eta, g0, n, sk, sv);
        __syncthreads();
        for (int32_t g = 0; g < n; ++g) {
            Frag8<T> kf, vf;
            kf.load(sk + g * D + li * 8);
            vf.load(sv + g * D + li * 8);
#pragma unroll
            for (int r = 0; r < kHybRounds; ++r) {
                const float s = a.scale * group_sum<L>(kf.dot(qf[r], 0.0f));
                const float da = group_sum<L>(vf.dot(gf[r], 0.0f));
                const float ag = __expf(s - lse[r]);
                const float ds = ag * (da - dsum[r]);
                kf.axpy(a.scale * ds, dq[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kHybRounds; ++r) {
        if (!valid[r]) continue;
        T* p = reinterpret_cast<T*>(a.dq) + tok[r] * C + (int64_t)eta * D + li * 8;
        Frag8<T> f;
        f.load(p);
        float x[8];
        f.to_f32(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += dq[r][e];
        f.from_f32(x);
        f.store(p);
        if (li == 0) a.dsum[tok[r] * a.heads + eta] = dsum[r];
    }
}

// Backward, global rows: one block per (batch*head, slab of queries, chunk of
// 256/L global rows); lane group gl owns global row g0 + gl and lane li its
// channels 8li .. 8li+7, keeping that row's GK/GV piece and its dGK/dGV sums in
// registers. The slab's queries pass through LDS in tiles of kTile (rows of q
// and dO, lse and <dO, o>), in token order, so each sum runs in a fixed order.
constexpr int kTile = 32;

template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_bwd_rows_kernel(HybArgs a) {
    constexpr int L = D / 8;
    constexpr int GPB = 256 / L;  // global rows per block
    __shared__ __attribute__((aligned(16))) T sq[kTile * D];
    __shared__ __attribute__((aligned(16))) T sg[kTile * D];
    __shared__ float slse[kTile], sds[kTile];
    const int gl = threadIdx.x / L, li = threadIdx.x % L;
    const int32_t ngc = (a.G + GPB - 1) / GPB;
    const int64_t per_bh = (int64_t)a.nslab * ngc;
    const int64_t bh = blockIdx.x / per_bh;
    const int32_t rem = (int32_t)(blockIdx.x - bh * per_bh);
    const int32_t slab = rem / ngc, gc = rem - slab * ngc;
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int32_t g = gc * GPB + gl;
    const bool gvalid = g < a.G;
    const int64_t C = (int64_t)a.heads * D;
    const int64_t per_slab = (a.ntok_b + a.nslab - 1) / a.nslab;
    const int64_t x0 = (int64_t)slab * per_slab, x1 = min(a.ntok_b, x0 + per_slab);
    Frag8<T> kf, vf;
    {
        const int64_t src = (((int64_t)b * a.G + (gvalid ? g : 0)) * a.heads + eta) * D + li * 8;
        kf.load(reinterpret_cast<const T*>(a.gk) + src);
        vf.load(reinterpret_cast<const T*>(a.gv) + src);
    }
    float dk[8], dv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { dk[e] = 0.0f; dv[e] = 0.0f; }
    constexpr int PIECES = D / 8;
    for (int64_t xt = x0; xt < x1; xt += kTile) {
        const int n = (int)min((int64_t)kTile, x1 - xt);
        __syncthreads();  // the previous tile has been read
        for (int i = threadIdx.x; i < n * PIECES; i += blockDim.x) {
            const int r = i / PIECES, c = (i - r * PIECES) * 8;
            const int64_t off = ((int64_t)b * a.ntok_b + xt + r) * C + (int64_t)eta * D + c;
            Frag8<T> f;
            f.load(reinterpret_cast<const T*>(a.q) + off);
            f.store(sq + r * D + c);
            f.load(reinterpret_cast<const T*>(a.dout) + off);
            f.store(sg + r * D + c);
        }
        if (threadIdx.x < n) {
            const int64_t i = ((int64_t)b * a.ntok_b + xt + threadIdx.x) * a.heads + eta;
            slse[threadIdx.x] = a.lse[i];
            sds[threadIdx.x] = a.dsum[i];
        }
        __syncthreads();
        for (int r = 0; r < n; ++r) {
            Frag8<T> qx, gx;
            qx.load(sq + r * D + li * 8);
            gx.load(sg + r * D + li * 8);
            const float s = a.scale * group_sum<L>(kf.dot(qx, 0.0f));
            const float da = group_sum<L>(vf.dot(gx, 0.0f));
            const float ag = __expf(s - slse[r]);
            const float ds = ag * (da - sds[r]);
            qx.axpy(a.scale * ds, dk);
            gx.axpy(ag, dv);
        }
    }
    if (gvalid) {
        const int64_t pk = (((bh * a.nslab + slab) * a.G) + g) * D + li * 8;
        const int64_t pv = pk + (int64_t)a.B * a.heads * a.nslab * a.G * D;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a.part[pk + e] = dk[e];
            a.part[pv + e] = dv[e];
        }
    }
}

// dGK / dGV [B, G, heads, D] = the sum over the slabs of the partials, slab by
// slab in increasing order, rounded once to the tensor's type.
template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_rows_sum_kernel(const float* part, T* dgk, T* dgv, int32_t B,
                                                                    int32_t heads, int32_t G, int32_t nslab) {
    const int64_t n = (int64_t)B * G * heads * D;
    const int64_t half = (int64_t)B * heads * nslab * G * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n; i += (int64_t)gridDim.x * blockDim.x) {
        const bool v = i >= n;
        const int64_t j = v ? i - n : i;  // index into [B, G, heads, D]
        const int32_t e = (int32_t)(j % D);
        const int64_t r = j / D;
        const int32_t eta = (int32_t)(r % heads);
        const int32_t g = (int32_t)((r / heads) % G);
        const int32_t b = (int32_t)(r / heads / G);
        const int64_t bh = (int64_t)b * heads + eta;
        const float* p = part + (v ? half : 0) + ((bh * nslab) * G + g) * D + e;
        float s = 0.0f;
        for (int32_t z = 0; z < nslab; ++z) s += p[(int64_t)z * G * D];
        store_scalar<T>((v ? dgv : dgk) + j, s);
    }
}

namespace {

HybArgs hyb_args(const dsa3d_desc& d, int32_t G) {
    HybArgs a{};
    a.ntok_b = d.T * d.H * d.W;
    a.B = (int32_t)d.B;
    a.heads = d.heads;
    a.G = G;
    a.scale = logit_scale(d);
    const int esz = d.dtype == DSA3D_F32 ? 4 : 2;
    a.gchunk = std::max(1, std::min<int>(G, kHybLds / (2 * d.head_dim * esz)));
    // slabs of at least 512 queries, about 2048 blocks in all
    const int64_t ngc = (G + 256 / (d.head_dim / 8) - 1) / (256 / (d.head_dim / 8));
    const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(1, d.B * d.heads * ngc));
    a.nslab = (int32_t)std::max<int64_t>(1, std::min<int64_t>(want, (a.ntok_b + 511) / 512));
    return a;
}

template <typename T, int D>
hipError_t hyb_fwd(const HybArgs& a, hipStream_t s) {
    constexpr int QPB = 256 / (D / 8);
    const int64_t blocks = (int64_t)a.B * a.heads * ((a.ntok_b + QPB * kHybRounds - 1) / (QPB * kHybRounds));
    LaunchScope ls(DSA3D_K_HYBRID_FORWARD, s);
    hipLaunchKernelGGL((dsa3d_hybrid_fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D> hipError_t hyb_fwd_f32(const HybArgs& a, hipStream_t s) { return hyb_fwd<float, D>(a, s); }
template <int D> hipError_t hyb_fwd_bf16(const HybArgs& a, hipStream_t s) { return hyb_fwd<bf16_t, D>(a, s); }

template <typename T, int D>
hipError_t hyb_bwd(const HybArgs& a, void* dgk, void* dgv, hipStream_t s) {
    constexpr int L = D / 8, QPB = 256 / L, GPB = 256 / L;
    const int64_t qblocks = (int64_t)a.B * a.heads * ((a.ntok_b + QPB * kHybRounds - 1) / (QPB * kHybRounds));
    {
        LaunchScope ls(DSA3D_K_HYBRID_BWD_QUERY, s);
        hipLaunchKernelGGL((dsa3d_hybrid_bwd_query_kernel<T, D>), dim3((unsigned)qblocks), dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ngc = (a.G + GPB - 1) / GPB;
    const int64_t rblocks = (int64_t)a.B * a.heads * a.nslab * ngc;
    {
        LaunchScope ls(DSA3D_K_HYBRID_BWD_ROWS, s);
        hipLaunchKernelGGL((dsa3d_hybrid_bwd_rows_kernel<T, D>), dim3((unsigned)rblocks), dim3(256), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = 2 * (int64_t)a.B * a.G * a.heads * D;
    LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
    hipLaunchKernelGGL((dsa3d_hybrid_rows_sum_kernel<T, D>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, a.part,
                       reinterpret_cast<T*>(dgk), reinterpret_cast<T*>(dgv), a.B, a.heads, a.G, a.nslab);
    return hipGetLastError();
}
template <int D> hipError_t hyb_bwd_f32(const HybArgs& a, void* k, void* v, hipStream_t s) { return hyb_bwd<float, D>(a, k, v, s); }
template <int D> hipError_t hyb_bwd_bf16(const HybArgs& a, void* k, void* v, hipStream_t s) { return hyb_bwd<bf16_t, D>(a, k, v, s); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t hybrid_global_workspace_bytes(const dsa3d_desc& d, int32_t G) {
    const HybArgs a = hyb_args(d, G);
    const size_t dsum = (size_t)(d.B * d.T * d.H * d.W) * d.heads * 4;
    const size_t part = 2 * (size_t)d.B * d.heads * a.nslab * G * d.head_dim * 4;
    return align256(dsum) + align256(part);
}

hipError_t launch_hybrid_forward(const dsa3d_desc& d, int32_t G, const void* q, const void* gk, const void* gv,
                                 void* out, float* lse, hipStream_t s) {
    if (G == 0 || d.B * d.T * d.H * d.W == 0) return hipSuccess;
    HybArgs a = hyb_args(d, G);
    a.q = q; a.gk = gk; a.gv = gv; a.out = out; a.lse = lse;
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, hyb_fwd_f32, a, s); }
    DSA3D_DISPATCH_D(d.head_dim, hyb_fwd_bf16, a, s);
}

hipError_t launch_hybrid_backward(const dsa3d_desc& d, int32_t G, const void* q, const void* gk, const void* gv,
                                  const void* out, const float* lse, const void* dout, void* dq, void* dgk, void* dgv,
                                  void* ws, hipStream_t s) {
    if (d.B * d.T * d.H * d.W == 0) return hipSuccess;
    if (G == 0) return hipSuccess;
    HybArgs a = hyb_args(d, G);
    a.q = q; a.gk = gk; a.gv = gv; a.out = const_cast<void*>(out); a.lse = const_cast<float*>(lse);
    a.dout = dout; a.dq = dq;
    a.dsum = reinterpret_cast<float*>(ws);
    a.part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      align256((size_t)(d.B * d.T * d.H * d.W) * d.heads * 4));
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, hyb_bwd_f32, a, dgk, dgv, s); }
    DSA3D_DISPATCH_D(d.head_dim, hyb_bwd_bf16, a, dgk, dgv, s);
}

}  // namespace dsa3d
