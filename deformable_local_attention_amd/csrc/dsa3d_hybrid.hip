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
// bf16 rows of 32, 64 or 128 channels run the three steps on the matrix cores
// (the products below); other rows run them on the vector units, where a
// global row is read by every query of a block from LDS, staged there once.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"
#include "dsa3d_mfma.h"

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

// ---------------------------------------------------------------------------
// The same three steps on the matrix cores, for bf16 rows of 32, 64 or 128
// channels: every query of a (batch, head) meets the same G global rows, so
// the logits and the weighted sums are dense products (16x16x32 bf16, float32
// accumulation). A block stages the global rows in LDS, 64 at a time, rows
// past G as zeros.
//
// Per-query kernels: a wave takes 16 consecutive queries (query c = lane%16)
// and walks the staged rows in slices of 32 keys:
//   S^T = GK_slice Q^T                 (two 16-key tiles, D/32 products each)
//   keys >= G -> -inf, online softmax per query (lazy maximum),
//   O^T += GV_slice^T P^T              (forward)
//   dP^T = GV_slice dO^T, dS = P (dP - <dO, o>), dq^T += GK_slice^T (scale dS)^T
//                                      (backward)
// The second product's k-slice for lane group g = lane/16 is the key set
// {4g..4g+3, 16+4g..16+4g+3}, where the first product left that group's
// logits, so the weights enter without data movement; they are split into a
// bf16 part and a bf16 remainder (two products) so that they keep about 2^-17
// relative precision. The first operand of the second product is read from
// LDS a channel pair at a time and sorted into even and odd channels, so a
// lane ends up with 8 consecutive channels 32*tau + 8g .. +7 of query c.
//
// Global rows' kernel: a block takes 64 keys (16 per wave, key c of wave w =
// row 64*chunk + 16w + c) and one slab of queries, which pass through LDS 32
// at a time:
//   S = Q_tile GK^T, dP = dO_tile GV^T  (two 16-query tiles; D[4g + r][c] is
//                                        query 16*QT + 4g + r, key c)
//   dGK^T += Q_tile^T (scale dS),  dGV^T += dO_tile^T P
// with the same k-slice trick over the tile's 32 queries; the slab's float32
// sums go to the partials, summed in slab order as on the vector units.
// ---------------------------------------------------------------------------
constexpr int kHybMfKeys = 64;    // global rows staged per round
constexpr int kHybMfRounds = 8;   // 64-query tiles per block in the per-query kernels
constexpr int kHybMfTile = 32;    // queries per LDS tile in the global rows' kernel

bool hybrid_on_mfma(const dsa3d_desc& d) {
    return d.dtype == DSA3D_BF16 && (d.head_dim == 32 || d.head_dim == 64 || d.head_dim == 128);
}

namespace {

// Rows [g0, g0 + 64) of (b, eta) of GK and GV into LDS, [64][D + 8] each; rows
// past G are zero.
template <int D>
__device__ __forceinline__ void stage_rows_mf(const HybArgs& a, int32_t b, int32_t eta, int32_t g0, bf16_t* sk,
                                              bf16_t* sv) {
    constexpr int RS = D + 8, PIECES = D / 8;
    const bf16_t* gk = reinterpret_cast<const bf16_t*>(a.gk);
    const bf16_t* gv = reinterpret_cast<const bf16_t*>(a.gv);
    for (int i = threadIdx.x; i < kHybMfKeys * PIECES; i += 256) {
        const int r = i / PIECES, c = (i - r * PIECES) * 8;
        uint4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        if (g0 + r < a.G) {
            const int64_t src = (((int64_t)b * a.G + g0 + r) * a.heads + eta) * D + c;
            xk = *reinterpret_cast<const uint4*>(gk + src);
            xv = *reinterpret_cast<const uint4*>(gv + src);
        }
        *reinterpret_cast<uint4*>(sk + r * RS + c) = xk;
        *reinterpret_cast<uint4*>(sv + r * RS + c) = xv;
    }
}

// The second operand of the products over a key (or query) slice: rows
// {4g..4g+3, 16+4g..16+4g+3} of `base` (row stride RS), channels col, col + 1
// of each, sorted into the even channel (e) and the odd one (o).
template <int RS>
__device__ __forceinline__ void slice_pairs(const bf16_t* base, int g, mf_bf16x8& e, mf_bf16x8& o) {
    uint32_t d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = i < 4 ? 4 * g + i : 12 + 4 * g + i;
        d[i] = *reinterpret_cast<const uint32_t*>(base + row * RS);
    }
    mf_u32x4 ve, vo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ve[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x05040100u);
        vo[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07060302u);
    }
    e = __builtin_bit_cast(mf_bf16x8, ve);
    o = __builtin_bit_cast(mf_bf16x8, vo);
}

__device__ __forceinline__ float dot8_bf16(const uint4& x, const uint4& y) {
    float c = dot2_bf16(x.x, y.x, 0.0f);
    c = dot2_bf16(x.y, y.y, c);
    c = dot2_bf16(x.z, y.z, c);
    return dot2_bf16(x.w, y.w, c);
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_fwd_mfma_kernel(HybArgs a) {
    constexpr int RS = D + 8, NJ = D / 32, QPB = 64 * kHybMfRounds;
    __shared__ __attribute__((aligned(16))) bf16_t sk[kHybMfKeys * RS];
    __shared__ __attribute__((aligned(16))) bf16_t sv[kHybMfKeys * RS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int64_t blocks_bh = (a.ntok_b + QPB - 1) / QPB;
    const int64_t bh = blockIdx.x / blocks_bh;
    const int64_t x0 = (blockIdx.x - bh * blocks_bh) * QPB;
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int64_t C = (int64_t)a.heads * D;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);  // 512 zero elements
    const bool one_round = a.G <= kHybMfKeys;
    if (one_round) {
        stage_rows_mf<D>(a, b, eta, 0, sk, sv);
        __syncthreads();
    }
    for (int r = 0; r < kHybMfRounds; ++r) {
        const int64_t xl = x0 + r * 64 + wv * 16 + c;  // query c of this wave (token within the batch item)
        const bool qin = xl < a.ntok_b;
        const int64_t tok = (int64_t)b * a.ntok_b + (qin ? xl : 0);
        const int64_t row = tok * C + (int64_t)eta * D;
        mf_bf16x8 qb[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            qb[j] = *reinterpret_cast<const mf_bf16x8*>(qin ? q + row + 32 * j + 8 * g : zero);
        mf_f32x4 oacc[NJ][2];
#pragma unroll
        for (int tau = 0; tau < NJ; ++tau) oacc[tau][0] = oacc[tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, lsum = 0.0f;
        for (int32_t g0 = 0; g0 < a.G; g0 += kHybMfKeys) {
            if (!one_round) {
                __syncthreads();  // the previous rows have been read
                stage_rows_mf<D>(a, b, eta, g0, sk, sv);
                __syncthreads();
            }
            for (int sl = 0; sl < kHybMfKeys / 32 && g0 + 32 * sl < a.G; ++sl) {
                const bf16_t* ks = sk + 32 * sl * RS;
                const bf16_t* vs = sv + 32 * sl * RS;
                mf_f32x4 sacc[2];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    sacc[T] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const mf_bf16x8*>(ks + (16 * T + c) * RS + 32 * j + 8 * g), qb[j],
                            sacc[T], 0, 0, 0);
                }
                float sv8[8];
                float mloc = -INFINITY;
#pragma unroll
                for (int i = 0; i < 8; ++i) {  // key 16*(i/4) + 4g + i%4 of the slice
                    const int32_t key = g0 + 32 * sl + 16 * (i >> 2) + 4 * g + (i & 3);
                    sv8[i] = key < a.G ? a.scale * sacc[i >> 2][i & 3] : -INFINITY;
                    mloc = fmaxf(mloc, sv8[i]);
                }
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
                if (!__all(mloc <= m + kMfmaLazyMax)) {  // always on the first slice (m = -inf)
                    const float m_new = fmaxf(m, mloc);
                    const float alpha = __expf(m - m_new);
#pragma unroll
                    for (int tau = 0; tau < NJ; ++tau) {
                        oacc[tau][0] *= alpha;
                        oacc[tau][1] *= alpha;
                    }
                    lsum *= alpha;
                    m = m_new;
                }
                mf_u32x4 phi, plo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __expf(sv8[2 * i] - m), p1 = __expf(sv8[2 * i + 1] - m);
                    lsum += p0 + p1;
                    const uint2 h = mf_split(p0, p1);
                    phi[i] = h.x;
                    plo[i] = h.y;
                }
                const mf_bf16x8 pb_hi = __builtin_bit_cast(mf_bf16x8, phi), pb_lo = __builtin_bit_cast(mf_bf16x8, plo);
#pragma unroll
                for (int tau = 0; tau < NJ; ++tau) {
                    mf_bf16x8 vE, vO;
                    slice_pairs<RS>(vs + 32 * tau + 2 * c, g, vE, vO);
                    oacc[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vE, pb_hi, oacc[tau][0], 0, 0, 0);
                    oacc[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vE, pb_lo, oacc[tau][0], 0, 0, 0);
                    oacc[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vO, pb_hi, oacc[tau][1], 0, 0, 0);
                    oacc[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vO, pb_lo, oacc[tau][1], 0, 0, 0);
                }
            }
        }
        float l = lsum;
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (!qin) continue;
        // merge with the local (o, lse) of this query: lse = log(e^{lse_l} + l e^m)
        float* lp = a.lse + tok * a.heads + eta;
        const float l1 = *lp;
        const float l2 = m + __logf(l);
        const float mx = fmaxf(l1, l2);
        const float lse = mx + __logf(__expf(l1 - mx) + __expf(l2 - mx));
        const float w1 = __expf(l1 - lse), w2 = __expf(m - lse);
        bf16_t* orow = reinterpret_cast<bf16_t*>(a.out) + row;
#pragma unroll
        for (int tau = 0; tau < NJ; ++tau) {  // channels 32*tau + 8g + 2r + par
            uint4* p = reinterpret_cast<uint4*>(orow + 32 * tau + 8 * g);
            const uint4 ol = *p;
            const uint32_t w[4] = {ol.x, ol.y, ol.z, ol.w};
            uint32_t o[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                o[rr] = pack_bf16x2(fmaf(w1, bf16_lo(w[rr]), w2 * oacc[tau][0][rr]),
                                    fmaf(w1, bf16_hi(w[rr]), w2 * oacc[tau][1][rr]));
            *p = uint4{o[0], o[1], o[2], o[3]};
        }
        if (g == 0) *lp = lse;
    }
}

template <int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_bwd_query_mfma_kernel(HybArgs a) {
    constexpr int RS = D + 8, NJ = D / 32, QPB = 64 * kHybMfRounds;
    __shared__ __attribute__((aligned(16))) bf16_t sk[kHybMfKeys * RS];
    __shared__ __attribute__((aligned(16))) bf16_t sv[kHybMfKeys * RS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int64_t blocks_bh = (a.ntok_b + QPB - 1) / QPB;
    const int64_t bh = blockIdx.x / blocks_bh;
    const int64_t x0 = (blockIdx.x - bh * blocks_bh) * QPB;
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int64_t C = (int64_t)a.heads * D;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
    const bf16_t* dout = reinterpret_cast<const bf16_t*>(a.dout);
    const bf16_t* out = reinterpret_cast<const bf16_t*>(a.out);
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);
    const bool one_round = a.G <= kHybMfKeys;
    if (one_round) {
        stage_rows_mf<D>(a, b, eta, 0, sk, sv);
        __syncthreads();
    }
    for (int r = 0; r < kHybMfRounds; ++r) {
        const int64_t xl = x0 + r * 64 + wv * 16 + c;
        const bool qin = xl < a.ntok_b;
        const int64_t tok = (int64_t)b * a.ntok_b + (qin ? xl : 0);
        const int64_t row = tok * C + (int64_t)eta * D;
        mf_bf16x8 qb[NJ], gb[NJ];
        float dpart = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            qb[j] = *reinterpret_cast<const mf_bf16x8*>(qin ? q + row + 32 * j + 8 * g : zero);
            gb[j] = *reinterpret_cast<const mf_bf16x8*>(qin ? dout + row + 32 * j + 8 * g : zero);
            const uint4 ov = *reinterpret_cast<const uint4*>(qin ? out + row + 32 * j + 8 * g : zero);
            dpart = dpart + dot8_bf16(__builtin_bit_cast(uint4, gb[j]), ov);
        }
        dpart += __shfl_xor(dpart, 16, 64);
        dpart += __shfl_xor(dpart, 32, 64);
        const float dsum = dpart;  // <dO, o> of query c
        const float lse = qin ? a.lse[tok * a.heads + eta] : 0.0f;
        mf_f32x4 dacc[NJ][2];
#pragma unroll
        for (int tau = 0; tau < NJ; ++tau) dacc[tau][0] = dacc[tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t g0 = 0; g0 < a.G; g0 += kHybMfKeys) {
            if (!one_round) {
                __syncthreads();
                stage_rows_mf<D>(a, b, eta, g0, sk, sv);
                __syncthreads();
            }
            for (int sl = 0; sl < kHybMfKeys / 32 && g0 + 32 * sl < a.G; ++sl) {
                const bf16_t* ks = sk + 32 * sl * RS;
                const bf16_t* vs = sv + 32 * sl * RS;
                mf_f32x4 sacc[2], pacc[2];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    sacc[T] = pacc[T] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int e = (16 * T + c) * RS + 32 * j + 8 * g;
                        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const mf_bf16x8*>(ks + e), qb[j], sacc[T], 0, 0, 0);
                        pacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const mf_bf16x8*>(vs + e), gb[j], pacc[T], 0, 0, 0);
                    }
                }
                float ck[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int32_t key = g0 + 32 * sl + 16 * (i >> 2) + 4 * g + (i & 3);
                    const float p = __expf(a.scale * sacc[i >> 2][i & 3] - lse);
                    ck[i] = key < a.G ? a.scale * (p * (pacc[i >> 2][i & 3] - dsum)) : 0.0f;
                }
                mf_u32x4 shi, slo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint2 h = mf_split(ck[2 * i], ck[2 * i + 1]);
                    shi[i] = h.x;
                    slo[i] = h.y;
                }
                const mf_bf16x8 ds_hi = __builtin_bit_cast(mf_bf16x8, shi), ds_lo = __builtin_bit_cast(mf_bf16x8, slo);
#pragma unroll
                for (int tau = 0; tau < NJ; ++tau) {
                    mf_bf16x8 kE, kO;
                    slice_pairs<RS>(ks + 32 * tau + 2 * c, g, kE, kO);
                    dacc[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kE, ds_hi, dacc[tau][0], 0, 0, 0);
                    dacc[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kE, ds_lo, dacc[tau][0], 0, 0, 0);
                    dacc[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kO, ds_hi, dacc[tau][1], 0, 0, 0);
                    dacc[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kO, ds_lo, dacc[tau][1], 0, 0, 0);
                }
            }
        }
        if (!qin) continue;
        bf16_t* drow = reinterpret_cast<bf16_t*>(a.dq) + row;
#pragma unroll
        for (int tau = 0; tau < NJ; ++tau) {  // the local dq plus the global rows' share, one rounding
            uint4* p = reinterpret_cast<uint4*>(drow + 32 * tau + 8 * g);
            const uint4 dl = *p;
            const uint32_t w[4] = {dl.x, dl.y, dl.z, dl.w};
            uint32_t o[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                o[rr] = pack_bf16x2(bf16_lo(w[rr]) + dacc[tau][0][rr], bf16_hi(w[rr]) + dacc[tau][1][rr]);
            *p = uint4{o[0], o[1], o[2], o[3]};
        }
        if (g == 0) a.dsum[tok * a.heads + eta] = dsum;
    }
}

template <int D>
__global__ void __launch_bounds__(256) dsa3d_hybrid_bwd_rows_mfma_kernel(HybArgs a) {
    constexpr int RS = D + 8, NJ = D / 32, PIECES = D / 8;
    __shared__ __attribute__((aligned(16))) bf16_t sq[kHybMfTile * RS];
    __shared__ __attribute__((aligned(16))) bf16_t sg[kHybMfTile * RS];
    __shared__ float slse[kHybMfTile], sds[kHybMfTile];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int32_t ngc = (a.G + kHybMfKeys - 1) / kHybMfKeys;
    const int64_t per_bh = (int64_t)a.nslab * ngc;
    const int64_t bh = blockIdx.x / per_bh;
    const int32_t rem = (int32_t)(blockIdx.x - bh * per_bh);
    const int32_t slab = rem / ngc, gc = rem - slab * ngc;
    const int32_t b = (int32_t)(bh / a.heads), eta = (int32_t)(bh - (int64_t)b * a.heads);
    const int32_t key = gc * kHybMfKeys + wv * 16 + c;  // this lane's key (column of the products)
    const bool kin = key < a.G;
    const int64_t C = (int64_t)a.heads * D;
    const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero_row);
    mf_bf16x8 kb[NJ], vb[NJ];
    {
        const int64_t src = (((int64_t)b * a.G + (kin ? key : 0)) * a.heads + eta) * D + 8 * g;
        const bf16_t* gk = reinterpret_cast<const bf16_t*>(a.gk) + src;
        const bf16_t* gv = reinterpret_cast<const bf16_t*>(a.gv) + src;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            kb[j] = *reinterpret_cast<const mf_bf16x8*>(kin ? gk + 32 * j : zero);
            vb[j] = *reinterpret_cast<const mf_bf16x8*>(kin ? gv + 32 * j : zero);
        }
    }
    mf_f32x4 dk[NJ][2], dv[NJ][2];
#pragma unroll
    for (int tau = 0; tau < NJ; ++tau) dk[tau][0] = dk[tau][1] = dv[tau][0] = dv[tau][1] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t per_slab = (a.ntok_b + a.nslab - 1) / a.nslab;
    const int64_t x0 = (int64_t)slab * per_slab, x1 = min(a.ntok_b, x0 + per_slab);
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q) + (int64_t)eta * D;
    const bf16_t* dout = reinterpret_cast<const bf16_t*>(a.dout) + (int64_t)eta * D;
    for (int64_t xt = x0; xt < x1; xt += kHybMfTile) {
        const int n = (int)min((int64_t)kHybMfTile, x1 - xt);
        __syncthreads();  // the previous tile has been read
        for (int i = threadIdx.x; i < kHybMfTile * PIECES; i += 256) {
            const int rr = i / PIECES, cc = (i - rr * PIECES) * 8;
            uint4 xq = {0u, 0u, 0u, 0u}, xg = {0u, 0u, 0u, 0u};
            if (rr < n) {
                const int64_t off = ((int64_t)b * a.ntok_b + xt + rr) * C + cc;
                xq = *reinterpret_cast<const uint4*>(q + off);
                xg = *reinterpret_cast<const uint4*>(dout + off);
            }
            *reinterpret_cast<uint4*>(sq + rr * RS + cc) = xq;
            *reinterpret_cast<uint4*>(sg + rr * RS + cc) = xg;
        }
        if (threadIdx.x < kHybMfTile) {
            float l = 0.0f, d = 0.0f;
            if ((int)threadIdx.x < n) {
                const int64_t i = ((int64_t)b * a.ntok_b + xt + threadIdx.x) * a.heads + eta;
                l = a.lse[i];
                d = a.dsum[i];
            }
            slse[threadIdx.x] = l;
            sds[threadIdx.x] = d;
        }
        __syncthreads();
        mf_f32x4 s[2], dp[2];
#pragma unroll
        for (int QT = 0; QT < 2; ++QT) {
            s[QT] = dp[QT] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e = (16 * QT + c) * RS + 32 * j + 8 * g;
                s[QT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const mf_bf16x8*>(sq + e), kb[j],
                                                                s[QT], 0, 0, 0);
                dp[QT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const mf_bf16x8*>(sg + e), vb[j],
                                                                 dp[QT], 0, 0, 0);
            }
        }
        float pw[8], cw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // query 16*(i/4) + 4g + i%4 of the tile, key c
            const int qi = 16 * (i >> 2) + 4 * g + (i & 3);
            const float p = qi < n ? __expf(a.scale * s[i >> 2][i & 3] - slse[qi]) : 0.0f;
            pw[i] = p;
            cw[i] = a.scale * (p * (dp[i >> 2][i & 3] - sds[qi]));
        }
        mf_u32x4 phi, plo, chi, clo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint2 hp = mf_split(pw[2 * i], pw[2 * i + 1]), hc = mf_split(cw[2 * i], cw[2 * i + 1]);
            phi[i] = hp.x;
            plo[i] = hp.y;
            chi[i] = hc.x;
            clo[i] = hc.y;
        }
        const mf_bf16x8 p_hi = __builtin_bit_cast(mf_bf16x8, phi), p_lo = __builtin_bit_cast(mf_bf16x8, plo);
        const mf_bf16x8 c_hi = __builtin_bit_cast(mf_bf16x8, chi), c_lo = __builtin_bit_cast(mf_bf16x8, clo);
#pragma unroll
        for (int tau = 0; tau < NJ; ++tau) {
            mf_bf16x8 qE, qO, gE, gO;
            slice_pairs<RS>(sq + 32 * tau + 2 * c, g, qE, qO);
            slice_pairs<RS>(sg + 32 * tau + 2 * c, g, gE, gO);
            dk[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qE, c_hi, dk[tau][0], 0, 0, 0);
            dk[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qE, c_lo, dk[tau][0], 0, 0, 0);
            dk[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qO, c_hi, dk[tau][1], 0, 0, 0);
            dk[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qO, c_lo, dk[tau][1], 0, 0, 0);
            dv[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gE, p_hi, dv[tau][0], 0, 0, 0);
            dv[tau][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gE, p_lo, dv[tau][0], 0, 0, 0);
            dv[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gO, p_hi, dv[tau][1], 0, 0, 0);
            dv[tau][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gO, p_lo, dv[tau][1], 0, 0, 0);
        }
    }
    if (!kin) return;  // no barrier follows
    float* pk = a.part + (((bh * a.nslab + slab) * a.G) + key) * D + 8 * g;
    float* pv = pk + (int64_t)a.B * a.heads * a.nslab * a.G * D;
#pragma unroll
    for (int tau = 0; tau < NJ; ++tau) {  // channels 32*tau + 8g + 2r + par
        const mf_f32x4 &k0 = dk[tau][0], &k1 = dk[tau][1], &v0 = dv[tau][0], &v1 = dv[tau][1];
        reinterpret_cast<float4*>(pk + 32 * tau)[0] = make_float4(k0[0], k1[0], k0[1], k1[1]);
        reinterpret_cast<float4*>(pk + 32 * tau)[1] = make_float4(k0[2], k1[2], k0[3], k1[3]);
        reinterpret_cast<float4*>(pv + 32 * tau)[0] = make_float4(v0[0], v1[0], v0[1], v1[1]);
        reinterpret_cast<float4*>(pv + 32 * tau)[1] = make_float4(v0[2], v1[2], v0[3], v1[3]);
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
    const int rows_per_block = hybrid_on_mfma(d) ? kHybMfKeys : 256 / (d.head_dim / 8);
    const int64_t ngc = (G + rows_per_block - 1) / rows_per_block;
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

template <int D>
hipError_t hyb_fwd_mfma(const HybArgs& a, hipStream_t s) {
    constexpr int QPB = 64 * kHybMfRounds;
    const int64_t blocks = (int64_t)a.B * a.heads * ((a.ntok_b + QPB - 1) / QPB);
    LaunchScope ls(DSA3D_K_HYBRID_FORWARD, s);
    hipLaunchKernelGGL((dsa3d_hybrid_fwd_mfma_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t hyb_bwd_mfma(const HybArgs& a, void* dgk, void* dgv, hipStream_t s) {
    constexpr int QPB = 64 * kHybMfRounds;
    const int64_t qblocks = (int64_t)a.B * a.heads * ((a.ntok_b + QPB - 1) / QPB);
    {
        LaunchScope ls(DSA3D_K_HYBRID_BWD_QUERY, s);
        hipLaunchKernelGGL((dsa3d_hybrid_bwd_query_mfma_kernel<D>), dim3((unsigned)qblocks), dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ngc = (a.G + kHybMfKeys - 1) / kHybMfKeys;
    const int64_t rblocks = (int64_t)a.B * a.heads * a.nslab * ngc;
    {
        LaunchScope ls(DSA3D_K_HYBRID_BWD_ROWS, s);
        hipLaunchKernelGGL((dsa3d_hybrid_bwd_rows_mfma_kernel<D>), dim3((unsigned)rblocks), dim3(256), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = 2 * (int64_t)a.B * a.G * a.heads * D;
    LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
    hipLaunchKernelGGL((dsa3d_hybrid_rows_sum_kernel<bf16_t, D>), dim3(grid_for(n, 256, 65536)), dim3(256), 0, s,
                       a.part, reinterpret_cast<bf16_t*>(dgk), reinterpret_cast<bf16_t*>(dgv), a.B, a.heads, a.G,
                       a.nslab);
    return hipGetLastError();
}

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
    if (hybrid_on_mfma(d)) {
        switch (d.head_dim) {
            case 32: return hyb_fwd_mfma<32>(a, s);
            case 64: return hyb_fwd_mfma<64>(a, s);
            default: return hyb_fwd_mfma<128>(a, s);
        }
    }
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
    if (hybrid_on_mfma(d)) {
        switch (d.head_dim) {
            case 32: return hyb_bwd_mfma<32>(a, dgk, dgv, s);
            case 64: return hyb_bwd_mfma<64>(a, dgk, dgv, s);
            default: return hyb_bwd_mfma<128>(a, dgk, dgv, s);
        }
    }
    if (d.dtype == DSA3D_F32) { DSA3D_DISPATCH_D(d.head_dim, hyb_bwd_f32, a, dgk, dgv, s); }
    DSA3D_DISPATCH_D(d.head_dim, hyb_bwd_bf16, a, dgk, dgv, s);
}

}  // namespace dsa3d
