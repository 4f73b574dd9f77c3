// dsa3d_proj.hip -- offset projection GEMMs on the matrix cores (gfx950).
//
// Forward:  offsets[N_tok, F] = q[N_tok, C] . W[F, C]^T + b      (both operands K-contiguous)
// Backward: dq[N_tok, C]     += doff[N_tok, F] . W[F, C]          (B is N-contiguous)
//           dW[F, C]          = doff^T . q                        (split over N_tok, fixed-order sum)
//           db[F]             = column sums of doff               (split over N_tok, fixed-order sum)
//
// One kernel template covers all three products: a 128x128 output tile per
// 256-thread workgroup, four waves of 64x64, staged through LDS in 32-deep K
// slices stored K-contiguous (padded rows), consumed by
// v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (float32) with
// float32 accumulation. Operands stored M/N-contiguous are transposed while
// they are written to LDS.
#include "dsa3d_device.h"
#include "dsa3d_internal.h"

namespace dsa3d {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int BM = 128, BN = 128, BK = 32;

enum GemmOut { OUT_BIAS = 0, OUT_ACCUM = 1, OUT_PARTIAL = 2 };

struct GemmArgs {
    const void* A;  // a(m,k) = A[m*lda + k] if A is K-contiguous else A[k*lda + m]
    const void* B;  // b(k,n) = B[n*ldb + k] if B is K-contiguous else B[k*ldb + n]
    int64_t lda, ldb;
    int64_t M, N, K;
    int64_t k_split;   // K range of one blockIdx.z slice (multiple of BK)
    void* C;           // output: dtype tensor (OUT_BIAS, OUT_ACCUM) or float32 partials
    int64_t ldc;
    const void* bias;  // [N] or null (OUT_BIAS)
    int a_vec, b_vec;  // 8-element vector loads are in bounds and aligned
};

template <typename T> struct LdsPad;
template <> struct LdsPad<bf16_t> { static constexpr int v = 8; };
template <> struct LdsPad<float> { static constexpr int v = 4; };

// Stage rows [r0, r0+128) x k-slice [k0, k0+32) of an operand into lds[128][BK+PAD].
template <typename T, bool KCONTIG>
__device__ __forceinline__ void stage_tile(const T* src, int64_t ld, int64_t rows, int64_t kend, int64_t r0,
                                           int64_t k0, bool vec, T* lds) {
    constexpr int S = BK + LdsPad<T>::v;
    const int tid = threadIdx.x;
    if (KCONTIG) {
        // 128 rows x 4 groups of 8 k
        for (int idx = tid; idx < BM * (BK / 8); idx += 256) {
            const int r = idx / (BK / 8), kc = (idx % (BK / 8)) * 8;
            const int64_t gr = r0 + r, gk = k0 + kc;
            T* dst = lds + r * S + kc;
            if (vec && gr < rows && gk + 8 <= kend) {
                Frag8<T> f;
                f.load(src + gr * ld + gk);
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<uint4*>(dst) = reinterpret_cast<const uint4&>(f);
                } else {
                    *reinterpret_cast<float4*>(dst) = reinterpret_cast<const float4*>(&f)[0];
                    *reinterpret_cast<float4*>(dst + 4) = reinterpret_cast<const float4*>(&f)[1];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool ok = gr < rows && gk + j < kend;
                    dst[j] = ok ? src[gr * ld + gk + j] : T(0);
                }
            }
        }
    } else {
        // 32 k x 16 groups of 8 rows; transposed into lds[row][k]
        for (int idx = tid; idx < BK * (BM / 8); idx += 256) {
            const int kk = idx / (BM / 8), rc = (idx % (BM / 8)) * 8;
            const int64_t gk = k0 + kk, gr = r0 + rc;
            T vals[8];
            if (vec && gk < kend && gr + 8 <= rows) {
                Frag8<T> f;
                f.load(src + gk * ld + gr);
                if constexpr (sizeof(T) == 2) {
                    const uint4 u = reinterpret_cast<const uint4&>(f);
                    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        vals[2 * j] = (T)(w[j] & 0xffffu);
                        vals[2 * j + 1] = (T)(w[j] >> 16);
                    }
                } else {
                    const float* fp = reinterpret_cast<const float*>(&f);
#pragma unroll
                    for (int j = 0; j < 8; ++j) vals[j] = fp[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool ok = gk < kend && gr + j < rows;
                    vals[j] = ok ? src[gk * ld + gr + j] : T(0);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) lds[(rc + j) * S + kk] = vals[j];
        }
    }
}

template <typename T>
__device__ __forceinline__ void mma_slice(const T* As, const T* Bs, int wm, int wn, int lane, f32x4_t acc[4][4]);

template <>
__device__ __forceinline__ void mma_slice<bf16_t>(const bf16_t* As, const bf16_t* Bs, int wm, int wn, int lane,
                                                  f32x4_t acc[4][4]) {
    constexpr int S = BK + 8;
    const int r = lane % 16, kg = (lane / 16) * 8;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 16 + r) * S + kg);
        b[i] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + i * 16 + r) * S + kg);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_slice<float>(const float* As, const float* Bs, int wm, int wn, int lane,
                                                 f32x4_t acc[4][4]) {
    constexpr int S = BK + 4;
    const int r = lane % 16, kq = lane / 16;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = As[(wm * 64 + i * 16 + r) * S + ks + kq];
            b[i] = Bs[(wn * 64 + i * 16 + r) * S + ks + kq];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

template <typename T, bool AK, bool BKC, int MODE>
__global__ void __launch_bounds__(256) dsa3d_gemm_kernel(GemmArgs g) {
    constexpr int S = BK + LdsPad<T>::v;
    __shared__ __attribute__((aligned(16))) T As[BM * S];
    __shared__ __attribute__((aligned(16))) T Bs[BN * S];
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const int wm = wv / 2, wn = wv % 2;
    // XCD-aware order over (m-tile, n-tile); n fastest within one m strip
    const uint32_t ntn = (uint32_t)((g.N + BN - 1) / BN);
    const uint32_t nblk = gridDim.x;
    const uint32_t lb = xcd_logical_block(blockIdx.x, nblk);
    const int64_t m0 = (int64_t)(lb / ntn) * BM, n0 = (int64_t)(lb % ntn) * BN;
    const int64_t kb = (int64_t)blockIdx.z * g.k_split;
    const int64_t ke = std::min<int64_t>(g.K, kb + g.k_split);
    const T* A = reinterpret_cast<const T*>(g.A);
    const T* B = reinterpret_cast<const T*>(g.B);

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = kb; k0 < ke; k0 += BK) {
        stage_tile<T, AK>(A, g.lda, g.M, ke, m0, k0, g.a_vec != 0, As);
        stage_tile<T, BKC>(B, g.ldb, g.N, ke, n0, k0, g.b_vec != 0, Bs);
        __syncthreads();
        mma_slice<T>(As, Bs, wm, wn, lane, acc);
        __syncthreads();
    }

    // accumulator layout: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + (lane / 16) * 4 + r;
                const int64_t n = n0 + wn * 64 + j * 16 + lane % 16;
                if (m >= g.M || n >= g.N) continue;
                const float x = acc[i][j][r];
                if (MODE == OUT_BIAS) {
                    const float bb = g.bias ? load_scalar<T>(reinterpret_cast<const T*>(g.bias) + n) : 0.0f;
                    store_scalar<T>(reinterpret_cast<T*>(g.C) + m * g.ldc + n, x + bb);
                } else if (MODE == OUT_ACCUM) {
                    T* p = reinterpret_cast<T*>(g.C) + m * g.ldc + n;
                    store_scalar<T>(p, load_scalar<T>(p) + x);
                } else {
                    reinterpret_cast<float*>(g.C)[(int64_t)blockIdx.z * g.M * g.ldc + m * g.ldc + n] = x;
                }
            }
}

// out[i] = sum_{z < nsplit} part[z*n + i], in order z = 0, 1, ...
__global__ void __launch_bounds__(256) dsa3d_split_sum_kernel(const float* part, float* out, int64_t n, int nsplit) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.0f;
        for (int z = 0; z < nsplit; ++z) s += part[(int64_t)z * n + i];
        out[i] = s;
    }
}

// part[z*F + f] = sum over rows of slice z of g[row, f], rows in increasing order.
template <typename T>
__global__ void __launch_bounds__(256) dsa3d_colsum_kernel(const T* g, float* part, int64_t rows, int64_t F,
                                                           int64_t rows_per_split) {
    const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= F) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rows_per_split);
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) s += load_scalar<T>(g + r * F + f);
    part[(int64_t)blockIdx.y * F + f] = s;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T, bool AK, bool BKC, int MODE>
static hipError_t gemm(GemmArgs g, int splits, int kernel_id, hipStream_t s) {
    const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    LaunchScope ls(kernel_id, s);
    g.a_vec = (g.lda % 8 == 0) && aligned16(g.A);
    g.b_vec = (g.ldb % 8 == 0) && aligned16(g.B);
    hipLaunchKernelGGL((dsa3d_gemm_kernel<T, AK, BKC, MODE>), dim3((unsigned)tiles, 1, splits), dim3(256), 0, s, g);
    return hipGetLastError();
}

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Split counts of the two long reductions over the N_tok rows.
void proj_bwd_splits(const dsa3d_desc& d, int& dw_splits, int& db_splits) {
    const int64_t ntok = d.B * d.T * d.H * d.W;
    const int64_t F = (int64_t)d.heads * d.P * 3, C = (int64_t)d.heads * d.head_dim;
    const int64_t tiles = ((F + BM - 1) / BM) * ((C + BN - 1) / BN);
    int64_t s = (1024 + tiles - 1) / std::max<int64_t>(tiles, 1);
    s = std::max<int64_t>(1, std::min<int64_t>(s, std::max<int64_t>(1, ntok / (8 * BK))));
    s = std::min<int64_t>(s, 64);
    dw_splits = (int)s;
    const int64_t fb = (F + 255) / 256;
    int64_t sb = (1024 + fb - 1) / fb;
    sb = std::max<int64_t>(1, std::min<int64_t>(sb, std::max<int64_t>(1, ntok / 64)));
    db_splits = (int)std::min<int64_t>(sb, 256);
}

size_t proj_bwd_workspace_bytes(const dsa3d_desc& d) {
    int sw, sb;
    proj_bwd_splits(d, sw, sb);
    const int64_t F = (int64_t)d.heads * d.P * 3, C = (int64_t)d.heads * d.head_dim;
    return (size_t)sw * F * C * 4 + (size_t)sb * F * 4 + 256;
}

hipError_t launch_proj_forward(const dsa3d_desc& d, const void* q, const void* w, const void* bias, void* off,
                               hipStream_t s) {
    GemmArgs g{};
    g.A = q; g.lda = (int64_t)d.heads * d.head_dim;
    g.B = w; g.ldb = g.lda;
    g.M = d.B * d.T * d.H * d.W;
    g.N = (int64_t)d.heads * d.P * 3;
    g.K = g.lda;
    g.k_split = round_up(g.K, BK);
    g.C = off; g.ldc = g.N;
    g.bias = bias;
    if (d.dtype == DSA3D_F32) return gemm<float, true, true, OUT_BIAS>(g, 1, DSA3D_K_PROJ_FORWARD, s);
    return gemm<bf16_t, true, true, OUT_BIAS>(g, 1, DSA3D_K_PROJ_FORWARD, s);
}

hipError_t launch_proj_backward(const dsa3d_desc& d, const void* q, const void* w, const void* doff, void* dq,
                                float* dw, float* db, void* ws, hipStream_t s) {
    const int64_t ntok = d.B * d.T * d.H * d.W;
    const int64_t F = (int64_t)d.heads * d.P * 3, C = (int64_t)d.heads * d.head_dim;
    if (ntok == 0) return hipSuccess;
    const bool f32 = d.dtype == DSA3D_F32;
    hipError_t e;
    // dq[ntok, C] += doff[ntok, F] . W[F, C]
    GemmArgs g{};
    g.A = doff; g.lda = F;
    g.B = w; g.ldb = C;
    g.M = ntok; g.N = C; g.K = F;
    g.k_split = round_up(F, BK);
    g.C = dq; g.ldc = C;
    e = f32 ? gemm<float, true, false, OUT_ACCUM>(g, 1, DSA3D_K_PROJ_BWD_DQ, s)
              : gemm<bf16_t, true, false, OUT_ACCUM>(g, 1, DSA3D_K_PROJ_BWD_DQ, s);
    if (e != hipSuccess) return e;
    // dW[F, C] = doff^T . q, split over the token rows, then a fixed-order sum
    int sw, sb;
    proj_bwd_splits(d, sw, sb);
    float* part = reinterpret_cast<float*>(ws);
    GemmArgs h{};
    h.A = doff; h.lda = F;   // a(m=f, k=n) = doff[n*F + f]: M-contiguous
    h.B = q; h.ldb = C;      // b(k=n, n=c) = q[n*C + c]: N-contiguous
    h.M = F; h.N = C; h.K = ntok;
    h.k_split = round_up((ntok + sw - 1) / sw, BK);
    const int splits = (int)((ntok + h.k_split - 1) / h.k_split);
    h.C = part; h.ldc = C;
    e = f32 ? gemm<float, false, false, OUT_PARTIAL>(h, splits, DSA3D_K_PROJ_BWD_DW, s)
              : gemm<bf16_t, false, false, OUT_PARTIAL>(h, splits, DSA3D_K_PROJ_BWD_DW, s);
    if (e != hipSuccess) return e;
    const int64_t nw = F * C;
    {
        LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
        hipLaunchKernelGGL(dsa3d_split_sum_kernel, dim3((unsigned)std::min<int64_t>((nw + 255) / 256, 65536)), dim3(256), 0,
                           s, part, dw, nw, splits);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (db) {
        float* bpart = part + (size_t)sw * F * C;
        const int64_t rps = (ntok + sb - 1) / sb;
        const int bsplits = (int)((ntok + rps - 1) / rps);
        dim3 grid((unsigned)((F + 255) / 256), (unsigned)bsplits);
        {
        LaunchScope ls(DSA3D_K_COLSUM, s);
        if (f32)
            hipLaunchKernelGGL((dsa3d_colsum_kernel<float>), grid, dim3(256), 0, s, (const float*)doff, bpart, ntok, F, rps);
        else
            hipLaunchKernelGGL((dsa3d_colsum_kernel<bf16_t>), grid, dim3(256), 0, s, (const bf16_t*)doff, bpart, ntok, F,
                               rps);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
        hipLaunchKernelGGL(dsa3d_split_sum_kernel, dim3((unsigned)((F + 255) / 256)), dim3(256), 0, s, bpart, db, F,
                           bsplits);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsa3d
