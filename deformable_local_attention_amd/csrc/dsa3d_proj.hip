// dsa3d_proj.hip -- offset projection GEMMs on the matrix cores (gfx950).
//
// Forward:  offsets[N_tok, F] = q[N_tok, C] . W[F, C]^T + b      (both operands K-contiguous)
// Backward: dq[N_tok, C]     += doff[N_tok, F] . W[F, C]          (B is N-contiguous)
//           dW[F, C]          = doff^T . q                        (split over N_tok, fixed-order sum)
//           db[F]             = column sums of doff               (split over N_tok, fixed-order sum)
//
// Four kernels, by operand layout and dtype:
//  - dsa3d_ntgemm_kernel (bf16, both operands K-contiguous: the forward, and dq
//    once W is transposed into the workspace): 256x256 tiles, eight waves,
//    operands copied from memory straight into two 64-deep LDS stages;
//  - dsa3d_mngemm_kernel (bf16, both operands M/N-contiguous: dW): the same
//    tiles, waves and stages, the tiles copied as they lie and the MFMA
//    operands built by the transposing LDS read;
//  - dsa3d_xgemm_kernel (bf16 layouts and alignments the two above do not
//    take): 256x256 tiles, two register-staged LDS stages, M/N-contiguous
//    operands transposed in registers;
//  - dsa3d_gemm_kernel (float32 runs, and bf16 shapes the others cannot
//    take): 128x128 tiles, four waves of 64x64, 32-deep K slices in padded LDS
//    rows, v_mfma_f32_16x16x32_bf16 or v_mfma_f32_16x16x4_f32.
// All accumulate in float32; dW and db are split over the tokens and summed in
// a fixed order.
#include "dsa3d_device.h"
#include "dsa3d_internal.h"

namespace dsa3d {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int BM = 128, BN = 128, BK = 32;

// OUT_BIAS: C = A.B + bias; OUT_ACCUM: C = A.B + bias + R (one rounding; R may be C itself);
// OUT_PARTIAL: float32 partial products of one K split.
enum GemmOut { OUT_BIAS = 0, OUT_ACCUM = 1, OUT_PARTIAL = 2 };

struct GemmArgs {
    const void* A;  // a(m,k) = A[m*lda + k] if A is K-contiguous else A[k*lda + m]
    const void* B;  // b(k,n) = B[n*ldb + k] if B is K-contiguous else B[k*ldb + n]
    int64_t lda, ldb;
    int64_t M, N, K;
    int64_t k_split;   // K range of one blockIdx.z slice (multiple of BK)
    void* C;           // output: dtype tensor (OUT_BIAS, OUT_ACCUM) or float32 partials
    int64_t ldc;
    const void* bias;  // [N] or null (OUT_BIAS, OUT_ACCUM)
    const void* R;     // OUT_ACCUM: C = A.B + bias + R, R with C's layout (R == C: accumulate in place)
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
                    const float bb = g.bias ? load_scalar<T>(reinterpret_cast<const T*>(g.bias) + n) : 0.0f;
                    const float r = load_scalar<T>(reinterpret_cast<const T*>(g.R) + m * g.ldc + n);
                    store_scalar<T>(reinterpret_cast<T*>(g.C) + m * g.ldc + n, r + (x + bb));
                } else {
                    reinterpret_cast<float*>(g.C)[(int64_t)blockIdx.z * g.M * g.ldc + m * g.ldc + n] = x;
                }
            }
}

// ---------------------------------------------------------------------------
// bf16 path: 256x256 outputs per 256-thread workgroup, each of the four waves
// a 128x128 quarter computed as 4x4 v_mfma_f32_32x32x16_bf16 tiles whose
// float32 accumulators stay in registers for the whole K loop. K advances in
// 64-deep slices through two LDS stages (2 x 64 KiB): while the waves multiply
// one stage, the next slice is already in flight from memory into registers
// and is written to the other stage afterwards, so one barrier per slice
// suffices and the barrier waits for LDS traffic only.
//
// LDS holds every operand tile as 256 rows x 128 B (64 bf16 of K), the 16-byte
// chunk c of row r at chunk c ^ ((r >> 1) & 7): eight (and sixteen)
// consecutive rows read at the same logical chunk then fall on distinct banks.
// A K-contiguous operand is copied chunk for chunk; an M/N-contiguous one is
// loaded as 8x8 blocks (8 rows of K, 8 elements along M/N) and transposed in
// registers with byte permutes before it is written.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int XM = 256, XN = 256, XK = 64;
constexpr int X_ROW_BYTES = XK * 2;                 // one LDS row: 64 bf16 of K
constexpr int X_TILE_BYTES = XM * X_ROW_BYTES;      // 32 KiB per operand and stage
constexpr int X_LDS_BYTES = 4 * X_TILE_BYTES;       // A and B, two stages

__device__ __forceinline__ uint32_t xswz(uint32_t r) { return (r >> 1) & 7u; }

struct XSlice { uint4 v[8]; };

// Rows [r0, r0+256) x k [k0, k0+64) of one operand, as one thread loads them:
// a wave-uniform base pointer plus 32-bit element offsets that stay fixed
// from slice to slice (only the base moves with k0).
//
// K-contiguous (element (r, k) at src[r*ld + k]): thread t takes chunk t%8 of
// rows t/8 + 32j. Rows past the end are clamped (their products are never
// stored); k past kend reads zero.
template <bool KC> struct XOperand;
template <> struct XOperand<true> {
    const bf16_t* base;  // src + r0*ld
    int64_t ld;
    uint32_t off[8];
    __device__ __forceinline__ void init(const bf16_t* src, int64_t ld_, int64_t rows, int64_t r0) {
        const int tid = threadIdx.x;
        ld = ld_;
        base = src + r0 * ld_;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t r = std::min<int64_t>(r0 + (tid >> 3) + 32 * j, rows - 1) - r0;
            off[j] = (uint32_t)(r * ld_ + (tid & 7) * 8);
        }
    }
    template <bool FULL>
    __device__ __forceinline__ void load(int64_t k0, int64_t kend, XSlice& s) const {
        const bf16_t* p = base + k0;
        if (FULL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) s.v[j] = *reinterpret_cast<const uint4*>(p + off[j]);
        } else {
            // read the last in-bounds chunk instead, then zero it
            const int64_t gk = k0 + (threadIdx.x & 7) * 8;
            const bool ok = gk < kend;
            const uint32_t back = ok ? 0u : (uint32_t)(gk - (kend - 8));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint4 v = *reinterpret_cast<const uint4*>(p + (off[j] - back));
                s.v[j] = make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
            }
        }
    }
};

// M/N-contiguous (element (r, k) at src[k*ld + r]; rows is a multiple of 8
// here, so an 8-row group is wholly in or out): thread t takes the 8x8 block
// of k-group t%8 and row group t/8, groups past the end clamped to the last.
template <> struct XOperand<false> {
    const bf16_t* base;  // src + r0
    int64_t ld;
    uint32_t off;
    __device__ __forceinline__ void init(const bf16_t* src, int64_t ld_, int64_t rows, int64_t r0) {
        const int tid = threadIdx.x;
        ld = ld_;
        base = src + r0;
        const int64_t gr = std::min<int64_t>(r0 + (tid >> 3) * 8, rows - 8);
        off = (uint32_t)((tid & 7) * 8 * ld_ + (gr - r0));
    }
    template <bool FULL>
    __device__ __forceinline__ void load(int64_t k0, int64_t kend, XSlice& s) const {
        const bf16_t* p = base + k0 * ld;
        if (FULL) {
#pragma unroll
            for (int i = 0; i < 8; ++i) s.v[i] = *reinterpret_cast<const uint4*>(p + i * ld + off);
        } else {
            const int64_t gk = k0 + (threadIdx.x & 7) * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = gk + i < kend;
                const int64_t back = ok ? 0 : (gk + i - (kend - 1)) * ld;
                const uint4 v = *reinterpret_cast<const uint4*>(p + i * ld + off - back);
                s.v[i] = make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
            }
        }
    }
};

template <bool KC>
__device__ __forceinline__ void x_load(const XOperand<KC>& op, int64_t k0, int64_t kend, XSlice& s) {
    if (k0 + XK <= kend) op.template load<true>(k0, kend, s);
    else op.template load<false>(k0, kend, s);
}

__device__ __forceinline__ void x_store_kc(const XSlice& s, char* lds) {
    const int tid = threadIdx.x;
    const uint32_t c = (uint32_t)(tid & 7) ^ xswz((uint32_t)(tid >> 3));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t r = (uint32_t)(tid >> 3) + 32u * j;
        *reinterpret_cast<uint4*>(lds + r * X_ROW_BYTES + c * 16u) = s.v[j];
    }
}

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Transposes the 8x8 block in registers (byte permutes) and writes its 8 rows.
__device__ __forceinline__ void x_store_mn(const XSlice& s, char* lds) {
    const int tid = threadIdx.x;
    const uint32_t kg = (uint32_t)(tid & 7);
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
        // row rg*8+mm holds, at k = kg*8 + i, element mm of s.v[i]
        const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            w[jj] = __builtin_amdgcn_perm(u4_word(s.v[2 * jj + 1], mm >> 1), u4_word(s.v[2 * jj], mm >> 1), sel);
        const uint32_t r = (uint32_t)(tid >> 3) * 8u + mm;
        *reinterpret_cast<uint4*>(lds + r * X_ROW_BYTES + ((kg ^ xswz(r)) * 16u)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <bool KC>
__device__ __forceinline__ void x_store(const XSlice& s, char* lds) {
    if constexpr (KC) x_store_kc(s, lds);
    else x_store_mn(s, lds);
}

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for the
// global loads of the next slice that are still in flight.
__device__ __forceinline__ void x_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Operand fragments of one k16 step (of 4x4 MFMAs on a wave's 128x128
// quarter): lane l holds row l%32 of each 32-row tile and 8 consecutive k
// (chunk 2s + l/32 of the slice in step s); both operands use the same k
// assignment, so the hardware's k order inside one MFMA does not matter.
struct XFrag { bf16x8_t a[4], b[4]; };

// Accumulator element e of tile (i, j) is row 8*(e/4) + 4*(lane/32) + e%4,
// column lane%32 of that 32x32 tile. EDGE: the tile crosses the end of M or N.
template <int MODE, bool EDGE, int NJ>
__device__ __forceinline__ void x_epilogue_t(const GemmArgs& g, f32x16_t (*acc)[NJ], int64_t m0, int64_t n0,
                                             int wm, int wn, int lane) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int64_t n = n0 + wn * 32 * NJ + j * 32 + (lane & 31);
        if (EDGE && n >= g.N) continue;
        const float bb = (MODE != OUT_PARTIAL && g.bias)
                             ? load_scalar<bf16_t>(reinterpret_cast<const bf16_t*>(g.bias) + n)
                             : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (EDGE && m >= g.M) continue;
                const float x = acc[i][j][e];
                if (MODE == OUT_BIAS) {
                    store_scalar<bf16_t>(reinterpret_cast<bf16_t*>(g.C) + m * g.ldc + n, x + bb);
                } else if (MODE == OUT_ACCUM) {
                    const float r = load_scalar<bf16_t>(reinterpret_cast<const bf16_t*>(g.R) + m * g.ldc + n);
                    store_scalar<bf16_t>(reinterpret_cast<bf16_t*>(g.C) + m * g.ldc + n, r + (x + bb));
                } else {
                    reinterpret_cast<float*>(g.C)[(int64_t)blockIdx.z * g.M * g.ldc + m * g.ldc + n] = x;
                }
            }
    }
}

template <bool AK, bool BKC, int MODE>
__global__ void __launch_bounds__(256, 1) dsa3d_xgemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char lds[X_LDS_BYTES];
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const int wm = wv / 2, wn = wv % 2;
    const uint32_t ntn = (uint32_t)((g.N + XN - 1) / XN);
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t m0 = (int64_t)(lb / ntn) * XM, n0 = (int64_t)(lb % ntn) * XN;
    const int64_t kb = (int64_t)blockIdx.z * g.k_split;
    const int64_t ke = std::min<int64_t>(g.K, kb + g.k_split);
    const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
    const bf16_t* B = reinterpret_cast<const bf16_t*>(g.B);
    // stage z: A at lds + 2z tiles, B at lds + (2z+1) tiles
#define XA(z) (lds + (z) * 2 * X_TILE_BYTES)
#define XB(z) (lds + ((z) * 2 + 1) * X_TILE_BYTES)

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const uint32_t r = (uint32_t)(lane & 31), kh = (uint32_t)(lane >> 5);
    const uint32_t a_off = ((uint32_t)wm * 128u + r) * X_ROW_BYTES;
    const uint32_t b_off = ((uint32_t)wn * 128u + r) * X_ROW_BYTES;
    const uint32_t sw = xswz(r);

    const int64_t nk = (ke - kb + XK - 1) / XK;
    XOperand<AK> opa;
    XOperand<BKC> opb;
    opa.init(A, g.lda, g.M, m0);
    opb.init(B, g.ldb, g.N, n0);
    XSlice sa, sb;
    if (nk > 0) {
        x_load<AK>(opa, kb, ke, sa);
        x_load<BKC>(opb, kb, ke, sb);
        x_store<AK>(sa, XA(0));
        x_store<BKC>(sb, XB(0));
        if (nk > 1) {
            x_load<AK>(opa, kb + XK, ke, sa);
            x_load<BKC>(opb, kb + XK, ke, sb);
        }
        x_barrier();
    }
    // Fragments are read one k16 step ahead of their products (and kept there:
    // left to itself the compiler sinks each read to its first use and waits
    // for it once every four MFMAs). After the first step's products the next
    // slice's registers go to the other stage (last read in the previous slice,
    // before the barrier) and the loads of the slice after it are issued, a
    // whole slice ahead of their use. The barrier sits in the middle of the
    // last step, whose remaining products cover the next slice's first reads.
    auto xread = [&](const char* As, const char* Bs, uint32_t s, XFrag& f) {
        const uint32_t c = ((2u * s + kh) ^ sw) * 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + a_off + i * 32 * X_ROW_BYTES + c);
            f.b[i] = *reinterpret_cast<const bf16x8_t*>(Bs + b_off + i * 32 * X_ROW_BYTES + c);
        }
    };
    auto xmma = [&](const XFrag& f, int q) {
        acc[q / 4][q % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[q / 4], f.b[q % 4], acc[q / 4][q % 4], 0, 0, 0);
    };
    XFrag f, fn;
    if (nk > 0) {
        xread(XA(0), XB(0), 0, f);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int64_t t = 0; t < nk; ++t) {
        const int cur = (int)(t & 1);
#pragma unroll
        for (uint32_t s = 0; s < 3; ++s) {
            xread(XA(cur), XB(cur), s + 1, fn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 16; ++q) xmma(f, q);
            __builtin_amdgcn_sched_barrier(0);
            if (s == 0) {
                if (t + 1 < nk) {
                    x_store<AK>(sa, XA(cur ^ 1));
                    x_store<BKC>(sb, XB(cur ^ 1));
                }
                if (t + 2 < nk) {
                    x_load<AK>(opa, kb + (t + 2) * XK, ke, sa);
                    x_load<BKC>(opb, kb + (t + 2) * XK, ke, sb);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            f = fn;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) xmma(f, q);
        __builtin_amdgcn_sched_barrier(0);
        x_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < nk) xread(XA(cur ^ 1), XB(cur ^ 1), 0, fn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 8; q < 16; ++q) xmma(f, q);
        __builtin_amdgcn_sched_barrier(0);
        f = fn;
    }
#undef XA
#undef XB

    if (m0 + XM <= g.M && n0 + XN <= g.N)
        x_epilogue_t<MODE, false, 4>(g, acc, m0, n0, wm, wn, lane);
    else
        x_epilogue_t<MODE, true, 4>(g, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// bf16 products whose operands are both K-contiguous (the projection forward,
// and dq with W transposed beforehand): the same 256x256 tile and 4 waves of
// 128x128, but the operand tiles travel from memory straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16*lane), so no
// register holds staged data. The products are formed transposed (D = B.A^T
// per 32x32 tile): a lane then holds 4 consecutive output columns of one row,
// which the epilogue writes to LDS as 8-byte pieces and streams out as whole
// 16-byte row chunks.
// ---------------------------------------------------------------------------
// M0 carries the LDS address of the copy; it is saved and restored around it
// (one wait state between setting M0 and the copy).
__device__ __forceinline__ void y_copy(const char* gbase, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(gbase)
        : "memory");
}

// Four copies into consecutive 1 KiB blocks of LDS with one M0 value: the
// instruction offset adds to both the global and the LDS address, so copy q
// takes offset q*1024 and a global base lowered by as much. (Writing M0 holds
// the wave until the texture unit has taken the copies issued before, so one
// M0 value serves four copies.)
__device__ __forceinline__ void y_copy4(const char* gbase, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                        uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "global_load_lds_dwordx4 %3, %7 offset:1024\n\t"
        "global_load_lds_dwordx4 %4, %8 offset:2048\n\t"
        "global_load_lds_dwordx4 %5, %9 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(gbase), "s"(gbase - 1024), "s"(gbase - 2048),
          "s"(gbase - 3072)
        : "memory");
}

template <int N>
__device__ __forceinline__ void y_wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void y_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc[i][j] element e: output row m = 32i + lane%32, columns n = 32j + 8*(e/4)
// + 4*(lane/32) + e%4 (four consecutive per e/4), of this wave's 128 x 32*NJ
// part of the tile. The part goes through LDS (rows of 64*NJ bytes at
// lds + wave * 128 * 64*NJ, 16-byte chunk c of row m at c ^ (m mod 4*NJ)) and
// out as whole 16-byte row chunks.
template <int MODE, int NJ>
__device__ __forceinline__ void y_epilogue(const GemmArgs& g, f32x16_t (*acc)[NJ], char* lds, int64_t m0, int64_t n0,
                                           int wm, int wn, int lane, int wave) {
    constexpr int ROWB = 64 * NJ, NCH = 4 * NJ;
    const int64_t mq = m0 + wm * 128, nq = n0 + wn * 32 * NJ;  // this wave's part
    char* tile = lds + wave * 128 * ROWB;
    const bf16_t* bias = reinterpret_cast<const bf16_t*>(g.bias);
    const bf16_t* R = reinterpret_cast<const bf16_t*>(g.R);
    bf16_t* C = reinterpret_cast<bf16_t*>(g.C);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int nl = 32 * j + 8 * e4 + 4 * (lane >> 5);  // first of 4 columns
            float add[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias) {
                const int64_t n = nq + nl;
                if (n + 4 <= g.N) {
                    const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
                    add[0] = bf16_lo(bw.x); add[1] = bf16_hi(bw.x); add[2] = bf16_lo(bw.y); add[3] = bf16_hi(bw.y);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ml = 32 * i + (lane & 31);
                float x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = acc[i][j][4 * e4 + u] + add[u];
                if (MODE == OUT_ACCUM) {
                    const int64_t m = mq + ml, n = nq + nl;
                    if (m < g.M && n + 4 <= g.N) {
                        const uint2 o = *reinterpret_cast<const uint2*>(R + m * g.ldc + n);
                        x[0] = bf16_lo(o.x) + x[0]; x[1] = bf16_hi(o.x) + x[1];
                        x[2] = bf16_lo(o.y) + x[2]; x[3] = bf16_hi(o.y) + x[3];
                    }
                }
                const uint2 w = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                const uint32_t chunk = ((uint32_t)nl >> 3) ^ ((uint32_t)ml & (NCH - 1u));
                *reinterpret_cast<uint2*>(tile + ml * ROWB + chunk * 16 + (nl & 4) * 2) = w;
            }
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // 128 rows x NCH chunks: lane takes chunk lane % NCH of rows (64/NCH)*it + lane/NCH
    const int cl = lane & (NCH - 1);
    const int64_t n = nq + cl * 8;
    if (n + 8 > g.N) return;
#pragma unroll 4
    for (int it = 0; it < 2 * NCH; ++it) {
        const int ml = (64 / NCH) * it + lane / NCH;
        const int64_t m = mq + ml;
        if (m >= g.M) break;
        const uint4 v = *reinterpret_cast<const uint4*>(tile + ml * ROWB + (((uint32_t)cl ^ ((uint32_t)ml & (NCH - 1u))) * 16));
        *reinterpret_cast<uint4*>(C + m * g.ldc + n) = v;
    }
}

// ---------------------------------------------------------------------------
// The tile is worked by eight waves, two per SIMD, each 128 rows x 64
// columns of it (wave w: rows 128*(w/4), columns 64*(w%4)); a wave held up
// issuing copies leaves its SIMD's matrix pipe to the other wave.
//
// The K loop takes 64-deep slices through two stages of 64 KiB (A then B, 256
// rows of 128 B). A lane's 16-byte copies come eight to a row, so each row's
// share of a slice is one 128-byte request, and the waves meet at a barrier
// once per 32 of their MFMAs (32x32x16). The copies of slice t+2 go into the
// stage slice t releases at the barrier in the middle of its last k16 step:
// A's right after that barrier, B's in the first step of slice t+1, so that
// they neither arrive in one burst nor too late to land before slice t+1
// ends. A wave's four copies of an operand share one M0 value (writing M0
// holds the wave until the texture unit has taken the copies before it).
//
// LDS rows are 128 B; chunk c of row r sits at c ^ ((r/2) mod 8), so the 16
// rows of a 16-lane group of a fragment read (two rows per 64-bank line) fall
// on all 64 banks once. Copy instruction q (0..3) of wave w fills rows
// 32w + 8q .. +7 of an operand, lane l taking row 32w + 8q + l/8 and stored
// chunk l%8.
// ---------------------------------------------------------------------------
constexpr int ZK = 64;
constexpr int Z_ROW = ZK * 2;              // 128 B
constexpr int Z_TILE = 256 * Z_ROW;        // 32 KiB per operand
constexpr int Z_STAGE = 2 * Z_TILE;        // A then B
constexpr int Z_LDS = 2 * Z_STAGE;         // 128 KiB

__device__ __forceinline__ uint32_t zswz(uint32_t r) { return (r >> 1) & 7u; }

struct ZOperand {
    const char* base;  // src + r0*ld, in bytes
    uint32_t off[4];   // byte offset of this lane's row in copy instruction q
    uint32_t kc[2];    // first k (elements) of this lane's chunk: even and odd q
    __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int64_t rows, int64_t r0, int wave,
                                         int lane) {
        base = reinterpret_cast<const char*>(src + r0 * ld);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t r = 32u * (uint32_t)wave + 8u * q + (uint32_t)(lane >> 3);
            const int64_t rr = std::min<int64_t>(r0 + r, rows - 1) - r0;
            off[q] = (uint32_t)(rr * ld * 2);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
            kc[p] = (((uint32_t)(lane & 7)) ^ zswz(8u * p + (uint32_t)(lane >> 3))) * 8u;
    }
    __device__ __forceinline__ uint32_t voff(int q, int64_t k0, int64_t kend) const {
        const uint32_t c = kc[q & 1];
        const int64_t gk = k0 + c;
        const uint32_t back = (k0 + ZK <= kend || gk < kend) ? 0u : (uint32_t)((gk - (kend - 8)) * 2);
        return off[q] + c * 2 - back;
    }
    // this wave's four copies of slice [k0, k0 + 64) into the operand's tile at tile_addr (LDS)
    __device__ __forceinline__ void copy4(int64_t k0, int64_t kend, uint32_t tile_addr, int wave) const {
        y_copy4(base + k0 * 2, voff(0, k0, kend), voff(1, k0, kend), voff(2, k0, kend), voff(3, k0, kend),
                tile_addr + 4u * (uint32_t)wave * 1024u);
    }
};

__device__ __forceinline__ void z_zero_tail(char* stage, const ZOperand& a, int64_t k0, int64_t kend, int wave,
                                             int lane) {
    if (k0 + ZK <= kend) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (k0 + a.kc[q & 1] < kend) continue;
        const int o = (4 * wave + q) * 1024 + lane * 16;
        *reinterpret_cast<uint4*>(stage + o) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(stage + Z_TILE + o) = make_uint4(0u, 0u, 0u, 0u);
    }
}

struct YFrag { bf16x8_t a[4], b[2]; };

__device__ __forceinline__ void z_read_piece(const char* stage, uint32_t a_off, uint32_t b_off, uint32_t c, int i,
                                              YFrag& f) {
    if (i < 4) f.a[i] = *reinterpret_cast<const bf16x8_t*>(stage + a_off + i * 32 * Z_ROW + c);
    else f.b[i - 4] = *reinterpret_cast<const bf16x8_t*>(stage + Z_TILE + b_off + (i - 4) * 32 * Z_ROW + c);
}

// MFMA q (0..7) of a k16 step: acc[q/2][q%2] = B_(q%2) . A_(q/2)^T
__device__ __forceinline__ void y_mma(const YFrag& f, int q, f32x16_t acc[4][2]) {
    acc[q / 2][q % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[q % 2], f.a[q / 2], acc[q / 2][q % 2], 0, 0, 0);
}

template <int MODE>
__global__ void __launch_bounds__(512, 1) dsa3d_ntgemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char lds[Z_LDS];
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int wm = wave / 4, wn = wave % 4;
    const uint32_t ntn = (uint32_t)((g.N + XN - 1) / XN);
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t m0 = (int64_t)(lb / ntn) * XM, n0 = (int64_t)(lb % ntn) * XN;
    const int64_t K = g.K;
    ZOperand opa, opb;
    opa.init(reinterpret_cast<const bf16_t*>(g.A), g.lda, g.M, m0, wave, lane);
    opb.init(reinterpret_cast<const bf16_t*>(g.B), g.ldb, g.N, n0, wave, lane);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const uint32_t r = (uint32_t)(lane & 31), kh = (uint32_t)(lane >> 5);
    const uint32_t a_off = ((uint32_t)wm * 128u + r) * Z_ROW;
    const uint32_t b_off = ((uint32_t)wn * 64u + r) * Z_ROW;
    const uint32_t sw = zswz(r);
    // Slices 0 and 1 fill the two stages; iteration t multiplies slice t in
    // four k16 steps, the next step's fragments read (and kept ahead of the
    // products) during the current one's MFMAs. In the last step each wave
    // waits for its copies of slice t+1 and meets the others at the barrier,
    // after which slice t's stage takes A's copies of slice t+2 and the first
    // fragments of slice t+1 are read, between that step's remaining MFMAs;
    // B's copies of slice t+2 follow in slice t+1's first step.
    const int64_t nk = (K + ZK - 1) / ZK;
    YFrag f, fn;
    if (nk > 0) {
        opa.copy4(0, K, lds0, wave);
        opb.copy4(0, K, lds0 + Z_TILE, wave);
        if (nk > 1) {
            opa.copy4(ZK, K, lds0 + Z_STAGE, wave);
            opb.copy4(ZK, K, lds0 + Z_STAGE + Z_TILE, wave);
            y_wait_vm<8>();  // slice 0 has landed (slice 1's 8 copies may still be in flight)
        } else {
            y_wait_vm<0>();
        }
        z_zero_tail(lds, opa, 0, K, wave, lane);
        y_barrier();
        const uint32_t c0 = ((0u + kh) ^ sw) * 16u;
#pragma unroll
        for (int i = 0; i < 6; ++i) z_read_piece(lds, a_off, b_off, c0, i, f);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int64_t t = 0; t < nk; ++t) {
        const char* stage = lds + (t & 1) * Z_STAGE;
        const bool spread = t >= 1 && t + 1 < nk;
        const int64_t k1 = (t + 1) * ZK;
        const uint32_t st1 = lds0 + (uint32_t)(((t + 1) & 1) * Z_STAGE);
#pragma unroll
        for (uint32_t s = 0; s < 3; ++s) {
            const uint32_t c = ((2u * (s + 1) + kh) ^ sw) * 16u;
#pragma unroll
            for (int i = 0; i < 6; ++i) z_read_piece(stage, a_off, b_off, c, i, fn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                y_mma(f, q, acc);
                // B's copies of slice t+1: waves 0-3 in the first step, waves 4-7 (the
                // other wave of each SIMD) a step later, so that the two waves of a SIMD
                // do not both wait on the texture unit to take their copies
                if (s == (wave < 4 ? 0u : 1u) && q == 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (spread) opb.copy4(k1, K, st1 + Z_TILE, wave);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f = fn;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) y_mma(f, q, acc);
        __builtin_amdgcn_sched_barrier(0);
        const bool more = t + 1 < nk;
        if (more) {
            y_wait_vm<0>();  // this wave's copies of slice t+1
            z_zero_tail(lds + ((t + 1) & 1) * Z_STAGE, opa, (t + 1) * ZK, K, wave, lane);
        }
        y_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
            const bool refill = t + 2 < nk;
            const int64_t k2 = (t + 2) * ZK;
            const uint32_t st = lds0 + (uint32_t)((t & 1) * Z_STAGE);
            const char* next = lds + ((t + 1) & 1) * Z_STAGE;
            const uint32_t c0 = ((0u + kh) ^ sw) * 16u;
#pragma unroll
            for (int q = 4; q < 8; ++q) {
                y_mma(f, q, acc);
                __builtin_amdgcn_sched_barrier(0);
                // A's copies of slice t+2: waves 4-7 two products after waves 0-3
                if (refill && q == (wave < 4 ? 4 : 6)) opa.copy4(k2, K, st, wave);
                if (more) {
                    if (q < 6) {
                        z_read_piece(next, a_off, b_off, c0, 2 * (q - 4), fn);
                        z_read_piece(next, a_off, b_off, c0, 2 * (q - 4) + 1, fn);
                    } else {
                        z_read_piece(next, a_off, b_off, c0, q - 2, fn);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            f = fn;
        }
    }
    y_barrier();  // every wave is done with the stages before they hold the output tile
    y_epilogue<MODE, 2>(g, acc, lds, m0, n0, wm, wn, lane, wave);
}

// ---------------------------------------------------------------------------
// bf16 products whose operands are both M/N-contiguous (dW = dy^T . x, the
// offset projection's dW): the same 256x256 tile, eight waves and two 64-deep
// LDS stages as the DMA-fed kernel, the tiles copied from memory as they lie
// (an LDS row is one k: 256 columns, 512 B) and the MFMA operands read with
// gfx950's transposing LDS read, ds_read_b64_tr_b16. In a 16-lane block of
// that read, lane j receives element j%4 of the 8-byte pieces read by lanes
// j/4, j/4 + 4, j/4 + 8 and j/4 + 12; so when lane L reads row k0 + L/4,
// columns c0 + 4(L%4) .. +3, lane j receives column c0 + j of rows k0 .. k0+3,
// and two such reads give a lane its 8 consecutive k of one column.
//
// The 32-byte unit u of LDS row r sits at u ^ (2 (r mod 4)): the 32 lanes a
// transposing read serves at once (4 rows, two 32-byte units each) then fall
// on distinct banks. Copy instruction q (0..3) of wave w fills rows
// 2(4w + q) and 2(4w + q) + 1, lane l taking row 2(4w + q) + l/32 and stored
// 16-byte slot l%32.
// ---------------------------------------------------------------------------
constexpr int T_ROWB = 512;              // one LDS row: 256 bf16 columns of one k
constexpr int T_TILE = 64 * T_ROWB;      // 32 KiB: the 64 k rows of one operand
constexpr int T_STAGE = 2 * T_TILE;      // A then B
constexpr int T_LDS = 2 * T_STAGE;       // 128 KiB

typedef __attribute__((ext_vector_type(4))) short s16x4_t;

struct TOperand {
    const char* base;   // src + c0 (this tile's first column), in bytes
    uint32_t ldb;       // bytes per k row
    uint32_t colb[2];   // byte offset of this lane's 16 bytes within its row: even and odd q
    // row of copy instruction q within the slice: 2(4w + q) + l/32 (its swizzle term depends on q's parity only)
    static __device__ __forceinline__ uint32_t row(int q, int wave, int lane) {
        return 2u * (4u * (uint32_t)wave + (uint32_t)q) + (uint32_t)(lane >> 5);
    }
    __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int64_t cols, int64_t c0, int wave,
                                         int lane) {
        base = reinterpret_cast<const char*>(src + c0);
        ldb = (uint32_t)(ld * 2);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t r = row(q, wave, lane);
            const uint32_t p = (uint32_t)(lane & 31);
            const uint32_t w = 2u * ((p >> 1) ^ (2u * (r & 3u))) + (p & 1u);  // the row's chunk stored at slot p
            // columns past the end read the last in-bounds chunk (never stored)
            const int64_t col = std::min<int64_t>(8 * (int64_t)w, cols - c0 - 8);
            colb[q] = (uint32_t)(col * 2);
        }
    }
    // byte offset of copy q of slice [k0, k0 + 64) from base + k0 * ldb: rows at or past kend read the last
    // in-bounds row instead (t_zero_tail clears them once they have landed)
    __device__ __forceinline__ uint32_t voff(int q, uint32_t last, int wave, int lane) const {
        return min(row(q, wave, lane), last) * ldb + colb[q & 1];
    }
    __device__ __forceinline__ void copy4(int64_t k0, int64_t kend, uint32_t tile_addr, int wave, int lane) const {
        const uint32_t last = (uint32_t)std::min<int64_t>(63, kend - 1 - k0);  // last in-bounds row of the slice
        y_copy4(base + k0 * (int64_t)ldb, voff(0, last, wave, lane), voff(1, last, wave, lane),
                voff(2, last, wave, lane), voff(3, last, wave, lane), tile_addr + 4u * (uint32_t)wave * 1024u);
    }
};

__device__ __forceinline__ void t_zero_tail(char* stage, int64_t k0, int64_t kend, int wave, int lane) {
    if (k0 + 64 <= kend) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (k0 + (int64_t)TOperand::row(q, wave, lane) < kend) continue;
        const int o = (4 * wave + q) * 1024 + lane * 16;
        *reinterpret_cast<uint4*>(stage + o) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(stage + T_TILE + o) = make_uint4(0u, 0u, 0u, 0u);
    }
}

struct TFrag { bf16x8_t a[4], b[2]; };

// The fragments of k16 step s: A tiles i (columns 32i + l%32 of the wave's
// 128) and B tiles j (columns 32j + l%32 of its 64), k rows 16s + 8(l/32) .. +7.
__device__ __forceinline__ bf16x8_t t_read8(const char* p) {
    typedef s16x4_t __attribute__((address_space(3))) * lds_s16x4_ptr;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p + 4 * T_ROWB));
    typedef __attribute__((ext_vector_type(8))) short s16x8_t;
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// A lane's transposing-read offsets: rows 8(l/32) + L/4 for L = l%16, the
// swizzled 32-byte unit of its block's 16 columns, its 8 bytes within it.
struct TReadOff {
    uint32_t row_b;  // row and in-unit bytes: (8(l/32) + L/4) * 512 + 8(L%4)
    uint32_t ua;     // A's unit before the swizzle, tile 0: 8 wm + block
    uint32_t ub;     // B's, tile 0: 4 wn + block
    uint32_t x;      // the swizzle term: 2 (L/4)
    __device__ __forceinline__ uint32_t a(int i) const { return row_b + ((ua + 2u * i) ^ x) * 32u; }
    __device__ __forceinline__ uint32_t b(int j) const { return row_b + ((ub + 2u * j) ^ x) * 32u; }
};

__device__ __forceinline__ void t_read_piece(const char* stage, const TReadOff& o, uint32_t s, int i, TFrag& f) {
    const uint32_t ro = 16u * s * T_ROWB;
    if (i < 4) f.a[i] = t_read8(stage + ro + o.a(i));
    else f.b[i - 4] = t_read8(stage + T_TILE + ro + o.b(i - 4));
}

// acc[i][j] = A_i . B_j (element e: row 8*(e/4) + 4*(lane/32) + e%4, column lane%32 of the 32x32 tile)
__device__ __forceinline__ void t_mma(const TFrag& f, int q, f32x16_t acc[4][2]) {
    acc[q / 2][q % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[q / 2], f.b[q % 2], acc[q / 2][q % 2], 0, 0, 0);
}

template <int MODE>
__global__ void __launch_bounds__(512, 1) dsa3d_mngemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char lds[T_LDS];
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int wm = wave / 4, wn = wave % 4;  // 128 rows x 64 columns of the tile
    const uint32_t ntn = (uint32_t)((g.N + XN - 1) / XN);
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t m0 = (int64_t)(lb / ntn) * XM, n0 = (int64_t)(lb % ntn) * XN;
    const int64_t kb = (int64_t)blockIdx.z * g.k_split;
    const int64_t ke = std::min<int64_t>(g.K, kb + g.k_split);
    TOperand opa, opb;
    opa.init(reinterpret_cast<const bf16_t*>(g.A), g.lda, g.M, m0, wave, lane);
    opb.init(reinterpret_cast<const bf16_t*>(g.B), g.ldb, g.N, n0, wave, lane);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    TReadOff ro;
    {
        const uint32_t L = (uint32_t)(lane & 15), blk = (uint32_t)((lane >> 4) & 1), kh = (uint32_t)(lane >> 5);
        ro.row_b = (8u * kh + (L >> 2)) * T_ROWB + 8u * (L & 3u);
        ro.ua = 8u * (uint32_t)wm + blk;
        ro.ub = 4u * (uint32_t)wn + blk;
        ro.x = 2u * (L >> 2);
    }

    // as in the DMA-fed kernel: two stages; after the barrier in the middle of
    // slice t's last step its stage takes A's copies of slice t+2, and B's
    // follow in slice t+1's first step
    const int64_t nk = (ke - kb + 63) / 64;
    TFrag f, fn;
    if (nk > 0) {
        opa.copy4(kb, ke, lds0, wave, lane);
        opb.copy4(kb, ke, lds0 + T_TILE, wave, lane);
        if (nk > 1) {
            opa.copy4(kb + 64, ke, lds0 + T_STAGE, wave, lane);
            opb.copy4(kb + 64, ke, lds0 + T_STAGE + T_TILE, wave, lane);
            y_wait_vm<8>();  // slice 0 has landed (slice 1's 8 copies may still be in flight)
        } else {
            y_wait_vm<0>();
        }
        t_zero_tail(lds, kb, ke, wave, lane);
        y_barrier();
#pragma unroll
        for (int i = 0; i < 6; ++i) t_read_piece(lds, ro, 0, i, f);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int64_t t = 0; t < nk; ++t) {
        const char* stage = lds + (t & 1) * T_STAGE;
        const bool spread = t >= 1 && t + 1 < nk;
        const int64_t k1 = kb + (t + 1) * 64;
        const uint32_t st1 = lds0 + (uint32_t)(((t + 1) & 1) * T_STAGE);
#pragma unroll
        for (uint32_t s = 0; s < 3; ++s) {
#pragma unroll
            for (int i = 0; i < 6; ++i) t_read_piece(stage, ro, s + 1, i, fn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                t_mma(f, q, acc);
                if (s == 0 && q == 1) {  // B's copies of slice t+1
                    __builtin_amdgcn_sched_barrier(0);
                    if (spread) opb.copy4(k1, ke, st1 + T_TILE, wave, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f = fn;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) t_mma(f, q, acc);
        __builtin_amdgcn_sched_barrier(0);
        const bool more = t + 1 < nk;
        if (more) {
            y_wait_vm<0>();  // this wave's copies of slice t+1
            t_zero_tail(lds + ((t + 1) & 1) * T_STAGE, k1, ke, wave, lane);
        }
        y_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
            const bool refill = t + 2 < nk;
            const int64_t k2 = kb + (t + 2) * 64;
            const uint32_t st = lds0 + (uint32_t)((t & 1) * T_STAGE);
            const char* next = lds + ((t + 1) & 1) * T_STAGE;
#pragma unroll
            for (int q = 4; q < 8; ++q) {
                t_mma(f, q, acc);
                __builtin_amdgcn_sched_barrier(0);
                if (refill && q == 4) opa.copy4(k2, ke, st, wave, lane);  // A's copies of slice t+2
                if (more) {
                    if (q < 6) {
                        t_read_piece(next, ro, 0, 2 * (q - 4), fn);
                        t_read_piece(next, ro, 0, 2 * (q - 4) + 1, fn);
                    } else {
                        t_read_piece(next, ro, 0, q - 2, fn);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            f = fn;
        }
    }
    if (m0 + XM <= g.M && n0 + XN <= g.N)
        x_epilogue_t<MODE, false, 2>(g, acc, m0, n0, wm, wn, lane);
    else
        x_epilogue_t<MODE, true, 2>(g, acc, m0, n0, wm, wn, lane);
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

// bf16 with F % 8 == 0: a thread owns 8 consecutive columns (16-byte loads)
// and keeps four running sums per column, over rows r = 0, 1, 2, 3 (mod 4) of
// its split, joined as (s0 + s1) + (s2 + s3): a fixed order, four loads in flight.
__global__ void __launch_bounds__(256) dsa3d_colsum8_kernel(const bf16_t* g, float* part, int64_t rows, int64_t F,
                                                            int64_t rows_per_split) {
    const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c >= F) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rows_per_split);
    float acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
    int64_t r = r0;
    for (; r + 4 <= r1; r += 4) {
        Frag8<bf16_t> v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u].load(g + (r + u) * F + c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float x[8];
            v[u].to_f32(x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u][e] += x[e];
        }
    }
    for (; r < r1; ++r) {
        Frag8<bf16_t> v;
        v.load(g + r * F + c);
        float x[8];
        v.to_f32(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[0][e] += x[e];
    }
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (acc[0][e] + acc[1][e]) + (acc[2][e] + acc[3][e]);
    Frag8<float> o;
    o.from_f32(out);
    o.store(part + (int64_t)blockIdx.y * F + c);
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

// The bf16 256x256 path needs 16-byte vectors everywhere: leading dimensions
// and the contiguous extent of each operand (K for a K-contiguous one, M or N
// for the other) multiples of 8, and 16-byte aligned bases.
static bool xgemm_ok(const GemmArgs& g, bool ak, bool bk) {
    const bool a = (g.lda % 8 == 0) && aligned16(g.A) && ((ak ? g.K : g.M) % 8 == 0);
    const bool b = (g.ldb % 8 == 0) && aligned16(g.B) && ((bk ? g.K : g.N) % 8 == 0);
    return a && b && (g.k_split % XK == 0 || g.k_split >= g.K);
}

template <bool AK, bool BKC, int MODE>
static hipError_t xgemm(GemmArgs g, int splits, int kernel_id, hipStream_t s) {
    const int64_t tiles = ((g.M + XM - 1) / XM) * ((g.N + XN - 1) / XN);
    if (tiles == 0) return hipSuccess;
    LaunchScope ls(kernel_id, s);
    hipLaunchKernelGGL((dsa3d_xgemm_kernel<AK, BKC, MODE>), dim3((unsigned)tiles, 1, splits), dim3(256), 0, s, g);
    return hipGetLastError();
}

// out[c*F + f] = w[f*C + c]: 64x64 tiles through LDS (odd row stride, no bank conflicts).
__global__ void __launch_bounds__(256) dsa3d_transpose_kernel(const bf16_t* w, bf16_t* out, int64_t F, int64_t C) {
    __shared__ bf16_t t[64][65];
    const int64_t f0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i / 64, c = i % 64;
        if (f0 + r < F && c0 + c < C) t[r][c] = w[(f0 + r) * C + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i / 64, c = i % 64;
        if (c0 + r < C && f0 + c < F) out[(c0 + r) * F + f0 + c] = t[c][r];
    }
}

// The DMA-fed kernel needs both operands K-contiguous and everything in
// 16-byte pieces: K, the leading dimensions and N multiples of 8, 16-byte
// aligned bases (bias included), one K range.
static bool ntgemm_ok(const GemmArgs& g) {
    return g.lda % 8 == 0 && g.ldb % 8 == 0 && g.ldc % 8 == 0 && g.K % 8 == 0 && g.N % 8 == 0 && aligned16(g.A) &&
           aligned16(g.B) && aligned16(g.C) && (g.bias == nullptr || aligned16(g.bias)) && g.k_split >= g.K;
}

template <int MODE>
static hipError_t ntgemm(GemmArgs g, int kernel_id, hipStream_t s) {
    const int64_t tiles = ((g.M + XM - 1) / XM) * ((g.N + XN - 1) / XN);
    if (tiles == 0) return hipSuccess;
    LaunchScope ls(kernel_id, s);
    hipLaunchKernelGGL((dsa3d_ntgemm_kernel<MODE>), dim3((unsigned)tiles), dim3(512), 0, s, g);
    return hipGetLastError();
}

// The transposing-read kernel needs both operands M/N-contiguous in 16-byte
// pieces: M, N and the leading dimensions multiples of 8, 16-byte aligned
// bases, K splits that are whole 64-deep slices.
static bool mngemm_ok(const GemmArgs& g) {
    return g.M % 8 == 0 && g.N % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && aligned16(g.A) && aligned16(g.B) &&
           (g.k_split % 64 == 0 || g.k_split >= g.K);
}

template <int MODE>
static hipError_t mngemm(GemmArgs g, int splits, int kernel_id, hipStream_t s) {
    const int64_t tiles = ((g.M + XM - 1) / XM) * ((g.N + XN - 1) / XN);
    if (tiles == 0) return hipSuccess;
    LaunchScope ls(kernel_id, s);
    hipLaunchKernelGGL((dsa3d_mngemm_kernel<MODE>), dim3((unsigned)tiles, 1, splits), dim3(512), 0, s, g);
    return hipGetLastError();
}

// bf16 products go to the 256x256 kernel when its vector conditions hold,
// everything else (float32, odd sizes) to the 128x128 one.
template <typename T, bool AK, bool BKC, int MODE>
static hipError_t gemm_any(GemmArgs g, int splits, int kernel_id, hipStream_t s) {
    if constexpr (sizeof(T) == 2) {
        if constexpr (!AK && !BKC) {
            if (mngemm_ok(g)) return mngemm<MODE>(g, splits, kernel_id, s);
        }
        if (xgemm_ok(g, AK, BKC)) return xgemm<AK, BKC, MODE>(g, splits, kernel_id, s);
    }
    return gemm<T, AK, BKC, MODE>(g, splits, kernel_id, s);
}

// Split counts of the two long reductions over the M rows of a linear layer's
// backward (dW over the rows, db over the rows).
void linear_bwd_splits(int dtype, int64_t M, int64_t N, int64_t K, int& dw_splits, int& db_splits) {
    const int64_t tm = dtype == DSA3D_BF16 ? XM : BM, tn = dtype == DSA3D_BF16 ? XN : BN;
    const int64_t tiles = ((N + tm - 1) / tm) * ((K + tn - 1) / tn);
    int64_t s = (1024 + tiles - 1) / std::max<int64_t>(tiles, 1);
    s = std::max<int64_t>(1, std::min<int64_t>(s, std::max<int64_t>(1, M / (4 * XK))));
    s = std::min<int64_t>(s, 64);
    dw_splits = (int)s;
    // column sums: up to 1024 splits of at least 256 rows
    db_splits = (int)std::max<int64_t>(1, std::min<int64_t>(1024, M / 256));
}

size_t linear_bwd_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K) {
    int sw, sb;
    linear_bwd_splits(dtype, M, N, K, sw, sb);
    size_t bytes = (size_t)sw * N * K * 4 + (size_t)sb * N * 4;
    if (dtype == DSA3D_BF16) bytes += 256 + (size_t)N * K * 2;  // w transposed, 256-aligned
    return bytes + 256;
}

void proj_bwd_splits(const dsa3d_desc& d, int& dw_splits, int& db_splits) {
    linear_bwd_splits(d.dtype, d.B * d.T * d.H * d.W, (int64_t)d.heads * d.P * 3, (int64_t)d.heads * d.head_dim,
                      dw_splits, db_splits);
}

size_t proj_bwd_workspace_bytes(const dsa3d_desc& d) {
    return linear_bwd_workspace_bytes(d.dtype, d.B * d.T * d.H * d.W, (int64_t)d.heads * d.P * 3,
                                      (int64_t)d.heads * d.head_dim);
}

hipError_t launch_linear_forward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                 const void* bias, const void* residual, void* y, int kernel_id, hipStream_t s) {
    GemmArgs g{};
    g.A = x; g.lda = K;
    g.B = w; g.ldb = K;
    g.M = M; g.N = N; g.K = K;
    g.k_split = round_up(g.K, BK);
    g.C = y; g.ldc = N;
    g.bias = bias;
    g.R = residual;
    const bool f32 = dtype == DSA3D_F32;
    if (residual == nullptr) {
        if (f32) return gemm<float, true, true, OUT_BIAS>(g, 1, kernel_id, s);
        if (ntgemm_ok(g)) return ntgemm<OUT_BIAS>(g, kernel_id, s);
        return gemm_any<bf16_t, true, true, OUT_BIAS>(g, 1, kernel_id, s);
    }
    if (f32) return gemm<float, true, true, OUT_ACCUM>(g, 1, kernel_id, s);
    if (ntgemm_ok(g) && aligned16(residual)) return ntgemm<OUT_ACCUM>(g, kernel_id, s);
    return gemm_any<bf16_t, true, true, OUT_ACCUM>(g, 1, kernel_id, s);
}

hipError_t launch_proj_forward(const dsa3d_desc& d, const void* q, const void* w, const void* bias, void* off,
                               hipStream_t s) {
    return launch_linear_forward(d.dtype, d.B * d.T * d.H * d.W, (int64_t)d.heads * d.P * 3,
                                 (int64_t)d.heads * d.head_dim, q, w, bias, nullptr, off, DSA3D_K_PROJ_FORWARD, s);
}

hipError_t launch_linear_backward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                  const void* dy, const void* dres, void* dx, float* dw, float* db, void* ws,
                                  const LinearKernelIds& ids, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const bool f32 = dtype == DSA3D_F32;
    hipError_t e;
    int sw, sb;
    linear_bwd_splits(dtype, M, N, K, sw, sb);
    // dx[M, K] = dres + dy[M, N] . w[N, K]
    GemmArgs g{};
    g.A = dy; g.lda = N;
    g.B = w; g.ldb = K;
    g.M = M; g.N = K; g.K = N;
    g.k_split = round_up(N, BK);
    g.C = dx; g.ldc = K;
    g.R = dres;
    // bf16: with w transposed into the workspace ([K, N], contiguous along N) the
    // product takes the DMA-fed kernel
    const uintptr_t wt_at = round_up((int64_t)(reinterpret_cast<uintptr_t>(ws) + (size_t)sw * N * K * 4 +
                                               (size_t)sb * N * 4), 256);
    GemmArgs gt = g;
    gt.B = reinterpret_cast<const void*>(wt_at);
    gt.ldb = N;
    if (!f32 && ntgemm_ok(gt)) {
        {
            LaunchScope ls(ids.transpose, s);
            hipLaunchKernelGGL(dsa3d_transpose_kernel, dim3((unsigned)((K + 63) / 64), (unsigned)((N + 63) / 64)),
                               dim3(256), 0, s, reinterpret_cast<const bf16_t*>(w), reinterpret_cast<bf16_t*>(wt_at),
                               N, K);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = dres ? ntgemm<OUT_ACCUM>(gt, ids.dx, s) : ntgemm<OUT_BIAS>(gt, ids.dx, s);
    } else if (dres) {
        e = f32 ? gemm<float, true, false, OUT_ACCUM>(g, 1, ids.dx, s)
                : gemm_any<bf16_t, true, false, OUT_ACCUM>(g, 1, ids.dx, s);
    } else {
        e = f32 ? gemm<float, true, false, OUT_BIAS>(g, 1, ids.dx, s)
                : gemm_any<bf16_t, true, false, OUT_BIAS>(g, 1, ids.dx, s);
    }
    if (e != hipSuccess) return e;
    // dw[N, K] = dy^T . x, split over the rows, then a fixed-order sum
    float* part = reinterpret_cast<float*>(ws);
    GemmArgs h{};
    h.A = dy; h.lda = N;   // a(m=n, k=row) = dy[row*N + n]: M-contiguous
    h.B = x; h.ldb = K;    // b(k=row, n=c) = x[row*K + c]: N-contiguous
    h.M = N; h.N = K; h.K = M;
    h.k_split = round_up((M + sw - 1) / sw, XK);  // a multiple of both kernels' K slice
    const int splits = (int)((M + h.k_split - 1) / h.k_split);
    h.C = part; h.ldc = K;
    e = f32 ? gemm<float, false, false, OUT_PARTIAL>(h, splits, ids.dw, s)
            : gemm_any<bf16_t, false, false, OUT_PARTIAL>(h, splits, ids.dw, s);
    if (e != hipSuccess) return e;
    const int64_t nw = N * K;
    {
        LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
        hipLaunchKernelGGL(dsa3d_split_sum_kernel, dim3((unsigned)std::min<int64_t>((nw + 255) / 256, 65536)),
                           dim3(256), 0, s, part, dw, nw, splits);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (db) {
        float* bpart = part + (size_t)sw * N * K;
        const int64_t rps = (M + sb - 1) / sb;
        const int bsplits = (int)((M + rps - 1) / rps);
        {
            LaunchScope ls(DSA3D_K_COLSUM, s);
            if (!f32 && N % 8 == 0 && aligned16(dy) && aligned16(bpart)) {
                dim3 grid((unsigned)((N / 8 + 255) / 256), (unsigned)bsplits);
                hipLaunchKernelGGL(dsa3d_colsum8_kernel, grid, dim3(256), 0, s, (const bf16_t*)dy, bpart, M, N, rps);
            } else {
                dim3 grid((unsigned)((N + 255) / 256), (unsigned)bsplits);
                if (f32)
                    hipLaunchKernelGGL((dsa3d_colsum_kernel<float>), grid, dim3(256), 0, s, (const float*)dy, bpart,
                                       M, N, rps);
                else
                    hipLaunchKernelGGL((dsa3d_colsum_kernel<bf16_t>), grid, dim3(256), 0, s, (const bf16_t*)dy,
                                       bpart, M, N, rps);
            }
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
        hipLaunchKernelGGL(dsa3d_split_sum_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, bpart, db, N,
                           bsplits);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_proj_backward(const dsa3d_desc& d, const void* q, const void* w, const void* doff, void* dq,
                                float* dw, float* db, void* ws, hipStream_t s) {
    const LinearKernelIds ids{DSA3D_K_TRANSPOSE, DSA3D_K_PROJ_BWD_DQ, DSA3D_K_PROJ_BWD_DW};
    return launch_linear_backward(d.dtype, d.B * d.T * d.H * d.W, (int64_t)d.heads * d.P * 3,
                                  (int64_t)d.heads * d.head_dim, q, w, doff, dq, dq, dw, db, ws, ids, s);
}

}  // namespace dsa3d
