// dsa3d_block.hip -- layer normalisation of the transformer block around the
// 3D-DSA operator (gfx950). The pages apply layer normalisation and residual
// connections around their attention as usual [MegaSlide-DiT, §5.3
// Implementation considerations]; the residual add lives in the output
// projection's epilogue (dsa3d_linear_forward with a residual), the
// normalisation here.
//
// Over the last axis of x [M, N] (M rows: tokens; N channels):
//   mean = sum(x) / N, var = sum((x - mean)^2) / N, rstd = 1 / sqrt(var + eps)
//   y = (x - mean) * rstd * gamma + beta                      (forward)
//   xh = (x - mean) * rstd, g = dy * gamma
//   dx = dres + rstd * (g - mean(g) - xh * mean(g * xh))     (backward)
//   dgamma = sum over rows of dy * xh, dbeta = sum over rows of dy
// in float32 with one rounding per stored element; dgamma/dbeta are summed in
// a fixed order (bitwise reproducible).
//
// Both kernels are bound by memory traffic: each row is read (and written)
// once, as 16-byte pieces of 8 channels per lane.
#include "dsa3d_device.h"
#include "dsa3d_internal.h"

namespace dsa3d {

namespace {

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

template <typename T>
__device__ __forceinline__ float load_param(const T* p, int64_t i) {
    return p ? load_scalar<T>(p + i) : 0.0f;
}

}  // namespace

// One wave per row, NC pieces of 512 channels (8 per lane) held in registers:
// the row is read once, the mean and the centred variance are two wave sums
// over those registers. Rows are dealt to the waves of the grid in turn.
template <typename T, int NC>
__global__ void __launch_bounds__(256) dsa3d_layernorm_kernel(const T* x, const T* gamma, const T* beta, T* y,
                                                              float* stats, int64_t M, int64_t N, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const float inv_n = 1.0f / (float)N;
    float gm[NC][8], bt[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t ch = (int64_t)c * 512 + lane * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool in = ch + e < N;
            gm[c][e] = in ? (gamma ? load_scalar<T>(gamma + ch + e) : 1.0f) : 0.0f;
            bt[c][e] = in ? load_param<T>(beta, ch + e) : 0.0f;
        }
    }
    for (int64_t row = wave; row < M; row += nwaves) {
        const T* xr = x + row * N;
        float v[NC][8];
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t ch = (int64_t)c * 512 + lane * 8;
            if (ch < N) {
                Frag8<T> f;
                f.load(xr + ch);
                f.to_f32(v[c]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[c][e];
        }
        const float mean = wave_sum(s) * inv_n;
        float q = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t ch = (int64_t)c * 512 + lane * 8;
            if (ch < N) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dv = v[c][e] - mean;
                    q = fmaf(dv, dv, q);
                }
            }
        }
        const float var = wave_sum(q) * inv_n;
        const float rstd = 1.0f / sqrtf(var + eps);
        T* yr = y + row * N;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t ch = (int64_t)c * 512 + lane * 8;
            if (ch < N) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf((v[c][e] - mean) * rstd, gm[c][e], bt[c][e]);
                Frag8<T> f;
                f.from_f32(o);
                f.store(yr + ch);
            }
        }
        if (lane == 0) reinterpret_cast<float2*>(stats)[row] = make_float2(mean, rstd);
    }
}

// Backward: one block of 256 threads per group of consecutive rows; a row is
// spread over the block (lane t of the block takes channels 8t .. 8t+7 of each
// 2048-channel piece), its two sums are block sums through LDS, and each
// thread keeps running sums of dy*xh and dy for its channels over the group's
// rows, written at the end as the group's partial dgamma/dbeta.
template <typename T, int NC>
__global__ void __launch_bounds__(256) dsa3d_layernorm_bwd_kernel(const T* x, const T* gamma, const float* stats,
                                                                  const T* dy, const T* dres, T* dx, float* part_g,
                                                                  float* part_b, int64_t M, int64_t N,
                                                                  int64_t rows_per_group) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_group;
    const int64_t r1 = min(M, r0 + rows_per_group);
    const float inv_n = 1.0f / (float)N;
    float gm[NC][8], ag[NC][8], ab[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t ch = (int64_t)c * 2048 + tid * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gm[c][e] = ch + e < N ? (gamma ? load_scalar<T>(gamma + ch + e) : 1.0f) : 0.0f;
            ag[c][e] = 0.0f;
            ab[c][e] = 0.0f;
        }
    }
    for (int64_t row = r0; row < r1; ++row) {
        const float2 st = reinterpret_cast<const float2*>(stats)[row];
        float xh[NC][8], g[NC][8], gy[NC][8];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t ch = (int64_t)c * 2048 + tid * 8;
            if (ch < N) {
                Frag8<T> fx, fg;
                fx.load(x + row * N + ch);
                fg.load(dy + row * N + ch);
                fx.to_f32(xh[c]);
                fg.to_f32(gy[c]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) { xh[c][e] = 0.0f; gy[c][e] = 0.0f; }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xh[c][e] = (xh[c][e] - st.x) * st.y;
                g[c][e] = gy[c][e] * gm[c][e];
                s1 += g[c][e];
                s2 = fmaf(g[c][e], xh[c][e], s2);
                ag[c][e] = fmaf(gy[c][e], xh[c][e], ag[c][e]);
                ab[c][e] += gy[c][e];
            }
        }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        if (lane == 0) { red[0][wid] = s1; red[1][wid] = s2; }
        __syncthreads();
        const float m1 = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) * inv_n;
        const float m2 = ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) * inv_n;
        __syncthreads();  // every thread has read the sums before the next row writes them
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t ch = (int64_t)c * 2048 + tid * 8;
            if (ch < N) {
                float o[8];
                if (dres) {
                    Frag8<T> fo;
                    fo.load(dres + row * N + ch);
                    fo.to_f32(o);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += st.y * ((g[c][e] - m1) - xh[c][e] * m2);
                Frag8<T> f;
                f.from_f32(o);
                f.store(dx + row * N + ch);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t ch = (int64_t)c * 2048 + tid * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (ch + e < N) {
                part_g[(int64_t)blockIdx.x * N + ch + e] = ag[c][e];
                part_b[(int64_t)blockIdx.x * N + ch + e] = ab[c][e];
            }
    }
}

// out[i] = sum_{z < nsplit} part[z*n + i], z in increasing order.
__global__ void __launch_bounds__(256) dsa3d_ln_split_sum_kernel(const float* part, float* out, int64_t n,
                                                                 int64_t nsplit) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.0f;
        for (int64_t z = 0; z < nsplit; ++z) s += part[z * n + i];
        out[i] = s;
    }
}

namespace {

// Groups of rows of the backward: about 2048 blocks, at most 1024 rows each
// summed in one block, and at least 16 rows per group.
int64_t ln_rows_per_group(int64_t M) {
    int64_t r = (M + 2047) / 2048;
    return std::max<int64_t>(16, std::min<int64_t>(r, 1024));
}

template <typename T, int NC>
hipError_t ln_fwd(int64_t M, int64_t N, float eps, const void* x, const void* gamma, const void* beta, void* y,
                  float* stats, hipStream_t s) {
    const int64_t blocks = std::min<int64_t>((M + 3) / 4, 8192);
    LaunchScope ls(DSA3D_K_LAYERNORM, s);
    hipLaunchKernelGGL((dsa3d_layernorm_kernel<T, NC>), dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const T*>(x), reinterpret_cast<const T*>(gamma),
                       reinterpret_cast<const T*>(beta), reinterpret_cast<T*>(y), stats, M, N, eps);
    return hipGetLastError();
}

template <typename T, int NC>
hipError_t ln_bwd(int64_t M, int64_t N, const void* x, const void* gamma, const float* stats, const void* dy,
                  const void* dres, void* dx, float* part_g, float* part_b, int64_t rpg, hipStream_t s) {
    const int64_t groups = (M + rpg - 1) / rpg;
    LaunchScope ls(DSA3D_K_LAYERNORM_BWD, s);
    hipLaunchKernelGGL((dsa3d_layernorm_bwd_kernel<T, NC>), dim3((unsigned)groups), dim3(256), 0, s,
                       reinterpret_cast<const T*>(x), reinterpret_cast<const T*>(gamma), stats,
                       reinterpret_cast<const T*>(dy), reinterpret_cast<const T*>(dres), reinterpret_cast<T*>(dx), part_g,
                       part_b, M, N, rpg);
    return hipGetLastError();
}

}  // namespace

size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N) {
    const int64_t rpg = ln_rows_per_group(M);
    const int64_t groups = (M + rpg - 1) / rpg;
    return 2 * (((size_t)groups * N * 4 + 255) & ~size_t(255));
}

hipError_t launch_layernorm_forward(int dtype, int64_t M, int64_t N, float eps, const void* x, const void* gamma,
                                    const void* beta, void* y, float* stats, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int nc = (int)((N + 511) / 512);
    const bool f32 = dtype == DSA3D_F32;
    switch (nc) {
#define DSA3D_LN_FWD_CASE(NCV)                                                                   \
    case NCV:                                                                                    \
        return f32 ? ln_fwd<float, NCV>(M, N, eps, x, gamma, beta, y, stats, s)                  \
                   : ln_fwd<bf16_t, NCV>(M, N, eps, x, gamma, beta, y, stats, s);
        DSA3D_LN_FWD_CASE(1) DSA3D_LN_FWD_CASE(2) DSA3D_LN_FWD_CASE(3) DSA3D_LN_FWD_CASE(4)
        DSA3D_LN_FWD_CASE(5) DSA3D_LN_FWD_CASE(6) DSA3D_LN_FWD_CASE(7) DSA3D_LN_FWD_CASE(8)
#undef DSA3D_LN_FWD_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_layernorm_backward(int dtype, int64_t M, int64_t N, const void* x, const void* gamma,
                                     const float* stats, const void* dy, const void* dres, void* dx, float* dgamma,
                                     float* dbeta, void* ws, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int64_t rpg = ln_rows_per_group(M);
    const int64_t groups = (M + rpg - 1) / rpg;
    float* part_g = reinterpret_cast<float*>(ws);
    float* part_b = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (((size_t)groups * N * 4 + 255) & ~size_t(255)));
    const int nc = (int)((N + 2047) / 2048);
    const bool f32 = dtype == DSA3D_F32;
    hipError_t e;
    if (nc == 1)
        e = f32 ? ln_bwd<float, 1>(M, N, x, gamma, stats, dy, dres, dx, part_g, part_b, rpg, s)
                : ln_bwd<bf16_t, 1>(M, N, x, gamma, stats, dy, dres, dx, part_g, part_b, rpg, s);
    else if (nc == 2)
        e = f32 ? ln_bwd<float, 2>(M, N, x, gamma, stats, dy, dres, dx, part_g, part_b, rpg, s)
                : ln_bwd<bf16_t, 2>(M, N, x, gamma, stats, dy, dres, dx, part_g, part_b, rpg, s);
    else
        return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    LaunchScope ls(DSA3D_K_SPLIT_SUM, s);
    const unsigned nb = (unsigned)std::min<int64_t>((N + 255) / 256, 65536);
    if (dgamma) hipLaunchKernelGGL(dsa3d_ln_split_sum_kernel, dim3(nb), dim3(256), 0, s, part_g, dgamma, N, groups);
    if (dbeta) hipLaunchKernelGGL(dsa3d_ln_split_sum_kernel, dim3(nb), dim3(256), 0, s, part_b, dbeta, N, groups);
    return hipGetLastError();
}

}  // namespace dsa3d
