// dsa3d_api.cpp -- the extern "C" boundary of libdsa3d: argument checks,
// workspace sizing and launches on the caller's stream. No C++ exception and
// no HIP allocation happens here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "dsa3d.h"
#include "dsa3d_internal.h"

namespace {

constexpr size_t kBackwardPassCap = size_t(16) << 30;  // recommended cap on one backward pass's workspace

bool pow2_in(int32_t x, int32_t lo, int32_t hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps) {
        if (p == nullptr) return DSA3D_ERR_INVALID_ARG;
    }
    for (const void* p : ps) {
        if (!aligned16(p)) return DSA3D_ERR_MISALIGNED;
    }
    return DSA3D_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_HIP; }

int64_t tokens(const dsa3d_desc& d) { return d.B * d.T * d.H * d.W; }

}  // namespace

namespace dsa3d {
dsa3d_launch_log*& launch_log() {
    static thread_local dsa3d_launch_log* log = nullptr;
    return log;
}
}  // namespace dsa3d

extern "C" {

int dsa3d_version(void) { return 100; }

int dsa3d_set_launch_log(dsa3d_launch_log* log) {
    if (log != nullptr && log->capacity > 0 &&
        (log->kernel == nullptr || log->start == nullptr || log->stop == nullptr))
        return DSA3D_ERR_INVALID_ARG;
    dsa3d::launch_log() = log;
    return DSA3D_OK;
}

const char* dsa3d_status_string(int status) {
    switch (status) {
        case DSA3D_OK: return "ok";
        case DSA3D_ERR_INVALID_ARG: return "invalid argument";
        case DSA3D_ERR_UNSUPPORTED: return "unsupported configuration";
        case DSA3D_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case DSA3D_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA3D_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int dsa3d_validate(const dsa3d_desc* d) {
    if (d == nullptr) return DSA3D_ERR_INVALID_ARG;
    if (d->B < 1 || d->T < 1 || d->H < 1 || d->W < 1) return DSA3D_ERR_INVALID_ARG;
    if (d->T >= (1 << 30) || d->H >= (1 << 30) || d->W >= (1 << 30)) return DSA3D_ERR_INVALID_ARG;
    const int64_t ntok = tokens(*d);
    if (ntok / d->B / d->T / d->H != d->W || ntok >= (int64_t(1) << 31)) return DSA3D_ERR_INVALID_ARG;
    if (d->heads < 1 || d->head_dim < 1) return DSA3D_ERR_INVALID_ARG;
    if (d->kt < 1 || d->kh < 1 || d->kw < 1) return DSA3D_ERR_INVALID_ARG;
    if (d->kt % 2 == 0 || d->kh % 2 == 0 || d->kw % 2 == 0) return DSA3D_ERR_INVALID_ARG;
    if (d->kt > 1023 || d->kh > 1023 || d->kw > 1023) return DSA3D_ERR_INVALID_ARG;
    if ((int64_t)d->kt * d->kh * d->kw != d->P) return DSA3D_ERR_INVALID_ARG;
    if (d->dil_t < 1 || d->dil_h < 1 || d->dil_w < 1) return DSA3D_ERR_INVALID_ARG;
    if (d->dil_t > (1 << 20) || d->dil_h > (1 << 20) || d->dil_w > (1 << 20)) return DSA3D_ERR_INVALID_ARG;
    if (!(d->scale >= 0.0f) || d->scale == __builtin_inff()) return DSA3D_ERR_INVALID_ARG;
    if (d->deterministic != 0 && d->deterministic != 1) return DSA3D_ERR_INVALID_ARG;
    if (d->dtype != DSA3D_F32 && d->dtype != DSA3D_BF16) return DSA3D_ERR_UNSUPPORTED;
    if (!pow2_in(d->head_dim, 8, 256)) return DSA3D_ERR_UNSUPPORTED;
    if (d->P > 1024) return DSA3D_ERR_UNSUPPORTED;
    if ((int64_t)d->heads * d->head_dim > (1 << 20)) return DSA3D_ERR_UNSUPPORTED;
    return DSA3D_OK;
}

size_t dsa3d_workspace_min(const dsa3d_desc* d, int kind) {
    if (dsa3d_validate(d) != DSA3D_OK) return 0;
    switch (kind) {
        case DSA3D_WS_BACKWARD: return dsa3d::bwd_workspace_bytes(*d, 1);
        case DSA3D_WS_PROJ_BACKWARD: return dsa3d::proj_bwd_workspace_bytes(*d);
        case DSA3D_WS_DWCONV_BACKWARD: return dsa3d::dwconv_bwd_workspace_bytes(*d);
        case DSA3D_WS_BACKWARD_FIXED: return dsa3d::fixed_bwd_workspace_bytes(*d);
        default: return 0;
    }
}

size_t dsa3d_workspace_size(const dsa3d_desc* d, int kind) {
    if (dsa3d_validate(d) != DSA3D_OK) return 0;
    if (kind == DSA3D_WS_BACKWARD) {
        const size_t one = dsa3d::bwd_workspace_bytes(*d, 1);
        if (one == 0) return 0;
        const int64_t nh = dsa3d::bwd_heads_per_pass(*d, kBackwardPassCap);
        return nh >= 1 ? dsa3d::bwd_workspace_bytes(*d, nh) : one;
    }
    return dsa3d_workspace_min(d, kind);
}

int dsa3d_offset_proj_forward(const dsa3d_desc* d, const void* q, const void* w, const void* bias, void* offsets,
                              void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, w, offsets})) != DSA3D_OK) return rc;
    if (bias != nullptr && !aligned16(bias)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_proj_forward(*d, q, w, bias, offsets, static_cast<hipStream_t>(stream)));
}

int dsa3d_forward(const dsa3d_desc* d, const void* q, const void* k, const void* v, const void* offsets, void* out,
                  float* lse, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, k, v, out, lse})) != DSA3D_OK) return rc;
    if (offsets == nullptr)  // fixed window: every offset zero
        return hip_status(dsa3d::launch_fixed_forward(*d, q, k, v, out, lse, static_cast<hipStream_t>(stream)));
    if (!aligned16(offsets)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_forward(*d, q, k, v, offsets, out, lse, static_cast<hipStream_t>(stream)));
}

int dsa3d_backward(const dsa3d_desc* d, const void* q, const void* k, const void* v, const void* offsets,
                   const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* doffsets,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, k, v, out, lse, dout, dq, dk, dv})) != DSA3D_OK) return rc;
    if ((offsets == nullptr) != (doffsets == nullptr)) return DSA3D_ERR_INVALID_ARG;
    if (offsets == nullptr) {  // fixed window: every offset zero, no offset gradient
        if (workspace == nullptr || workspace_bytes < dsa3d::fixed_bwd_workspace_bytes(*d))
            return DSA3D_ERR_WORKSPACE;
        if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
        return hip_status(dsa3d::launch_fixed_backward(*d, q, k, v, out, lse, dout, dq, dk, dv, workspace,
                                                       static_cast<hipStream_t>(stream)));
    }
    if (!aligned16(offsets) || !aligned16(doffsets)) return DSA3D_ERR_MISALIGNED;
    const size_t need = dsa3d::bwd_workspace_bytes(*d, 1);
    if (need == 0) return DSA3D_ERR_UNSUPPORTED;  // sample or cell numbers of one head exceed 32 bits
    if (workspace == nullptr || workspace_bytes < need) return DSA3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_backward(*d, q, k, v, offsets, out, lse, dout, dq, dk, dv, doffsets, workspace,
                                             workspace_bytes, static_cast<hipStream_t>(stream)));
}

int dsa3d_offset_proj_backward(const dsa3d_desc* d, const void* q, const void* w, const void* doffsets,
                               void* dq_accum, float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                               void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, w, doffsets, dq_accum, dw})) != DSA3D_OK) return rc;
    if (dbias != nullptr && !aligned16(dbias)) return DSA3D_ERR_MISALIGNED;
    const size_t need = dsa3d::proj_bwd_workspace_bytes(*d);
    if (workspace == nullptr || workspace_bytes < need) return DSA3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_proj_backward(*d, q, w, doffsets, dq_accum, dw, dbias, workspace,
                                                  static_cast<hipStream_t>(stream)));
}

int dsa3d_dwconv_forward(const dsa3d_desc* d, const void* q, const void* wt, const void* bias, void* y, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, wt, y})) != DSA3D_OK) return rc;
    if (bias != nullptr && !aligned16(bias)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_dwconv_forward(*d, q, wt, bias, y, static_cast<hipStream_t>(stream)));
}

int dsa3d_dwconv_backward(const dsa3d_desc* d, const void* q, const void* wt, const void* dy, void* dq_accum,
                          float* dwt, float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({q, wt, dy, dq_accum, dwt})) != DSA3D_OK) return rc;
    if (dbias != nullptr && !aligned16(dbias)) return DSA3D_ERR_MISALIGNED;
    const size_t need = dsa3d::dwconv_bwd_workspace_bytes(*d);
    if (workspace == nullptr || workspace_bytes < need) return DSA3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_dwconv_backward(*d, q, wt, dy, dq_accum, dwt, dbias, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

static bool hybrid_g_ok(int32_t G) { return G >= 1 && G <= 1024; }

size_t dsa3d_hybrid_workspace_size(const dsa3d_desc* d, int32_t G, int kind) {
    if (dsa3d_validate(d) != DSA3D_OK || !hybrid_g_ok(G)) return 0;
    if (kind != DSA3D_WS_BACKWARD && kind != DSA3D_WS_BACKWARD_FIXED) return 0;
    return std::max(dsa3d_workspace_size(d, kind), dsa3d::hybrid_global_workspace_bytes(*d, G));
}

size_t dsa3d_hybrid_workspace_min(const dsa3d_desc* d, int32_t G, int kind) {
    if (dsa3d_validate(d) != DSA3D_OK || !hybrid_g_ok(G)) return 0;
    if (kind != DSA3D_WS_BACKWARD && kind != DSA3D_WS_BACKWARD_FIXED) return 0;
    const size_t local = dsa3d_workspace_min(d, kind);
    if (local == 0) return 0;
    return std::max(local, dsa3d::hybrid_global_workspace_bytes(*d, G));
}

int dsa3d_forward_hybrid(const dsa3d_desc* d, const void* q, const void* k, const void* v, const void* offsets,
                         int32_t G, const void* gk, const void* gv, void* out, float* lse, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if (!hybrid_g_ok(G)) return DSA3D_ERR_INVALID_ARG;
    if ((rc = check_ptrs({gk, gv})) != DSA3D_OK) return rc;
    if ((rc = dsa3d_forward(d, q, k, v, offsets, out, lse, stream)) != DSA3D_OK) return rc;
    return hip_status(dsa3d::launch_hybrid_forward(*d, G, q, gk, gv, out, lse, static_cast<hipStream_t>(stream)));
}

int dsa3d_backward_hybrid(const dsa3d_desc* d, const void* q, const void* k, const void* v, const void* offsets,
                          const void* out, const float* lse, const void* dout, int32_t G, const void* gk,
                          const void* gv, void* dq, void* dk, void* dv, void* doffsets, void* dgk, void* dgv,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if (!hybrid_g_ok(G)) return DSA3D_ERR_INVALID_ARG;
    if ((rc = check_ptrs({gk, gv, dgk, dgv})) != DSA3D_OK) return rc;
    if (workspace == nullptr || workspace_bytes < dsa3d::hybrid_global_workspace_bytes(*d, G))
        return DSA3D_ERR_WORKSPACE;
    // the operator's backward (it checks its own arguments and workspace), then the global rows on the
    // same workspace
    if ((rc = dsa3d_backward(d, q, k, v, offsets, out, lse, dout, dq, dk, dv, doffsets, workspace, workspace_bytes,
                             stream)) != DSA3D_OK)
        return rc;
    return hip_status(dsa3d::launch_hybrid_backward(*d, G, q, gk, gv, out, lse, dout, dq, dgk, dgv, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

static int check_dtype(int dtype) { return dtype == DSA3D_F32 || dtype == DSA3D_BF16 ? DSA3D_OK : DSA3D_ERR_UNSUPPORTED; }

static bool size_ok(int64_t x) { return x >= 1 && x < (int64_t(1) << 31); }

static int check_layernorm(int dtype, int64_t M, int64_t N) {
    if (!size_ok(M) || !size_ok(N)) return DSA3D_ERR_INVALID_ARG;
    if (check_dtype(dtype) != DSA3D_OK) return DSA3D_ERR_UNSUPPORTED;
    if (N % 8 != 0 || N > 4096) return DSA3D_ERR_UNSUPPORTED;
    return DSA3D_OK;
}

static int check_linear(int dtype, int64_t M, int64_t N, int64_t K) {
    if (!size_ok(M) || !size_ok(N) || !size_ok(K)) return DSA3D_ERR_INVALID_ARG;
    if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31) ||
        ((N + 255) / 256) * ((K + 255) / 256) >= (int64_t(1) << 31))
        return DSA3D_ERR_UNSUPPORTED;
    return check_dtype(dtype);
}

int dsa3d_layernorm_forward(int dtype, int64_t M, int64_t N, float eps, const void* x, const void* gamma,
                            const void* beta, void* y, float* stats, void* stream) {
    int rc = check_layernorm(dtype, M, N);
    if (rc != DSA3D_OK) return rc;
    if (!(eps > 0.0f) || eps == __builtin_inff()) return DSA3D_ERR_INVALID_ARG;
    if ((rc = check_ptrs({x, y, stats})) != DSA3D_OK) return rc;
    if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return DSA3D_ERR_MISALIGNED;
    if (x == y) return DSA3D_ERR_INVALID_ARG;
    return hip_status(
        dsa3d::launch_layernorm_forward(dtype, M, N, eps, x, gamma, beta, y, stats, static_cast<hipStream_t>(stream)));
}

size_t dsa3d_layernorm_workspace_size(int64_t M, int64_t N) {
    if (!size_ok(M) || !size_ok(N) || N % 8 != 0 || N > 4096) return 0;
    return dsa3d::layernorm_bwd_workspace_bytes(M, N);
}

int dsa3d_layernorm_backward(int dtype, int64_t M, int64_t N, const void* x, const void* gamma, const float* stats,
                             const void* dy, const void* dres, void* dx, float* dgamma, float* dbeta, void* workspace,
                             size_t workspace_bytes, void* stream) {
    int rc = check_layernorm(dtype, M, N);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({x, stats, dy, dx})) != DSA3D_OK) return rc;
    if ((gamma && !aligned16(gamma)) || (dgamma && !aligned16(dgamma)) || (dbeta && !aligned16(dbeta)) ||
        (dres && !aligned16(dres)))
        return DSA3D_ERR_MISALIGNED;
    if (dx == x || dx == dy) return DSA3D_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < dsa3d::layernorm_bwd_workspace_bytes(M, N)) return DSA3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
    return hip_status(dsa3d::launch_layernorm_backward(dtype, M, N, x, gamma, stats, dy, dres, dx, dgamma, dbeta,
                                                       workspace, static_cast<hipStream_t>(stream)));
}

int dsa3d_linear_forward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w, const void* bias,
                         const void* residual, void* y, void* stream) {
    int rc = check_linear(dtype, M, N, K);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({x, w, y})) != DSA3D_OK) return rc;
    if ((bias && !aligned16(bias)) || (residual && !aligned16(residual))) return DSA3D_ERR_MISALIGNED;
    if (x == y || w == y) return DSA3D_ERR_INVALID_ARG;
    return hip_status(dsa3d::launch_linear_forward(dtype, M, N, K, x, w, bias, residual, y, DSA3D_K_LINEAR_FORWARD,
                                                   static_cast<hipStream_t>(stream)));
}

size_t dsa3d_linear_workspace_size(int dtype, int64_t M, int64_t N, int64_t K) {
    if (check_linear(dtype, M, N, K) != DSA3D_OK) return 0;
    return dsa3d::linear_bwd_workspace_bytes(dtype, M, N, K);
}

int dsa3d_linear_backward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w, const void* dy,
                          const void* dres, void* dx, float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                          void* stream) {
    int rc = check_linear(dtype, M, N, K);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({x, w, dy, dx, dw})) != DSA3D_OK) return rc;
    if ((dbias && !aligned16(dbias)) || (dres && !aligned16(dres))) return DSA3D_ERR_MISALIGNED;
    if (dx == dy || dx == w || dx == x) return DSA3D_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < dsa3d::linear_bwd_workspace_bytes(dtype, M, N, K))
        return DSA3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA3D_ERR_MISALIGNED;
    const dsa3d::LinearKernelIds ids{DSA3D_K_TRANSPOSE, DSA3D_K_LINEAR_BWD_DX, DSA3D_K_LINEAR_BWD_DW};
    return hip_status(dsa3d::launch_linear_backward(dtype, M, N, K, x, w, dy, dres, dx, dw, dbias, workspace, ids,
                                                    static_cast<hipStream_t>(stream)));
}

int dsa3d_debug_geometry(const dsa3d_desc* d, const void* offsets, int32_t* base, float* frac, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    if ((rc = check_ptrs({offsets, base, frac})) != DSA3D_OK) return rc;
    return hip_status(dsa3d::launch_geometry(*d, offsets, base, frac, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
