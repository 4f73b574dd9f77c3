// dsa3d_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "dsa3d.h"

namespace dsa3d {

// Opt-in per-launch event log of the calling host thread (dsa3d_set_launch_log).
dsa3d_launch_log*& launch_log();

// Brackets one kernel launch with the log's events, if a log is set.
class LaunchScope {
public:
    LaunchScope(int kernel, hipStream_t s) : log_(launch_log()), s_(s), slot_(-1) {
        if (log_ && log_->count < log_->capacity) {
            slot_ = log_->count++;
            log_->kernel[slot_] = kernel;
            (void)hipEventRecord(static_cast<hipEvent_t>(log_->start[slot_]), s_);
        }
    }
    ~LaunchScope() {
        if (slot_ >= 0) (void)hipEventRecord(static_cast<hipEvent_t>(log_->stop[slot_]), s_);
    }
    LaunchScope(const LaunchScope&) = delete;
    LaunchScope& operator=(const LaunchScope&) = delete;

private:
    dsa3d_launch_log* log_;
    hipStream_t s_;
    int slot_;
};

// Instantiates FN<D>(args...) for the supported head dimensions.
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

// Same, assigning FN<D>(args...) to E_ instead of returning it.
#define DSA3D_DISPATCH_D_E(D_, FN, E_, ...)                  \
    switch (D_) {                                           \
        case 8: E_ = FN<8>(__VA_ARGS__); break;             \
        case 16: E_ = FN<16>(__VA_ARGS__); break;           \
        case 32: E_ = FN<32>(__VA_ARGS__); break;           \
        case 64: E_ = FN<64>(__VA_ARGS__); break;           \
        case 128: E_ = FN<128>(__VA_ARGS__); break;         \
        case 256: E_ = FN<256>(__VA_ARGS__); break;         \
        default: E_ = hipErrorInvalidValue; break;          \
    }

struct Window;
struct TaskGrid;
struct BlockOrder;
// Supertile of the attention kernels' block order: the XCDs take one
// supertile of (at most) frames x rows x tokens each in turn, so the eight
// supertiles in flight are neighbours and the rows their samples gather are
// shared through the memory-side cache. A negative `rows` asks for bands of
// about -rows rows of equal height (68 rows and -14: five bands of 14 or 13).
struct Supertile {
    int frames, rows, tokens;
};
// Fixed-window kernels (one token per task). Measured on the 256x68x120 grid
// (3x5x5 window, offsets N(0,2)) for the deformable kernels: the step runs 15%
// faster than with one contiguous range of 4 x 8 x 64 supertiles per XCD.
constexpr Supertile kGatherSupertile = {16, 32, 16};
// Forward: 64 frames x bands of ~14 rows x 16 tokens, 520-524 ms on that grid,
// against 529-539 ms with bands of ~23 rows, 551-554 with ~12 or ~17, and
// 558-562 ms with 16 x 32 x 16.
constexpr Supertile kForwardSupertile = {64, -14, 16};
// Backward query kernel: 32 frames x bands of ~14 rows x 16 tokens, 1-2% faster
// per pass than 32 x ~23 x 16 or 16 x 32 x 16.
constexpr Supertile kQuerySupertile = {32, -14, 16};
// Key kernel (tasks of 2 frames x 2 tokens; its frames count pairs of frames):
// 32 frames x 16 rows x 32 tokens, deeper in t and shallower in h than the
// others; on the same grid 72 ms per 3-head pass, against 76 ms with tasks of
// one frame and 91 ms with those at 16 x 32 x 32.
constexpr Supertile kKeySupertile = {16, 16, 32};
// Block order for tasks of G tokens along w; `tuning_env` names the variable
// that overrides the supertile in tuning builds.
BlockOrder make_block_order(const dsa3d_desc& d, int G, Supertile st, const char* tuning_env);
int attn_tokens_per_block(int head_dim);
Window make_window(const dsa3d_desc& d);
TaskGrid make_task_grid(const dsa3d_desc& d, int32_t head0, int32_t nheads);
float logit_scale(const dsa3d_desc& d);
unsigned grid_for(int64_t n, int threads, int64_t cap = 1 << 20);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

// Backward workspace: bytes for a pass over `nheads` heads (0 if such a pass
// cannot be indexed with 32-bit sample and cell numbers) and the largest head
// count per pass that fits in `ws_bytes`.
size_t bwd_workspace_bytes(const dsa3d_desc& d, int64_t nheads);
int64_t bwd_heads_per_pass(const dsa3d_desc& d, size_t ws_bytes);

void proj_bwd_splits(const dsa3d_desc& d, int& dw_splits, int& db_splits);
size_t proj_bwd_workspace_bytes(const dsa3d_desc& d);

// Linear layers y[M, N] = x[M, K] . w[N, K]^T + bias (+ residual): the offset
// projection is one (M = tokens, N = heads*P*3, K = heads*head_dim).
struct LinearKernelIds {
    int transpose, dx, dw;  // launch-log ids of the backward's kernels
};
void linear_bwd_splits(int dtype, int64_t M, int64_t N, int64_t K, int& dw_splits, int& db_splits);
size_t linear_bwd_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_forward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                 const void* bias, const void* residual, void* y, int kernel_id, hipStream_t s);
hipError_t launch_linear_backward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                  const void* dy, const void* dres, void* dx, float* dw, float* db, void* ws,
                                  const LinearKernelIds& ids, hipStream_t s);

hipError_t launch_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                          void* out, float* lse, hipStream_t s);
hipError_t launch_backward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* doff, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_geometry(const dsa3d_desc& d, const void* off, int32_t* base, float* frac, hipStream_t s);
hipError_t launch_proj_forward(const dsa3d_desc& d, const void* q, const void* w, const void* bias, void* off,
                               hipStream_t s);
hipError_t launch_proj_backward(const dsa3d_desc& d, const void* q, const void* w, const void* doff, void* dq,
                                float* dw, float* db, void* ws, hipStream_t s);
size_t dwconv_bwd_workspace_bytes(const dsa3d_desc& d);
size_t fixed_bwd_workspace_bytes(const dsa3d_desc& d);
hipError_t launch_fixed_forward(const dsa3d_desc& d, const void* q, const void* k, const void* v, void* out,
                                float* lse, hipStream_t s);
hipError_t launch_fixed_backward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                                 hipStream_t s);
size_t hybrid_global_workspace_bytes(const dsa3d_desc& d, int32_t G);
hipError_t launch_hybrid_forward(const dsa3d_desc& d, int32_t G, const void* q, const void* gk, const void* gv,
                                 void* out, float* lse, hipStream_t s);
hipError_t launch_hybrid_backward(const dsa3d_desc& d, int32_t G, const void* q, const void* gk, const void* gv,
                                  const void* out, const float* lse, const void* dout, void* dq, void* dgk, void* dgv,
                                  void* ws, hipStream_t s);
size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N);
hipError_t launch_layernorm_forward(int dtype, int64_t M, int64_t N, float eps, const void* x, const void* gamma,
                                    const void* beta, void* y, float* stats, hipStream_t s);
hipError_t launch_layernorm_backward(int dtype, int64_t M, int64_t N, const void* x, const void* gamma,
                                     const float* stats, const void* dy, const void* dres, void* dx, float* dgamma,
                                     float* dbeta, void* ws, hipStream_t s);
hipError_t launch_dwconv_forward(const dsa3d_desc& d, const void* q, const void* w, const void* bias, void* y,
                                 hipStream_t s);
hipError_t launch_dwconv_backward(const dsa3d_desc& d, const void* q, const void* w, const void* dy, void* dq,
                                  float* dw, float* db, void* ws, hipStream_t s);

}  // namespace dsa3d
