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

int fwd_groups_per_block(int head_dim, int P);
size_t bwd_accumulator_bytes_per_head(const dsa3d_desc& d);
void proj_bwd_splits(const dsa3d_desc& d, int& dw_splits, int& db_splits);
size_t proj_bwd_workspace_bytes(const dsa3d_desc& d);

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

}  // namespace dsa3d
