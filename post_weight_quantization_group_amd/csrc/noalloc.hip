// cq_quantize_groups without a caller workspace: the scratch space its kernels need (queue
// counters, group lists and the slice parts of the bounded search) lives in a fixed device array
// of this file, one copy per GPU, so that the call allocates nothing.  For callers that cannot
// allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc.
//
// The array's name is a host-side stand-in in host code; its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that address is handed to
// the kernels.  Every call on one GPU shares the array: the kernels clear their counters at the
// start of each call, and calls that overlap on one GPU race.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <mutex>

#include "cq.h"
#include "launch.h"

namespace {

constexpr size_t ALIGN = 256;
constexpr size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
// The candidate method's workspace for CQ_NOALLOC_MAX_GROUPS groups (the largest of the three
// methods): [tie counter][tie list][binary64 counter][queue][slice parts].
constexpr size_t SCRATCH_BYTES = ALIGN + round_up((size_t)CQ_NOALLOC_MAX_GROUPS * 4u) + ALIGN +
                                 round_up((size_t)CQ_NOALLOC_MAX_GROUPS * 4u) +
                                 round_up(sizeof(cqk::SlicePart) * cqk::SLICE_PARTS);

}  // namespace

// This GPU's scratch space (one copy per device, alive until the process ends).
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];

// The device address of this GPU's copy of `scratch`, looked up on the first call on the device.
hipError_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int32_t cq_quantize_groups_noalloc(const float* w, const float* d, int64_t d_period, int32_t E, int64_t n_groups,
                                   int32_t method, uint16_t* scales, int8_t* codes, double* objective,
                                   uint8_t* flags, uint16_t* pooled_scales, double* pooled_objective, void* stream) {
    if (n_groups > CQ_NOALLOC_MAX_GROUPS) return CQ_ELIMIT;
    if (n_groups < 0 || E < 1 || E > CQ_MAX_ENVS) return CQ_EINVAL;
    const size_t need = cq_workspace_size(method, E, n_groups);
    if (n_groups > 0 && need == 0) return CQ_EINVAL;  // unknown method
    if (need > SCRATCH_BYTES) return CQ_ELIMIT;
    void* ws = nullptr;
    if (n_groups > 0 && scratch_for_current_device(&ws) != hipSuccess) return CQ_EHIP;
    return cq_quantize_groups(w, d, d_period, E, n_groups, method, scales, codes, objective, flags, pooled_scales,
                              pooled_objective, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"
