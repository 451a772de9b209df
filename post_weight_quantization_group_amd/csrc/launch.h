// Internal launchers of the gfx950 kernels (host side, C++ linkage).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cqk {

struct SweepArgs {
    const float* w;
    const float* d;
    int64_t d_period;
    int E;                     // environments in d; kernels run the next power of two, padded
                               // with zero diagonals (which change no maximum and no sum)
    int64_t group_offset;      // direct mode: first group of this launch
    const int32_t* list;       // indirect mode: group ids (nullable)
    const int32_t* list_count; // indirect mode: device count of `list`
    uint16_t* scales;
    int8_t* codes;
    double* objective;
    uint8_t* flags;
    uint16_t* pscales;
    double* pobjective;
    int32_t* fb_count;         // groups queued for the binary64 sweep
    int32_t* fb_list;
    int want_minimax;
    int want_pooled;
    int mark_fallback;         // OR CQ_FLAG_FALLBACK into the flags written
};

// Exhaustive sweep (binary32 screen + binary64 rescoring + binary64 sweep of
// unsettled groups) for n_groups groups, or for the groups listed in
// a.list when a.list is set (then n_groups bounds the list length).
hipError_t launch_sweep(const SweepArgs& a, int E, int64_t n_groups, hipStream_t st);

struct CandArgs {
    const float* w;
    const float* d;
    int64_t d_period;
    int E;
    int64_t n_groups;
    uint16_t* scales;
    int8_t* codes;
    double* objective;
    uint8_t* flags;
    int32_t* tie_count;   // groups handed to the exhaustive sweep
    int32_t* tie_list;
};
hipError_t launch_candidate(const CandArgs& a, int E, hipStream_t st);

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st);

hipError_t launch_pack(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                       int32_t* qweight, uint16_t* scales, hipStream_t st);

hipError_t launch_proxy(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                        const uint16_t* scales, const int64_t* module_offsets, int n_modules,
                        double* module_mean, double* macro, double* per_group, hipStream_t st);

}  // namespace cqk
