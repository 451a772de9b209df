// Arguments and launchers of the three scale searches (full grid, bounded search, candidate
// solver): host side, C++ linkage.  Kept apart from the other launchers so that a kernel's sources
// are its .hip file, device.h and this header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cqk {

// One slice's share of a group's binary32 screen when several workgroups split the scale range:
// per policy (0 minimax, 1 pooled) the slice's best and second keys (value bits << 32 | pattern),
// the keys within the screen ratio of the slice's best, and the smallest value it could not keep.
constexpr int SLICE_KEYS = 128;
struct SlicePart {
    uint32_t status;  // 0 screened, 1 bad input, 2 outside the screen's range
    uint32_t n[2];
    uint32_t ov[2];   // binary32 bits of the smallest value not stored (0xFFFFFFFF: none)
    uint32_t b_top;   // last pattern screened (the same in every slice)
    uint64_t m1[2], s2[2];
    uint64_t keys[2][SLICE_KEYS];
};
constexpr int SLICE_PARTS = 2048;  // parts in a sweep workspace
constexpr int LIST_SLICES = 8;     // slices per listed group
constexpr int LIST_SLICED = SLICE_PARTS / LIST_SLICES;  // listed groups handled by slices

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
    SlicePart* parts;          // SLICE_PARTS entries of workspace
    int slices;                // workgroups per group (set by the launcher)
    int list_split;            // indirect mode: workgroups below this serve the sliced entries,
                               // the others one entry each (set by the launcher)
    int fb_zeroed;             // the caller has zeroed fb_count earlier on the same stream
};

// Exhaustive sweep (binary32 screen + binary64 rescoring + binary64 sweep of
// unsettled groups) for n_groups groups, or for the groups listed in
// a.list when a.list is set (then n_groups bounds the list length).
hipError_t launch_sweep(const SweepArgs& a, int E, int64_t n_groups, hipStream_t st);

// Full-grid exhaustive search (every scale, every weight; binary32 screen, binary64 rescoring,
// binary64 sweep of unsettled groups) for groups of G weights and codes in [qmin, qmax].
struct FullArgs {
    const float* w;            // [n_groups][G]
    const float* d;            // [n_d][E][G]
    int64_t d_period;
    int E;                     // environments in d (kernels run the next power of two, zero-padded)
    int G;                     // 1..256
    int qmin, qmax;            // -128 <= qmin <= 0 <= qmax <= 127, qmin < qmax
    float ratio;               // shortlist ratio (fullgrid_ratio)
    int64_t group_offset;      // first group of this launch (set by the launcher)
    uint16_t* scales;
    int8_t* codes;             // [n_groups][G]
    double* objective;
    uint8_t* flags;
    uint16_t* pscales;
    double* pobjective;
    int want_minimax;
    int want_pooled;
    int32_t* fb_count;         // groups queued for the binary64 sweep (cleared by the launcher)
    int32_t* fb_list;          // n_groups entries
    SlicePart* parts;          // SLICE_PARTS entries (few groups split over slices); nullable
    int slices;                // workgroups per group (set by the launcher)
    const int32_t* list;       // list mode: the group ids to search (nullable: groups 0..n_groups-1)
    const int32_t* list_count; // list mode: device count of `list` (at most n_groups)
    uint8_t flag_or;           // ORed into every flags byte written (CQ_FLAG_FALLBACK in list mode)
};
float fullgrid_ratio(int G, int qmin, int qmax, int E);
hipError_t launch_fullgrid(const FullArgs& a, int E, int64_t n_groups, hipStream_t st);

struct CandArgs {
    const float* w;       // [n_groups][G]
    const float* d;       // [n_d][E][G]
    int64_t d_period;
    int E;
    int G;                // 1..128 weights per group (the kernel pads to 128 with zero weights)
    int qmin, qmax;       // code range: -8 <= qmin <= 0 <= qmax <= 8, qmin < qmax
    float start_ratio;    // binary32 1/(max(qmax, -qmin) + 1): the probe scale is max|w| times this
    int64_t n_groups;
    uint16_t* scales;
    int8_t* codes;
    double* objective;
    uint8_t* flags;
    int32_t* tie_count;   // groups handed to the exhaustive sweep
    int32_t* tie_list;
    int32_t* zero_also;   // nullable: another counter to clear with tie_count (one launch)
};
hipError_t launch_candidate(const CandArgs& a, int E, hipStream_t st);

}  // namespace cqk
