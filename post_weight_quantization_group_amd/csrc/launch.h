// Internal launchers of the gfx950 kernels (host side, C++ linkage).
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
    int32_t* zero_also;   // nullable: another counter to clear with tie_count (one launch)
};
hipError_t launch_candidate(const CandArgs& a, int E, hipStream_t st);

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st);

hipError_t launch_pack(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                       int32_t* qweight, uint16_t* scales, hipStream_t st);

// W4A16 matmul y [M][out] = x [M][in] (bf16) times the GPTQ-v1 tensors dequantized.
hipError_t launch_w4a16(const uint16_t* x, const int32_t* qw, const uint16_t* scales, int64_t M, int64_t out,
                        int64_t in, float* y, hipStream_t st);

// Environment diagonals from bf16 activations [E][T][in] into d [in/128][E][128]; part
// (E * diag_chunks * in) and msq (E * in) are workspace.
int64_t diag_chunks(int E, int64_t T, int64_t in);
hipError_t launch_diagonals(const uint16_t* x, int E, int64_t T, int64_t in, float* d, double* part, double* msq,
                            hipStream_t st);

// Held-out comparison of two policies' per-group values: counts, effect, sorted bootstrap
// replicates and the percentile interval; mm ((B + 1) * M), reps (B) and rank (B) are workspace.
hipError_t launch_heldout(const double* pa, const double* pb, int64_t n, const int64_t* off, int M,
                          const int32_t* idx, int B, double alpha, int64_t* counts, double* effect,
                          double* boot, double* ci, double* mm, double* reps, int32_t* rank, hipStream_t st);

hipError_t launch_proxy(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups, int P,
                        const uint16_t* scales, const int64_t* module_offsets, int n_modules,
                        double* module_mean, double* macro, double* per_group, hipStream_t st);

}  // namespace cqk
