// Host-side launchers of the gfx950 kernels (called by the C ABI in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e31 {

// ---------------------------------------------------------------- row stats
hipError_t launch_row_stats(const uint16_t* h0, const uint16_t* h1, const uint16_t* h2, int M, int d, int norm,
                            float eps, float* mu, float* rstd, hipStream_t st);

// ------------------------------------------------------------------- decode
// Small-M path: one launch, split-K over W in its stored [3d, d] layout.
struct DecodeArgs {
    const uint16_t* h[3];
    const uint16_t* gamma[3];  // NULL entry: gamma = 1
    const uint16_t* beta[3];   // NULL entry: beta = 0
    const uint16_t* W;         // [3d, d] (stored layout)
    const uint16_t* wt;        // [d, 3d] folded + transposed (folded variant)
    const float* u;            // [3, d] (folded variant)
    const float* c;            // [d] (folded variant)
    const uint16_t* bias;      // [d] or NULL
    uint16_t* out;             // [M, d]
    int M, d;
    float eps;
    int nb;    // column blocks (16*J columns each)
    int kps;   // K chunks per state segment
    int* counters;   // [nb], zero on entry, left zero on exit
    float* stats;    // [nb * 3*kps * 64 * 3]
    float* part;     // [nb * 3*kps * rows * 16*J]
};

struct DecodePlan {
    int J = 8, MT = 1, nb = 0, kps = 0;
    size_t counters_bytes = 0, stats_bytes = 0, part_bytes = 0;
    size_t total() const { return counters_bytes + stats_bytes + part_bytes; }
};

constexpr int DECODE_MAX_M = 64;
DecodePlan plan_decode(int M, int d, int norm, bool folded);
hipError_t launch_decode(const DecodeArgs& a, int norm, bool folded, const DecodePlan& p, hipStream_t st);

// Small-M path on the folded weight: one workgroup per 16 columns over the
// whole K, statistics from the row-statistics pass (no workspace, no atomics).
struct DecodeColsArgs {
    const uint16_t* h[3];
    const uint16_t* wt;   // [d, 3d] folded + transposed
    const float* u;       // [3, d]
    const float* c;       // [d]
    const float* mu;      // [3, M]
    const float* rstd;    // [3, M]
    uint16_t* out;        // [M, d]
    int M, d;
    float eps;
    bool instats;         // statistics in the kernel (M <= 16) instead of mu / rstd
};
hipError_t launch_decode_cols(const DecodeColsArgs& a, int norm, hipStream_t st);

// -------------------------------------------------------------- fold prepare
hipError_t launch_fold_prepare(int d, int norm, const uint16_t* const gamma[3], const uint16_t* const beta[3],
                               const uint16_t* W, const uint16_t* bias, uint16_t* wt, float* u, float* c,
                               hipStream_t st);

// ------------------------------------------------------------------ prefill
// Large-M path: NT GEMM on raw hidden states and the folded, transposed W',
// per-row rescale at the state boundaries (fold), optional split-K.
struct PrefillArgs {
    const uint16_t* h[3];
    const uint16_t* wt;   // [d, 3d] folded + transposed
    const float* u;       // [3, d]
    const float* c;       // [d]
    const float* mu;      // [3, M]
    const float* rstd;    // [3, M]
    uint16_t* out;        // [M, d]
    int M, d;
    int norm;
    int splits;           // 1 or a multiple of 3
    int* counters;        // [tiles] for split-K
    float* part;          // split partials
};

struct PrefillPlan {
    int splits = 1;
    int tiles_m = 0, tiles_n = 0;
    size_t counters_bytes = 0, part_bytes = 0;
};

PrefillPlan plan_prefill(int M, int d);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st);

// zero-fill helper (a kernel, not hipMemsetAsync)
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace e31
