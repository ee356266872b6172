// Host-side launchers of the gfx950 kernels (called by the C ABI in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e31 {

// ---------------------------------------------------------------- row view
// Where a call's rows are.  Token m reads row src(m) of each state s, at
// h[s] + src(m) * ld[s] (elements), with src(m) = idx[m] when an index list
// is given, else m; its output row is at out + m * ld_out.  An index outside
// [0, n_src) reads row 0 instead, and that token's output row is written as
// zeros.
struct RowView {
    long long ld[3] = {0, 0, 0};
    long long ld_out = 0;
    const int32_t* idx = nullptr;  // [M] (device) or null
    int n_src = 0;                 // rows of each state buffer an index may name
};
inline RowView dense_rows(int M, int d) {
    RowView v;
    v.ld[0] = v.ld[1] = v.ld[2] = d;
    v.ld_out = d;
    v.n_src = M;
    return v;
}
// leading dimension of state s (selects, no dynamic indexing of the argument)
__device__ __forceinline__ long long rv_ld(const RowView& v, int s) {
    return s == 0 ? v.ld[0] : (s == 1 ? v.ld[1] : v.ld[2]);
}
// source row of token m and whether it is valid (row 0 when it is not)
__device__ __forceinline__ int rv_src(const RowView& v, int m, bool& ok) {
    if (v.idx == nullptr) {
        ok = true;
        return m;
    }
    const int r = v.idx[m];
    ok = r >= 0 && r < v.n_src;
    return ok ? r : 0;
}
// For calls of at most 128 tokens, per wave: lane l holds the source rows
// of tokens l and 64 + l (0 from M on), and masks of the valid tokens.
struct WaveRows {
    int src, src_hi;
    uint64_t ok, ok_hi;
};
__device__ __forceinline__ WaveRows rv_wave(const RowView& v, int M) {
    const int lane = threadIdx.x & 63;
    bool ok = false, ok_hi = false;
    int src = 0, src_hi = 0;
    if (lane < M) src = rv_src(v, lane, ok);
    if (64 + lane < M) src_hi = rv_src(v, 64 + lane, ok_hi);
    WaveRows w;
    w.src = src;
    w.src_hi = src_hi;
    w.ok = __ballot(ok);
    w.ok_hi = __ballot(ok_hi);
    return w;
}
// token m's source row (m < 128, any lane); m itself without an index list
__device__ __forceinline__ int rv_lane_src(const RowView& v, const WaveRows& w, int m) {
    if (v.idx == nullptr) return m;
    const int lo = __shfl(w.src, m & 63, 64), hi = __shfl(w.src_hi, m & 63, 64);
    return m < 64 ? lo : hi;
}
__device__ __forceinline__ bool rv_ok(const WaveRows& w, int m) {
    return (((m < 64 ? w.ok : w.ok_hi) >> (m & 63)) & 1ull) != 0;
}

// ---------------------------------------------------------------- row stats
// Post-norm feedback rows (out = norm(x) * gamma + beta, one row per wave).
constexpr int NORM_ROWS_MAX_D = 8192;
hipError_t launch_norm_rows(const uint16_t* x, int M, int d, int norm, float eps, const uint16_t* gamma,
                            const uint16_t* beta, uint16_t* out, hipStream_t st);

// Drafter-input concatenation (dst[m] = [embed[tokens[m]] | fused[m]]).
constexpr int EMBED_CONCAT_MAX_D = 8192;
hipError_t launch_embed_concat(const int32_t* tokens, int M, int d, int vocab, const uint16_t* embed,
                               const uint16_t* fused, uint16_t* dst, int32_t* bad_count, hipStream_t st);

hipError_t launch_row_stats(const uint16_t* h0, const uint16_t* h1, const uint16_t* h2, const RowView& rv, int M,
                            int d, int norm, float eps, float* mu, float* rstd, hipStream_t st);

// ------------------------------------------------------------------- decode
// Small-M path on the stored W: one launch, split-K over W in its [3d, d]
// layout, the norm applied to the A operand (LayerNorm with a shift).
struct DecodeArgs {
    const uint16_t* h[3];
    const uint16_t* gamma[3];  // NULL entry: gamma = 1
    const uint16_t* beta[3];   // NULL entry: beta = 0
    const uint16_t* W;         // [3d, d] (stored layout)
    const uint16_t* bias;      // [d] or NULL
    uint16_t* out;             // [M, d] (rows at rv.ld_out)
    RowView rv;
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
    int one = 0;  // 1: one token, the VALU kernel (nb groups of 64 columns x kps K chunks)
    size_t counters_bytes = 0, stats_bytes = 0, part_bytes = 0;
    size_t total() const { return counters_bytes + stats_bytes + part_bytes; }
};

constexpr int DECODE_MAX_M = 64;
constexpr int GEMVN_MAX_M = 128;  // the folded column-split kernel takes up to 8 token tiles
DecodePlan plan_decode(int M, int d, int norm);
hipError_t launch_decode(const DecodeArgs& a, int norm, const DecodePlan& p, hipStream_t st);

// ------------------------------------------------------- folded weight tiles
// The folded weight W' (3d x d, W'[k][n] = bf16(gamma_s[k - s d] W[k][n]))
// is stored as 1 KiB tiles of 16 columns x 32 k in MFMA B-fragment order:
// tile (n / 16, k / 32) starts at element ((n / 16) * (3d / 32) + k / 32) * 512,
// and inside it element (n, k) sits at lane l = 16 * ((k % 32) / 8) + n % 16,
// position k % 8: offset 8 * l + k % 8.  A 16-column block is one contiguous
// run of 3d / 32 tiles along k.
__host__ __device__ inline size_t wtile_index(size_t n, size_t k, size_t d) {
    return ((n >> 4) * (3 * d / 32) + (k >> 5)) * 512 + ((((k & 31) >> 3) << 4) + (n & 15)) * 8 + (k & 7);
}

// Small-M path on the folded weight: workgroups of 64 or 128 columns x one K chunk
// (a piece of one state); the last workgroup of each column group reduces
// the chunks through the workspace.  Row statistics are reduced once per
// call and handed over as records stamped with the call id.
struct GemvArgs {
    const uint16_t* h[3];
    const uint16_t* wp;   // folded weight tiles
    const float* u;       // [3, d]
    const float* c;       // [d]
    uint16_t* out;        // [M, d] (rows at rv.ld_out)
    RowView rv;
    int M, d;
    float eps;
    int kps;              // K chunks per state (from the plan)
    int waves;            // waves per workgroup (from the plan)
    int* counters;        // [column groups], zero on entry, left zero on exit
    float* part;          // [column groups * 3 kps * 16 MT * 16 nb]
    uint64_t* rstats;     // [3 M][4]: K, S1, S2 per (state, token) row, each (value bits | call id << 32)
    uint32_t call_id;     // nonzero, different from the previous calls' on this workspace
    int stats_recompute;  // nonzero: readers recompute the statistics instead of waiting for the records
    int nch;              // column-split kernel: K chunks (from the plan)
};

struct GemvPlan {
    int kps = 0, ring = 0, waves = 0, nb = 4, MT = 1, grid = 0;  // nb: 16-column blocks per workgroup
    int whole = 0;  // 1: few tokens, the whole-K kernel (one 16-column block per workgroup, no split)
    int cols = 0;   // 1: the column-split kernel (a 16-column block per wave, nch K chunks)
    int pack = 0;   // 1: few tokens, the packed-block whole-K kernel; sb: its k-steps per packed block
    int nch = 0, sb = 0;
    size_t counters_bytes = 0, part_bytes = 0;
    static constexpr size_t rstats_bytes = 3 * GEMVN_MAX_M * 4 * sizeof(uint64_t);
};

GemvPlan plan_gemv(int M, int d, int norm);
hipError_t launch_gemv(const GemvArgs& a, int norm, const GemvPlan& p, hipStream_t st);

// -------------------------------------------------------------- fold prepare
// counters: [d / 64] zero on entry, left zero; cpart: [3, d] float32 scratch
hipError_t launch_fold_prepare(int d, int norm, const uint16_t* const gamma[3], const uint16_t* const beta[3],
                               const uint16_t* W, const uint16_t* bias, uint16_t* wt, float* u, float* c,
                               int* counters, float* cpart, hipStream_t st);

// ------------------------------------------------------------------ prefill
// Large-M path: GEMM on raw hidden states and the folded weight tiles,
// per-row rescale at the state boundaries (fold), optional split-K (the
// chunks' partials are summed by a reduction kernel launched after it).
struct PrefillArgs {
    const uint16_t* h[3];
    const uint16_t* wt;   // folded weight tiles
    const float* u;       // [3, d]
    const float* c;       // [d]
    const float* mu;      // [3, M]
    const float* rstd;    // [3, M]
    uint16_t* out;        // [M, d] (rows at rv.ld_out)
    RowView rv;
    int M, d;
    int norm;
    int splits;           // partial slots per tile: 1 (no split) or 3 x (parts per state)
    int chunks;           // K chunks (workgroups) per tile: splits, or 4 chunks that cross the states
    float* part;          // split-K partials (summed by a second kernel)
};

struct PrefillPlan {
    int splits = 1, chunks = 1;
    int tiles_m = 0, tiles_n = 0;
    size_t part_bytes = 0;
};

PrefillPlan plan_prefill(int M, int d);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st);

// ------------------------------------------------------------ verify / accept
constexpr int VERIFY_MAX_N = 64;  // drafts per sequence (one wave decides them)
constexpr long long VERIFY_TARGET_WGS = 256;  // chunk size grows (up to 8192 tokens) past one workgroup per CU
struct VerifyArgs {
    const float* p;        // [B, N, V]
    const float* q;        // [B, N + 1, V]
    const int32_t* draft;  // [B, N]
    const float* u_acc;    // [B, N]
    const float* u_res;    // [B]
    int B, N, V;
    int C, L;              // chunks per sequence, tokens per chunk (from the plan)
    int32_t* n_acc;        // [B]
    int32_t* next;         // [B]
    int* counters;         // [B], zero on entry, left zero
    uint64_t* rec;         // [B][C][8]: exact digit sums and flags of each chunk
};
struct VerifyPlan {
    int ok = 0, C = 0, L = 0;
    size_t rec_bytes = 0;
};
VerifyPlan plan_verify(int B, int N, int V);
hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, bool vec, hipStream_t st);

// zero-fill helper (a kernel, not hipMemsetAsync)
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace e31
