// C ABI of the fused per-state norm + FC (declared in include/eagle31.h).
//
// Every argument check runs on the host before the first HIP call; a failed
// check enqueues nothing.  Dispatch: M <= 64 runs a single-launch decode
// kernel, on W in its stored layout or on the folded weight tiles (split-K,
// statistics inside the launch; one token on the folded tiles: the whole-K
// kernel).  Larger M runs the row-statistics pass and the folded GEMM,
// preparing W', u and c into the workspace first when the caller passed the
// stored W.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/eagle31.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

using namespace e31;

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return EAGLE31_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};

bool overlaps(const void* p, size_t bytes, const void* q, size_t qbytes) {
    if (p == nullptr || q == nullptr || bytes == 0 || qbytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + bytes, b0 = (uintptr_t)q, b1 = b0 + qbytes;
    return a0 < b1 && b0 < a1;
}

constexpr int64_t MAX_M = 16777216;
constexpr int64_t MAX_D = 65536;
constexpr int64_t VERIFY_MAX_V = 1 << 26;  // vocabulary size, at most

int check_common(int64_t M, int64_t d, int norm_kind, float eps) {
    if (M < 0 || M > MAX_M || d <= 0 || d > MAX_D || (d % 64) != 0) return EAGLE31_ERR_SHAPE;
    if (norm_kind != EAGLE31_NORM_NONE && norm_kind != EAGLE31_NORM_LAYERNORM && norm_kind != EAGLE31_NORM_RMSNORM)
        return EAGLE31_ERR_NORM_KIND;
    if (!std::isfinite(eps) || eps < 0.f) return EAGLE31_ERR_EPS;
    return EAGLE31_OK;
}

int check_params(int64_t d, int norm_kind, const void* const* gamma, const void* const* beta) {
    if (norm_kind != EAGLE31_NORM_NONE && gamma != nullptr)
        for (int s = 0; s < 3; ++s)
            if (gamma[s] != nullptr && !aligned16(gamma[s])) return EAGLE31_ERR_ALIGN;
    if (norm_kind == EAGLE31_NORM_LAYERNORM && beta != nullptr)
        for (int s = 0; s < 3; ++s)
            if (beta[s] != nullptr && !aligned16(beta[s])) return EAGLE31_ERR_ALIGN;
    (void)d;
    return EAGLE31_OK;
}

// Where a call's rows are (see RowView), with the byte extents the alias
// checks use: state s spans ((n_src - 1) ld_s + d) elements from h_s, the
// output ((M - 1) ld_out + d) from out.
struct Rows {
    const void* h[3] = {nullptr, nullptr, nullptr};
    RowView rv;
    size_t hext[3] = {0, 0, 0}, oext = 0, iext = 0;
};
constexpr int64_t MAX_LD = (int64_t)1 << 22;  // elements between rows, at most

int check_rows(int64_t M, int64_t d, const void* h0, const void* h1, const void* h2, const int64_t* ld,
               const int32_t* row_index, int64_t n_src, const void* out, int64_t ld_out, Rows& R) {
    if (M == 0) return EAGLE31_OK;
    if (h0 == nullptr || h1 == nullptr || h2 == nullptr || out == nullptr) return EAGLE31_ERR_NULL;
    const void* h[3] = {h0, h1, h2};
    for (int s = 0; s < 3; ++s) {
        const int64_t l = ld ? ld[s] : d;
        if (l < d || l > MAX_LD || (l % 8) != 0) return EAGLE31_ERR_SHAPE;
        R.h[s] = h[s];
        R.rv.ld[s] = l;
    }
    if (ld_out < d || ld_out > MAX_LD || (ld_out % 8) != 0) return EAGLE31_ERR_SHAPE;
    if (n_src < 1 || n_src > INT32_MAX || (row_index == nullptr && n_src < M)) return EAGLE31_ERR_SHAPE;
    // an index reaches any row: its byte offset in a state buffer stays below 2^32
    if (row_index != nullptr)
        for (int s = 0; s < 3; ++s)
            if ((uint64_t)n_src * (uint64_t)R.rv.ld[s] * 2 > ((uint64_t)1 << 32)) return EAGLE31_ERR_SHAPE;
    if (!aligned16(h0) || !aligned16(h1) || !aligned16(h2) || !aligned16(out) || ((uintptr_t)row_index & 3u) != 0)
        return EAGLE31_ERR_ALIGN;
    R.rv.ld_out = ld_out;
    R.rv.idx = row_index;
    R.rv.n_src = (int)n_src;
    for (int s = 0; s < 3; ++s) R.hext[s] = (size_t)((n_src - 1) * R.rv.ld[s] + d) * 2;
    R.oext = (size_t)((M - 1) * ld_out + d) * 2;
    R.iext = row_index ? (size_t)M * 4 : 0;
    for (int s = 0; s < 3; ++s)
        if (overlaps(out, R.oext, h[s], R.hext[s])) return EAGLE31_ERR_ALIAS;
    if (overlaps(out, R.oext, row_index, R.iext)) return EAGLE31_ERR_ALIAS;
    return EAGLE31_OK;
}

int check_io(int64_t M, int64_t d, const void* h0, const void* h1, const void* h2, const void* out, Rows& R) {
    return check_rows(M, d, h0, h1, h2, nullptr, nullptr, M > 0 ? M : 1, out, d, R);
}

// ------------------------------------------------------------- workspace
struct WsLayout {
    size_t counters = 0, counters_bytes = 0;
    size_t stats = 0, part = 0, mu = 0, rstd = 0, wt = 0, u = 0, c = 0, cpart = 0;
    size_t total = 0;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// The workspace starts with a fixed region of synchronisation counters that
// every call leaves at zero, whatever path (and so whatever layout of the
// rest) the previous call used.
constexpr size_t COUNTER_REGION = 16384;  // 4096 counters
constexpr int MAX_COUNTERS = (int)(COUNTER_REGION / sizeof(int));
// The folded path takes the decode kernels up to 64 tokens, and the
// column-split decode kernel up to 128 where its plan exists; more tokens
// take the prefill kernel.
bool folded_decode(int64_t M, int64_t d, int norm) {
    if (M <= DECODE_MAX_M) return true;
    return M <= GEMVN_MAX_M && plan_gemv((int)M, (int)d, norm).cols != 0;
}

WsLayout layout_for(int64_t M, int64_t d, int norm, bool folded) {
    WsLayout L;
    if (M <= 0) return L;
    L.counters = 0;
    L.counters_bytes = COUNTER_REGION;
    size_t off = COUNTER_REGION;
    if (folded && folded_decode(M, d, norm)) {
        const GemvPlan p = plan_gemv((int)M, (int)d, norm);
        L.stats = off;
        off += up256(GemvPlan::rstats_bytes);
        L.part = off;
        off += up256(p.part_bytes);
        L.total = off;
        return L;
    }
    if (M <= DECODE_MAX_M) {
        const DecodePlan p = plan_decode((int)M, (int)d, norm);
        L.stats = off;
        off += up256(p.stats_bytes);
        L.part = off;
        off += up256(p.part_bytes);
        L.total = off;
        return L;
    }
    const PrefillPlan p = plan_prefill((int)M, (int)d);
    L.part = off;
    off += up256(p.part_bytes);
    L.mu = off;
    off += up256((size_t)3 * M * sizeof(float));
    L.rstd = off;
    off += up256((size_t)3 * M * sizeof(float));
    if (!folded) {
        L.wt = off;
        off += up256((size_t)3 * d * d * 2);
        L.u = off;
        off += up256((size_t)3 * d * sizeof(float));
        L.c = off;
        off += up256((size_t)d * sizeof(float));
        L.cpart = off;
        off += up256((size_t)3 * d * sizeof(float));
    }
    L.total = off;
    return L;
}

// Library-owned workspace: one buffer per (device, stream), grown on demand.
// Counters are zeroed on allocation; every call leaves them at zero.
struct OwnedWs {
    void* ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
// Test hook (eagle31_debug_fail_workspace_zero): the counter zeroing of a new
// library-owned workspace reports a launch failure instead of running.
std::atomic<int> g_zero_hook{0};
std::map<std::pair<int, void*>, OwnedWs> g_ws;

int owned_workspace(size_t need, hipStream_t st, void** out_ptr, size_t* out_bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    OwnedWs& w = g_ws[std::make_pair(dev, (void*)st)];
    if (w.bytes < need) {
        if (w.ptr != nullptr) {
            // work queued earlier may still use the old buffer
            e = hipStreamSynchronize(st);
            if (e != hipSuccess) return hip_fail(e);
            e = hipFree(w.ptr);
            if (e != hipSuccess) return hip_fail(e);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        size_t grow = need + need / 4;
        grow = up256(grow);
        void* fresh = nullptr;
        e = hipMalloc(&fresh, grow);
        if (e != hipSuccess) return hip_fail(e);
        // the buffer is kept only once its counters are zeroed: a buffer whose
        // zeroing failed to launch is freed, so no later call can find it
        e = g_zero_hook ? hipErrorLaunchFailure : launch_zero(fresh, COUNTER_REGION, st);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(st);
            (void)hipFree(fresh);
            return hip_fail(e);
        }
        w.ptr = fresh;
        w.bytes = grow;
    }
    *out_ptr = w.ptr;
    *out_bytes = w.bytes;
    return EAGLE31_OK;
}

// ------------------------------------------- fixed scratch of the no-alloc entry
// eagle31_fuse_folded_noalloc runs on this array instead of allocated
// workspace.  Each device holds its own copy (for as long as the library is
// loaded).  In host code its name is only a stand-in: the device address is
// taken once per device with hipGetSymbolAddress, and only that address is
// passed to kernels or zeroed.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// The device address of the current device's scratch.  On the first call on
// a device it is looked up and the counter region (which every call leaves at
// zero) is zeroed by a kernel on `st`.
int noalloc_scratch(hipStream_t st, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hip_fail(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hip_fail(hipErrorInvalidSymbol);
        e = launch_zero(p, COUNTER_REGION, st);
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return EAGLE31_OK;
}

// Id stamped on the statistics records of one decode call: process-wide,
// never 0 (a zeroed workspace holds no valid record), so a record left by an
// earlier call on the same workspace never matches.
// Set by eagle31_debug_stats_recompute: the folded decode kernel's readers
// take their fallback path (recompute the statistics rows) at once.
std::atomic<int> g_stats_recompute{0};

uint32_t next_call_id() {
    static std::atomic<uint32_t> counter{0};
    uint32_t id;
    do {
        id = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (id == 0);
    return id;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// ------------------------------------------------------------- dispatch
int run_fuse(const Rows& R, int64_t M, int64_t d, int norm, float eps, const void* const* gamma,
             const void* const* beta, const void* W, const void* bias, const void* wt, const float* u, const float* c,
             bool folded, void* out, void* ws, size_t ws_bytes, hipStream_t st) {
    const WsLayout L = layout_for(M, d, norm, folded);
    if (ws_bytes < L.total) return EAGLE31_ERR_WORKSPACE;
    const uint16_t* h[3] = {static_cast<const uint16_t*>(R.h[0]), static_cast<const uint16_t*>(R.h[1]),
                            static_cast<const uint16_t*>(R.h[2])};
    const uint16_t* g[3] = {nullptr, nullptr, nullptr};
    const uint16_t* b[3] = {nullptr, nullptr, nullptr};
    if (!folded && norm != NORM_NONE && gamma != nullptr)
        for (int s = 0; s < 3; ++s) g[s] = static_cast<const uint16_t*>(gamma[s]);
    if (!folded && norm == NORM_LN && beta != nullptr)
        for (int s = 0; s < 3; ++s) b[s] = static_cast<const uint16_t*>(beta[s]);

    hipError_t e;
    if (folded && folded_decode(M, d, norm)) {
        const GemvPlan p = plan_gemv((int)M, (int)d, norm);
        if (p.waves == 0 || d / (16 * p.nb) > MAX_COUNTERS) return EAGLE31_ERR_SHAPE;
        GemvArgs a;
        for (int s = 0; s < 3; ++s) a.h[s] = h[s];
        a.wp = static_cast<const uint16_t*>(wt);
        a.u = u;
        a.c = c;
        a.out = static_cast<uint16_t*>(out);
        a.rv = R.rv;
        a.M = (int)M;
        a.d = (int)d;
        a.eps = eps;
        a.kps = p.kps;
        a.waves = p.waves;
        a.counters = at<int>(ws, L.counters);
        a.part = at<float>(ws, L.part);
        a.rstats = at<uint64_t>(ws, L.stats);
        a.call_id = next_call_id();
        a.stats_recompute = g_stats_recompute.load(std::memory_order_relaxed);
        a.nch = p.nch;
        e = launch_gemv(a, norm, p, st);
        if (e != hipSuccess) return hip_fail(e);
        return EAGLE31_OK;
    }
    if (M <= DECODE_MAX_M) {
        const DecodePlan p = plan_decode((int)M, (int)d, norm);
        if (p.nb > MAX_COUNTERS) return EAGLE31_ERR_SHAPE;
        DecodeArgs a;
        for (int s = 0; s < 3; ++s) {
            a.h[s] = h[s];
            a.gamma[s] = g[s];
            a.beta[s] = b[s];
        }
        a.W = static_cast<const uint16_t*>(W);
        a.bias = static_cast<const uint16_t*>(bias);
        a.out = static_cast<uint16_t*>(out);
        a.rv = R.rv;
        a.M = (int)M;
        a.d = (int)d;
        a.eps = eps;
        a.nb = p.nb;
        a.kps = p.kps;
        a.counters = at<int>(ws, L.counters);
        a.stats = at<float>(ws, L.stats);
        a.part = at<float>(ws, L.part);
        e = launch_decode(a, norm, p, st);
        if (e != hipSuccess) return hip_fail(e);
        return EAGLE31_OK;
    }

    // prefill: statistics, (fold the stored W), GEMM
    const PrefillPlan p = plan_prefill((int)M, (int)d);
    float* mu = at<float>(ws, L.mu);
    float* rstd = at<float>(ws, L.rstd);
    if (norm != NORM_NONE) {
        e = launch_row_stats(h[0], h[1], h[2], R.rv, (int)M, (int)d, norm, eps, mu, rstd, st);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (!folded) {
        uint16_t* wtw = at<uint16_t>(ws, L.wt);
        float* uw = at<float>(ws, L.u);
        float* cw = at<float>(ws, L.c);
        e = launch_fold_prepare((int)d, norm, g, b, static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(bias),
                                wtw, uw, cw, at<int>(ws, L.counters), at<float>(ws, L.cpart), st);
        if (e != hipSuccess) return hip_fail(e);
        wt = wtw;
        u = uw;
        c = cw;
    }
    PrefillArgs a;
    for (int s = 0; s < 3; ++s) a.h[s] = h[s];
    a.wt = static_cast<const uint16_t*>(wt);
    a.u = u;
    a.c = c;
    a.mu = mu;
    a.rstd = rstd;
    a.out = static_cast<uint16_t*>(out);
    a.rv = R.rv;
    a.M = (int)M;
    a.d = (int)d;
    a.norm = norm;
    a.splits = p.splits;
    a.chunks = p.chunks;
    a.part = at<float>(ws, L.part);
    e = launch_prefill(a, p, st);
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

// The rows are checked by the caller (check_io or check_rows) after
// check_common; these check the rest.
int validate_fuse_params(const Rows& R, int64_t M, int64_t d, int norm, const void* const* gamma,
                         const void* const* beta, const void* W, const void* bias, void* out) {
    if (W == nullptr) return EAGLE31_ERR_NULL;
    if (!aligned16(W) || (bias != nullptr && !aligned16(bias))) return EAGLE31_ERR_ALIGN;
    int r = check_params(d, norm, gamma, beta);
    if (r != EAGLE31_OK) return r;
    if (M > 0) {
        const size_t ob = R.oext;
        if (overlaps(out, ob, W, (size_t)3 * d * d * 2) || overlaps(out, ob, bias, (size_t)d * 2)) return EAGLE31_ERR_ALIAS;
        for (int s = 0; s < 3; ++s) {
            if (gamma != nullptr && overlaps(out, ob, gamma[s], (size_t)d * 2)) return EAGLE31_ERR_ALIAS;
            if (beta != nullptr && overlaps(out, ob, beta[s], (size_t)d * 2)) return EAGLE31_ERR_ALIAS;
        }
    }
    return EAGLE31_OK;
}

int validate_folded_params(const Rows& R, int64_t M, int64_t d, const void* wt, const float* u, const float* c,
                           void* out) {
    if (wt == nullptr || u == nullptr || c == nullptr) return EAGLE31_ERR_NULL;
    if (!aligned16(wt) || !aligned16(u) || !aligned16(c)) return EAGLE31_ERR_ALIGN;
    if (M > 0) {
        const size_t ob = R.oext;
        if (overlaps(out, ob, wt, (size_t)3 * d * d * 2) || overlaps(out, ob, u, (size_t)3 * d * 4) ||
            overlaps(out, ob, c, (size_t)d * 4))
            return EAGLE31_ERR_ALIAS;
    }
    return EAGLE31_OK;
}

// check_common, the rows (dense: contiguous [M, d] rows, else the row view
// arguments), then the weight-side arguments
int prep_fuse(bool dense, const void* h0, const void* h1, const void* h2, const int64_t* ld, const int32_t* idx,
              int64_t n_src, int64_t M, int64_t d, int norm, float eps, const void* const* gamma,
              const void* const* beta, const void* W, const void* bias, void* out, int64_t ld_out, Rows& R) {
    int r = check_common(M, d, norm, eps);
    if (r != EAGLE31_OK) return r;
    r = dense ? check_io(M, d, h0, h1, h2, out, R) : check_rows(M, d, h0, h1, h2, ld, idx, n_src, out, ld_out, R);
    if (r != EAGLE31_OK) return r;
    return validate_fuse_params(R, M, d, norm, gamma, beta, W, bias, out);
}

int prep_folded(bool dense, const void* h0, const void* h1, const void* h2, const int64_t* ld, const int32_t* idx,
                int64_t n_src, int64_t M, int64_t d, int norm, float eps, const void* wt, const float* u,
                const float* c, void* out, int64_t ld_out, Rows& R) {
    int r = check_common(M, d, norm, eps);
    if (r != EAGLE31_OK) return r;
    r = dense ? check_io(M, d, h0, h1, h2, out, R) : check_rows(M, d, h0, h1, h2, ld, idx, n_src, out, ld_out, R);
    if (r != EAGLE31_OK) return r;
    return validate_folded_params(R, M, d, wt, u, c, out);
}

}  // namespace

extern "C" {

int eagle31_fuse(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d, int norm_kind,
                 float eps, const void* const* gamma, const void* const* beta, const void* W, const void* bias,
                 void* out, void* stream) {
    Rows R;
    int r = prep_fuse(true, h_low, h_mid, h_high, nullptr, nullptr, 0, M, d, norm_kind, eps, gamma, beta, W, bias,
                      out, d, R);
    if (r != EAGLE31_OK || M == 0) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    r = owned_workspace(layout_for(M, d, norm_kind, false).total, st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    return run_fuse(R, M, d, norm_kind, eps, gamma, beta, W, bias, nullptr, nullptr, nullptr, false, out, ws, wsb, st);
}

int eagle31_fuse_rows(const void* h_low, const void* h_mid, const void* h_high, const int64_t* ld,
                      const int32_t* row_index, int64_t n_src, int64_t M, int64_t d, int norm_kind, float eps,
                      const void* const* gamma, const void* const* beta, const void* W, const void* bias, void* out,
                      int64_t ld_out, void* stream) {
    Rows R;
    int r = prep_fuse(false, h_low, h_mid, h_high, ld, row_index, n_src, M, d, norm_kind, eps, gamma, beta, W, bias,
                      out, ld_out, R);
    if (r != EAGLE31_OK || M == 0) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    r = owned_workspace(layout_for(M, d, norm_kind, false).total, st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    return run_fuse(R, M, d, norm_kind, eps, gamma, beta, W, bias, nullptr, nullptr, nullptr, false, out, ws, wsb, st);
}

size_t eagle31_workspace_size(int64_t M, int64_t d, int norm_kind) {
    if (check_common(M, d, norm_kind, 0.f) != EAGLE31_OK) return 0;
    const WsLayout a = layout_for(M, d, norm_kind, false);
    const WsLayout b = layout_for(M, d, norm_kind, true);
    return a.total > b.total ? a.total : b.total;
}

int eagle31_debug_fail_workspace_zero(int on) {
    g_zero_hook.store(on ? 1 : 0, std::memory_order_relaxed);
    return EAGLE31_OK;
}

int eagle31_debug_stats_recompute(int on) {
    g_stats_recompute.store(on ? 1 : 0, std::memory_order_relaxed);
    return EAGLE31_OK;
}

int eagle31_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
    if (workspace == nullptr) return EAGLE31_ERR_NULL;
    if (((uintptr_t)workspace & 255u) != 0) return EAGLE31_ERR_ALIGN;
    if (ws_bytes < COUNTER_REGION) return EAGLE31_ERR_WORKSPACE;
    const hipError_t e = launch_zero(workspace, COUNTER_REGION, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_fuse_ws(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d, int norm_kind,
                    float eps, const void* const* gamma, const void* const* beta, const void* W, const void* bias,
                    void* out, void* workspace, size_t ws_bytes, void* stream) {
    Rows R;
    int r = prep_fuse(true, h_low, h_mid, h_high, nullptr, nullptr, 0, M, d, norm_kind, eps, gamma, beta, W, bias,
                      out, d, R);
    if (r != EAGLE31_OK || M == 0) return r;
    if (workspace == nullptr) return EAGLE31_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return EAGLE31_ERR_ALIGN;
    if (ws_bytes < layout_for(M, d, norm_kind, false).total) return EAGLE31_ERR_WORKSPACE;
    return run_fuse(R, M, d, norm_kind, eps, gamma, beta, W, bias, nullptr, nullptr, nullptr, false, out, workspace,
                    ws_bytes, static_cast<hipStream_t>(stream));
}

int eagle31_fold_prepare(int64_t d, int norm_kind, const void* const* gamma, const void* const* beta, const void* W,
                         const void* bias, void* w_folded, float* u, float* c, void* stream) {
    int r = check_common(0, d, norm_kind, 0.f);
    if (r != EAGLE31_OK) return r;
    if (W == nullptr || w_folded == nullptr || u == nullptr || c == nullptr) return EAGLE31_ERR_NULL;
    if (!aligned16(W) || !aligned16(w_folded) || !aligned16(u) || !aligned16(c) ||
        (bias != nullptr && !aligned16(bias)))
        return EAGLE31_ERR_ALIGN;
    r = check_params(d, norm_kind, gamma, beta);
    if (r != EAGLE31_OK) return r;
    const size_t wb = (size_t)3 * d * d * 2;
    if (overlaps(w_folded, wb, W, wb) || overlaps(u, (size_t)3 * d * 4, W, wb) || overlaps(c, (size_t)d * 4, W, wb) ||
        overlaps(u, (size_t)3 * d * 4, w_folded, wb) || overlaps(c, (size_t)d * 4, w_folded, wb) ||
        overlaps(c, (size_t)d * 4, u, (size_t)3 * d * 4))
        return EAGLE31_ERR_ALIAS;
    const uint16_t* g[3] = {nullptr, nullptr, nullptr};
    const uint16_t* b[3] = {nullptr, nullptr, nullptr};
    if (norm_kind != NORM_NONE && gamma != nullptr)
        for (int s = 0; s < 3; ++s) g[s] = static_cast<const uint16_t*>(gamma[s]);
    if (norm_kind == NORM_LN && beta != nullptr)
        for (int s = 0; s < 3; ++s) b[s] = static_cast<const uint16_t*>(beta[s]);
    // scratch: the strips' counters and the per-state partials of c
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    r = owned_workspace(COUNTER_REGION + up256((size_t)3 * d * sizeof(float)), st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    const hipError_t e = launch_fold_prepare((int)d, norm_kind, g, b, static_cast<const uint16_t*>(W),
                                             static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(w_folded), u,
                                             c, at<int>(ws, 0), at<float>(ws, COUNTER_REGION), st);
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_fuse_folded(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d, int norm_kind,
                        float eps, const void* w_folded, const float* u, const float* c, void* out, void* stream) {
    Rows R;
    int r = prep_folded(true, h_low, h_mid, h_high, nullptr, nullptr, 0, M, d, norm_kind, eps, w_folded, u, c, out, d,
                        R);
    if (r != EAGLE31_OK || M == 0) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    r = owned_workspace(layout_for(M, d, norm_kind, true).total, st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    return run_fuse(R, M, d, norm_kind, eps, nullptr, nullptr, nullptr, nullptr, w_folded, u, c, true, out, ws, wsb,
                    st);
}

int eagle31_fuse_folded_rows(const void* h_low, const void* h_mid, const void* h_high, const int64_t* ld,
                             const int32_t* row_index, int64_t n_src, int64_t M, int64_t d, int norm_kind, float eps,
                             const void* w_folded, const float* u, const float* c, void* out, int64_t ld_out,
                             void* stream) {
    Rows R;
    int r = prep_folded(false, h_low, h_mid, h_high, ld, row_index, n_src, M, d, norm_kind, eps, w_folded, u, c, out,
                        ld_out, R);
    if (r != EAGLE31_OK || M == 0) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    r = owned_workspace(layout_for(M, d, norm_kind, true).total, st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    return run_fuse(R, M, d, norm_kind, eps, nullptr, nullptr, nullptr, nullptr, w_folded, u, c, true, out, ws, wsb,
                    st);
}

int eagle31_fuse_folded_ws(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                           int norm_kind, float eps, const void* w_folded, const float* u, const float* c, void* out,
                           void* workspace, size_t ws_bytes, void* stream) {
    Rows R;
    int r = prep_folded(true, h_low, h_mid, h_high, nullptr, nullptr, 0, M, d, norm_kind, eps, w_folded, u, c, out, d,
                        R);
    if (r != EAGLE31_OK || M == 0) return r;
    if (workspace == nullptr) return EAGLE31_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return EAGLE31_ERR_ALIGN;
    if (ws_bytes < layout_for(M, d, norm_kind, true).total) return EAGLE31_ERR_WORKSPACE;
    return run_fuse(R, M, d, norm_kind, eps, nullptr, nullptr, nullptr, nullptr, w_folded, u, c, true, out, workspace,
                    ws_bytes, static_cast<hipStream_t>(stream));
}

int eagle31_fuse_folded_noalloc(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                                int norm_kind, float eps, const void* w_folded, const float* u, const float* c,
                                void* out, void* stream) {
    Rows R;
    int r = prep_folded(true, h_low, h_mid, h_high, nullptr, nullptr, 0, M, d, norm_kind, eps, w_folded, u, c, out, d,
                        R);
    if (r != EAGLE31_OK || M == 0) return r;
    const size_t need = layout_for(M, d, norm_kind, true).total;
    if (need > NOALLOC_SCRATCH_BYTES) return EAGLE31_ERR_TOO_LARGE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    r = noalloc_scratch(st, &ws);
    if (r != EAGLE31_OK) return r;
    return run_fuse(R, M, d, norm_kind, eps, nullptr, nullptr, nullptr, nullptr, w_folded, u, c, true, out, ws,
                    NOALLOC_SCRATCH_BYTES, st);
}

size_t eagle31_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int eagle31_row_stats(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d, int norm_kind,
                      float eps, float* mu, float* rstd, void* stream) {
    int r = check_common(M, d, norm_kind, eps);
    if (r != EAGLE31_OK || M == 0) return r;
    if (h_low == nullptr || h_mid == nullptr || h_high == nullptr || mu == nullptr || rstd == nullptr)
        return EAGLE31_ERR_NULL;
    if (!aligned16(h_low) || !aligned16(h_mid) || !aligned16(h_high) || !aligned16(mu) || !aligned16(rstd))
        return EAGLE31_ERR_ALIGN;
    const hipError_t e = launch_row_stats(static_cast<const uint16_t*>(h_low), static_cast<const uint16_t*>(h_mid),
                                          static_cast<const uint16_t*>(h_high), dense_rows((int)M, (int)d), (int)M,
                                          (int)d, norm_kind, eps, mu, rstd, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_norm_output(const void* x, int64_t M, int64_t d, int norm_kind, float eps, const void* gamma,
                        const void* beta, void* out, void* stream) {
    int r = check_common(M, d, norm_kind, eps);
    if (r != EAGLE31_OK) return r;
    if (d > NORM_ROWS_MAX_D) return EAGLE31_ERR_SHAPE;
    if (M == 0) return EAGLE31_OK;
    if (x == nullptr || out == nullptr) return EAGLE31_ERR_NULL;
    const bool use_g = norm_kind != EAGLE31_NORM_NONE && gamma != nullptr;
    const bool use_b = norm_kind == EAGLE31_NORM_LAYERNORM && beta != nullptr;
    if (!aligned16(x) || !aligned16(out) || (use_g && !aligned16(gamma)) || (use_b && !aligned16(beta)))
        return EAGLE31_ERR_ALIGN;
    // out == x is the in-place form; any other overlap is refused
    const size_t rb = (size_t)M * (size_t)d * 2;
    if ((out != x && overlaps(out, rb, x, rb)) || (use_g && overlaps(out, rb, gamma, (size_t)d * 2)) ||
        (use_b && overlaps(out, rb, beta, (size_t)d * 2)))
        return EAGLE31_ERR_ALIAS;
    const hipError_t e = launch_norm_rows(static_cast<const uint16_t*>(x), (int)M, (int)d, norm_kind, eps,
                                          use_g ? static_cast<const uint16_t*>(gamma) : nullptr,
                                          use_b ? static_cast<const uint16_t*>(beta) : nullptr,
                                          static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_embed_concat(const int32_t* tokens, int64_t M, int64_t d, int64_t vocab, const void* embed,
                         const void* fused, void* dst, int32_t* bad_count, void* stream) {
    if (M < 0 || M > MAX_M || d <= 0 || d > EMBED_CONCAT_MAX_D || (d % 64) != 0 || vocab < 1 || vocab > INT32_MAX)
        return EAGLE31_ERR_SHAPE;
    if (M == 0) return EAGLE31_OK;
    if (tokens == nullptr || embed == nullptr || dst == nullptr) return EAGLE31_ERR_NULL;
    if (!aligned16(embed) || (fused != nullptr && !aligned16(fused)) || !aligned16(dst) || ((uintptr_t)tokens & 3u) != 0 ||
        ((uintptr_t)bad_count & 3u) != 0)
        return EAGLE31_ERR_ALIGN;
    const size_t db = (size_t)M * (size_t)d * 4, rb = (size_t)M * (size_t)d * 2;
    if (overlaps(dst, db, tokens, (size_t)M * 4) || overlaps(dst, db, embed, (size_t)vocab * (size_t)d * 2) ||
        overlaps(dst, db, fused, rb) || overlaps(dst, db, bad_count, 4))
        return EAGLE31_ERR_ALIAS;
    const hipError_t e = launch_embed_concat(tokens, (int)M, (int)d, (int)vocab, static_cast<const uint16_t*>(embed),
                                             static_cast<const uint16_t*>(fused), static_cast<uint16_t*>(dst),
                                             bad_count, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_verify_accept(const float* p, const float* q, const int32_t* draft, const float* u_acc,
                          const float* u_res, int64_t B, int64_t N, int64_t V, int32_t* n_accepted,
                          int32_t* next_token, void* stream) {
    if (B < 0 || B > MAX_COUNTERS || N < 1 || N > VERIFY_MAX_N || V < 1 || V > VERIFY_MAX_V) return EAGLE31_ERR_SHAPE;
    if (B == 0) return EAGLE31_OK;
    if (p == nullptr || q == nullptr || draft == nullptr || u_acc == nullptr || u_res == nullptr ||
        n_accepted == nullptr || next_token == nullptr)
        return EAGLE31_ERR_NULL;
    const void* in4[5] = {p, q, draft, u_acc, u_res};
    for (const void* x : in4)
        if (((uintptr_t)x & 3u) != 0) return EAGLE31_ERR_ALIGN;
    if (((uintptr_t)n_accepted & 3u) != 0 || ((uintptr_t)next_token & 3u) != 0) return EAGLE31_ERR_ALIGN;
    const size_t pb = (size_t)B * N * V * 4, qb = (size_t)B * (N + 1) * V * 4, nb = (size_t)B * N * 4,
                 ob = (size_t)B * 4;
    const void* outs[2] = {n_accepted, next_token};
    for (const void* o : outs)
        if (overlaps(o, ob, p, pb) || overlaps(o, ob, q, qb) || overlaps(o, ob, draft, nb) ||
            overlaps(o, ob, u_acc, nb) || overlaps(o, ob, u_res, ob))
            return EAGLE31_ERR_ALIAS;
    if (overlaps(n_accepted, ob, next_token, ob)) return EAGLE31_ERR_ALIAS;
    const VerifyPlan plan = plan_verify((int)B, (int)N, (int)V);
    if (!plan.ok) return EAGLE31_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    size_t wsb = 0;
    const int r = owned_workspace(COUNTER_REGION + up256(plan.rec_bytes), st, &ws, &wsb);
    if (r != EAGLE31_OK) return r;
    VerifyArgs a;
    a.p = p;
    a.q = q;
    a.draft = draft;
    a.u_acc = u_acc;
    a.u_res = u_res;
    a.B = (int)B;
    a.N = (int)N;
    a.V = (int)V;
    a.C = plan.C;
    a.L = plan.L;
    a.n_acc = n_accepted;
    a.next = next_token;
    a.counters = at<int>(ws, 0);
    a.rec = at<uint64_t>(ws, COUNTER_REGION);
    const bool vec = (V % 4) == 0 && ((uintptr_t)p & 15u) == 0 && ((uintptr_t)q & 15u) == 0;
    const hipError_t e = launch_verify(a, plan, vec, st);
    if (e != hipSuccess) return hip_fail(e);
    return EAGLE31_OK;
}

int eagle31_verify_chunking(int64_t B, int64_t N, int64_t V, int32_t* chunks, int32_t* tokens_per_chunk) {
    if (B < 1 || B > MAX_COUNTERS || N < 1 || N > VERIFY_MAX_N || V < 1 || V > VERIFY_MAX_V) return EAGLE31_ERR_SHAPE;
    if (chunks == nullptr || tokens_per_chunk == nullptr) return EAGLE31_ERR_NULL;
    const VerifyPlan plan = plan_verify((int)B, (int)N, (int)V);
    if (!plan.ok) return EAGLE31_ERR_SHAPE;
    *chunks = plan.C;
    *tokens_per_chunk = plan.L;
    return EAGLE31_OK;
}

const char* eagle31_status_string(int status) {
    switch (status) {
        case EAGLE31_OK: return "ok";
        case EAGLE31_ERR_NULL: return "a required pointer is NULL";
        case EAGLE31_ERR_SHAPE: return "M or d out of range (d must be a positive multiple of 64)";
        case EAGLE31_ERR_NORM_KIND: return "unknown norm_kind";
        case EAGLE31_ERR_EPS: return "eps must be finite and >= 0";
        case EAGLE31_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case EAGLE31_ERR_HIP: return "a HIP runtime call failed";
        case EAGLE31_ERR_WORKSPACE: return "workspace missing or too small";
        case EAGLE31_ERR_ALIAS: return "out overlaps an input";
        case EAGLE31_ERR_TOO_LARGE: return "the problem needs more scratch than the no-alloc entry point's fixed array";
        default: return "unknown status";
    }
}

int eagle31_last_hip_error(void) { return g_last_hip_error; }

int eagle31_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    int rc = EAGLE31_OK;
    for (auto& kv : g_ws) {
        if (kv.second.ptr == nullptr) continue;
        e = hipSetDevice(kv.first.first);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipFree(kv.second.ptr);
        if (e != hipSuccess) rc = hip_fail(e);
        kv.second.ptr = nullptr;
        kv.second.bytes = 0;
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
    return rc;
}

}  // extern "C"
