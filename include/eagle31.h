/*
 * eagle31.h - C ABI of the EAGLE-3.1 normalized multi-layer feature fusion
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (EAGLE 3.1 explainer, llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html,
 * sections "EAGLE-3의 다층 특성 융합 구조" and "FC 정규화: EAGLE 3.1의 핵심 수정"):
 * the target model's hidden states from an early, a middle and a late layer,
 * h_low, h_mid, h_high (each [M, d], one row per token), are each normalised on
 * their own, concatenated in that order to [M, 3d] and projected by the FC
 * layer W [3d, d] (+ bias) to the draft head's input [M, d]:
 *
 *     out = [norm_0(h_low) | norm_1(h_mid) | norm_2(h_high)] . W + bias
 *
 * norm_s is one of (per state s, with its own gamma_s / beta_s):
 *   EAGLE31_NORM_LAYERNORM  (x - mean) * (var + eps)^-1/2 * gamma_s + beta_s,
 *                           var = mean((x - mean)^2) (divide by d);
 *   EAGLE31_NORM_RMSNORM    x * (mean(x^2) + eps)^-1/2 * gamma_s   (the per-state
 *                           RMSNorm of the vLLM EAGLE 3.1 release post,
 *                           devlery.com/blog/vllm-eagle31-attention-drift, section
 *                           "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다");
 *   EAGLE31_NORM_NONE       identity: EAGLE-3's un-normalised fusion.
 *
 * Data types and layouts (all row-major, contiguous, no strides):
 *   hidden states, gamma, beta, W, bias, out: bfloat16;
 *   statistics and accumulation: float32; out is rounded to nearest even.
 *   W is [3d, d]: element (k, n) at k*d + n; rows [s*d, (s+1)*d) multiply state s.
 *
 * Conventions shared by every entry point:
 *   - pointers are device pointers on the calling thread's current HIP device,
 *     16-byte aligned; the caller owns every buffer.  Work is enqueued on
 *     `stream` (a hipStream_t passed as void*, NULL = default stream); the
 *     caller keeps buffers alive until the stream has reached the work.
 *   - arguments are checked on the host before any HIP call; a failed check
 *     returns its status and enqueues nothing.  M == 0 returns EAGLE31_OK
 *     without launching (h_* and out may then be NULL).
 *   - limits: 1 <= d, d % 64 == 0, d <= 65536; 0 <= M <= 16777216;
 *     eps finite and >= 0 (eps == 0 leaves constant rows undefined).
 *   - out must not overlap any input.
 *   - launch failures return EAGLE31_ERR_HIP (eagle31_last_hip_error() gives
 *     the HIP code); faults inside kernels surface when the stream is
 *     synchronised, as for any HIP work.  The library never prints or aborts.
 *   - results are deterministic: the same inputs give the same bits.
 */
#ifndef EAGLE31_H
#define EAGLE31_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum eagle31_norm_kind {
    EAGLE31_NORM_NONE = 0,
    EAGLE31_NORM_LAYERNORM = 1,
    EAGLE31_NORM_RMSNORM = 2
};

enum eagle31_status {
    EAGLE31_OK = 0,
    EAGLE31_ERR_NULL = -1,       /* a required pointer is NULL */
    EAGLE31_ERR_SHAPE = -2,      /* M or d out of range, d % 64 != 0 */
    EAGLE31_ERR_NORM_KIND = -3,  /* norm_kind not one of eagle31_norm_kind */
    EAGLE31_ERR_EPS = -4,        /* eps negative, NaN or infinite */
    EAGLE31_ERR_ALIGN = -5,      /* a pointer is not 16-byte aligned */
    EAGLE31_ERR_HIP = -6,        /* a HIP runtime call failed */
    EAGLE31_ERR_WORKSPACE = -7,  /* caller workspace NULL or too small */
    EAGLE31_ERR_ALIAS = -8,      /* out overlaps an input */
    EAGLE31_ERR_TOO_LARGE = -9   /* needs more scratch than eagle31_fuse_folded_noalloc has */
};

/*
 * eagle31_fuse - the fused step with library-owned scratch memory.
 *
 * gamma: array of 3 pointers (bf16 [d] each) or NULL; a NULL array or a NULL
 *        entry means gamma_s = 1.  Ignored for EAGLE31_NORM_NONE.
 * beta:  array of 3 pointers (bf16 [d] each) or NULL; NULL means beta_s = 0.
 *        Used by EAGLE31_NORM_LAYERNORM only.
 * bias:  bf16 [d] or NULL (no bias).
 * out:   bf16 [M, d].
 *
 * Scratch memory (split-K partials, the folded weight of the large-M path,
 * row statistics) is allocated by the library on first use per device and
 * grown when a larger problem needs it; it is freed by eagle31_release().
 * Allocation happens outside any kernel launch, so the first call at a new
 * size may return EAGLE31_ERR_HIP if the device is out of memory.  Calls
 * from several host threads are serialised on the scratch memory of a device.
 */
int eagle31_fuse(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                 int norm_kind, float eps, const void* const* gamma, const void* const* beta,
                 const void* W, const void* bias, void* out, void* stream);

/*
 * eagle31_workspace_size - bytes of caller workspace eagle31_fuse_ws needs for
 * (M, d, norm_kind).  Returns 0 for invalid arguments.
 */
size_t eagle31_workspace_size(int64_t M, int64_t d, int norm_kind);

/*
 * eagle31_workspace_init - zero the workspace's synchronisation counters.
 * Must be enqueued once on a new workspace before its first eagle31_fuse_ws /
 * eagle31_fuse_folded_ws call; every call leaves the counters at zero again.
 */
int eagle31_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/*
 * eagle31_fuse_ws - eagle31_fuse with caller-provided workspace of at least
 * eagle31_workspace_size(M, d, norm_kind) bytes (device memory, 256-byte
 * aligned, initialised once with eagle31_workspace_init).  Calls that share a
 * workspace must be ordered (same stream or synchronised).
 */
int eagle31_fuse_ws(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                    int norm_kind, float eps, const void* const* gamma, const void* const* beta,
                    const void* W, const void* bias, void* out, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * eagle31_fold_prepare - absorb the norm parameters into the FC once per
 * weight set (EAGLE 3.1 explainer, section "FC 정규화: EAGLE 3.1의 핵심 수정":
 * the LayerNorm parameters are taken into the FC layer, no weights are added).
 *
 * Outputs (caller-owned device memory):
 *   w_folded  bf16, 3*d*d elements: W'[k, n] = bf16_rne(gamma_s[k - s*d] * W[k, n])
 *             for LAYERNORM / RMSNORM and W[k, n] for NONE (s = k / d), stored
 *             as 1 KiB tiles of 16 columns x 32 k in the operand order of the
 *             gfx950 16x16x32 bf16 matrix instruction:
 *                 tile (n / 16, k / 32) starts at element
 *                     ((n / 16) * (3d / 32) + k / 32) * 512,
 *                 and holds W'[k, n] at offset 8 * (16 * ((k % 32) / 8) + n % 16) + k % 8
 *             (the 16 bytes of lane l = 16 * ((k % 32) / 8) + n % 16 are 8
 *             consecutive k of one column; the tiles of a 16-column block
 *             are consecutive along k, so that block is one contiguous run);
 *   u         float32 [3, d]: u[s][n] = sum over k in state s of W'[k, n]
 *             (from the stored, rounded values; unused by NONE);
 *   c         float32 [d]: c[n] = bias[n] + sum_s sum_k beta_s[k] W[s*d + k, n]
 *             (the beta term for LAYERNORM only).
 * Then, for the same norm_kind,
 *   out = sum_s rstd_s * (h_s . W'_s - mu_s * u_s) + c
 * equals eagle31_fuse's result up to rounding.  Uses a little library-owned
 * scratch memory (3 d floats and d / 64 counters, per device and stream, as
 * eagle31_fuse).  Deterministic.
 */
int eagle31_fold_prepare(int64_t d, int norm_kind, const void* const* gamma, const void* const* beta,
                         const void* W, const void* bias, void* w_folded, float* u, float* c,
                         void* stream);

/*
 * eagle31_fuse_folded - the fused step on prepared weights (see
 * eagle31_fold_prepare; norm_kind must be the one used to prepare them).
 * Uses library-owned scratch memory like eagle31_fuse.
 */
int eagle31_fuse_folded(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                        int norm_kind, float eps, const void* w_folded, const float* u, const float* c,
                        void* out, void* stream);

/* eagle31_fuse_folded with caller workspace (same rules as eagle31_fuse_ws). */
int eagle31_fuse_folded_ws(const void* h_low, const void* h_mid, const void* h_high, int64_t M,
                           int64_t d, int norm_kind, float eps, const void* w_folded, const float* u,
                           const float* c, void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * eagle31_fuse_rows, eagle31_fuse_folded_rows - eagle31_fuse and
 * eagle31_fuse_folded reading the hidden states where they already are and
 * writing into a wider buffer, with no copy on either side (the vLLM EAGLE 3.1
 * release post, devlery.com/blog/vllm-eagle31-attention-drift, section
 * "vLLM main에 들어갔다는 것이 뉴스입니다": no hard-coded assumption about
 * the target's hidden-state buffers):
 *
 *   token m (0 <= m < M) reads row src(m) of each state, at h_s + src(m) * ld[s]
 *   elements, where src(m) = row_index[m] when row_index is given, else m;
 *   its output row goes to out + m * ld_out.
 *
 * ld:        host int64[3]: elements between consecutive rows of h_low, h_mid,
 *            h_high, each in [d, 2^22] and a multiple of 8 (NULL: d each).  The
 *            states may be column blocks of one buffer, e.g. [n, 3d] with
 *            h_mid = h_low + d, h_high = h_low + 2d and ld = 3d each.
 * row_index: device int32 [M] or NULL, e.g. the positions of the accepted
 *            tokens; any order, repeats allowed.  An index outside [0, n_src)
 *            reads row 0 instead and that token's output row is written as
 *            zeros (never a fault).
 * n_src:     rows each state buffer holds, 1 <= n_src <= 2^31 - 1; at least M
 *            without an index list.  With one, n_src * ld[s] * 2 bytes must not
 *            exceed 2^32 for any state.
 * out:       bf16, row m at out + m * ld_out, ld_out in [d, 2^22] and a
 *            multiple of 8; e.g. the right half of the drafter-input buffer
 *            [M, 2d] (out = dst + d, ld_out = 2d).  Only d values per row are
 *            written.
 * h_s and out 16-byte aligned, row_index 4-byte aligned.  out's extent
 * ((M - 1) ld_out + d elements) must not overlap any state's
 * ((n_src - 1) ld[s] + d), the index list or the weight-side arguments
 * (EAGLE31_ERR_ALIAS).  Violations of the limits above: EAGLE31_ERR_SHAPE.
 * Everything else (norm, weights, library-owned scratch, M == 0) as
 * eagle31_fuse / eagle31_fuse_folded, whose results these equal bit for bit
 * on the gathered rows.
 */
int eagle31_fuse_rows(const void* h_low, const void* h_mid, const void* h_high, const int64_t* ld,
                      const int32_t* row_index, int64_t n_src, int64_t M, int64_t d, int norm_kind, float eps,
                      const void* const* gamma, const void* const* beta, const void* W, const void* bias, void* out,
                      int64_t ld_out, void* stream);
int eagle31_fuse_folded_rows(const void* h_low, const void* h_mid, const void* h_high, const int64_t* ld,
                             const int32_t* row_index, int64_t n_src, int64_t M, int64_t d, int norm_kind, float eps,
                             const void* w_folded, const float* u, const float* c, void* out, int64_t ld_out,
                             void* stream);

/*
 * eagle31_fuse_folded_noalloc - eagle31_fuse_folded for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the scratch memory (split-K partials,
 * statistics records, counters) is a fixed array inside the library, one per
 * device, eagle31_noalloc_scratch_bytes() bytes (16 MiB), held until the
 * process ends.  The call performs no allocation of its own; the caller still
 * provides every input and output.  Arguments, result and errors are those of
 * eagle31_fuse_folded, plus EAGLE31_ERR_TOO_LARGE (nothing enqueued) when the
 * problem's scratch exceeds the array: every call of at most 64 tokens up to
 * d = 8192 fits (calls of 65 to 128 tokens, whose partials grow with the
 * token count, may not), and prefill calls whose tile count needs no split-K
 * (e.g. d = 8192, M = 4096; d = 7168, M = 32768).
 * The first call on a device also enqueues the zeroing of the array's
 * counters on `stream`.  All calls on one device share its array and each
 * leaves its counters at zero: calls that overlap in time on one device (two
 * streams, two host threads) race and give undefined results; order them.
 */
int eagle31_fuse_folded_noalloc(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                                int norm_kind, float eps, const void* w_folded, const float* u, const float* c,
                                void* out, void* stream);

/* Bytes of the fixed scratch array behind eagle31_fuse_folded_noalloc. */
size_t eagle31_noalloc_scratch_bytes(void);

/*
 * eagle31_row_stats - the statistics pass on its own: per state s and token m,
 * mu[s*M + m] and rstd[s*M + m] (float32 [3, M]) as defined above
 * (LAYERNORM: mean and (var + eps)^-1/2; RMSNORM: 0 and (mean(x^2) + eps)^-1/2;
 * NONE: 0 and 1).
 */
int eagle31_row_stats(const void* h_low, const void* h_mid, const void* h_high, int64_t M, int64_t d,
                      int norm_kind, float eps, float* mu, float* rstd, void* stream);

/*
 * eagle31_norm_output - post-norm hidden-state feedback: the drafter's output
 * hidden state x [M, d] is normalised row by row before it is fed to the next
 * draft step (vLLM EAGLE 3.1 release post, devlery.com/blog/vllm-eagle31-attention-drift,
 * sections "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다" and "vLLM main에 들어갔다는
 * 것이 뉴스입니다"; the model card cited there names the layer norm_output):
 *
 *     out[m, :] = norm(x[m, :]) with the same three kinds as above, one gamma
 *                 and one beta for every row.
 *
 * x, out: bf16 [M, d] row-major.  out == x (in place) is allowed; any other
 *         overlap returns EAGLE31_ERR_ALIAS.
 * gamma:  bf16 [d] or NULL (ones); ignored for EAGLE31_NORM_NONE.
 * beta:   bf16 [d] or NULL (zeros); used by EAGLE31_NORM_LAYERNORM only.
 * Statistics and arithmetic in float32, out rounded to nearest even;
 * EAGLE31_NORM_NONE copies x.  d is limited to 8192 here (EAGLE31_ERR_SHAPE
 * above); every other limit and convention is the shared one.  Needs no
 * scratch memory.
 */
int eagle31_norm_output(const void* x, int64_t M, int64_t d, int norm_kind, float eps, const void* gamma,
                        const void* beta, void* out, void* stream);

/*
 * eagle31_embed_concat - the drafter's input row: the embedding of the token
 * sampled just before, followed by the fused feature (EAGLE-3 paper summary,
 * honbul.tistory.com/173, section "EAGLE-3가 바꾼 것 2"):
 *
 *     dst[m, 0:d]  = embed[tokens[m], :]       (zeros if tokens[m] < 0 or >= vocab)
 *     dst[m, d:2d] = fused[m, :]               (left untouched when fused is NULL)
 *
 * With fused NULL only the embedding half is written: the fused feature can
 * be written into dst[:, d:2d] directly by eagle31_fuse_rows /
 * eagle31_fuse_folded_rows (out = dst + d, ld_out = 2d), with no copy.
 * tokens:    int32 [M], device, 4-byte aligned.
 * embed:     bf16 [vocab, d] row-major; fused: bf16 [M, d] (e.g. the output of
 *            eagle31_fuse) or NULL; dst: bf16 [M, 2d]; all 16-byte aligned.
 * bad_count: device int32 or NULL; incremented once per token outside the
 *            table (the caller zeroes it).  Such a token never faults.
 * Bits are copied, nothing is rounded.  dst must not overlap any input.
 * Limits: 1 <= vocab <= 2^31 - 1, d % 64 == 0, d <= 8192 (EAGLE31_ERR_SHAPE);
 * M == 0 launches nothing.  Needs no scratch memory.
 */
int eagle31_embed_concat(const int32_t* tokens, int64_t M, int64_t d, int64_t vocab, const void* embed,
                         const void* fused, void* dst, int32_t* bad_count, void* stream);

/*
 * eagle31_verify_accept - the speculative-decoding verify / accept step for a
 * batch of B sequences with N drafts each (the Leviathan rule of the
 * speculative-decoding lesson, factory.pai-world.com/.../15-speculative-decoding-eagle3,
 * section "불변식: Leviathan 거부 샘플링"):
 *
 *   the drafts are taken left to right; draft d = draft[b][i] is kept iff
 *       u_acc[b][i] * p[b][i][d] < q[b][i][d]   (the product rounded to float32:
 *   the keep probability min(1, q/p) without a division; a draft with p = 0 is
 *   kept iff q > 0; an id outside [0, V) is rejected);
 *   at the first rejection j the next token is drawn from the residual
 *   w = max(q[b][j] - p[b][j], 0) (float32 difference), or from q[b][j] when
 *   every residual weight is zero; when all N are kept, from q[b][N];
 *   the draw is the inverse CDF in token order in exact arithmetic: the
 *   smallest t with w_0 + ... + w_t > u_res[b] * (w_0 + ... + w_{V-1}).
 *
 * p:          float32 [B, N, V], the drafter's distribution at each draft position;
 * q:          float32 [B, N + 1, V], the verifier's;
 * draft:      int32 [B, N]; u_acc: float32 [B, N]; u_res: float32 [B] (uniforms in
 *             [0, 1), supplied by the caller);
 * n_accepted: int32 [B], the drafts kept (j);
 * next_token: int32 [B], the token emitted after them, or -1 when the weights it
 *             is drawn from are all zero, hold NaN or a value above 1, or
 *             u_res is outside [0, 1).
 * All device memory, row-major, 4-byte aligned; outputs must not overlap
 * inputs.  Limits: 0 <= B <= 4096, 1 <= N <= 64, 1 <= V <= 2^26
 * (EAGLE31_ERR_SHAPE).  B == 0 launches nothing.  Uses library-owned scratch
 * memory (per device and stream, as eagle31_fuse).  Deterministic: the result
 * is unique (exact arithmetic), whatever the order of summation.
 */
int eagle31_verify_accept(const float* p, const float* q, const int32_t* draft, const float* u_acc,
                          const float* u_res, int64_t B, int64_t N, int64_t V, int32_t* n_accepted,
                          int32_t* next_token, void* stream);

/*
 * eagle31_verify_chunking - how eagle31_verify_accept splits a row: into
 * *chunks pieces of *tokens_per_chunk tokens (the last may be shorter), one
 * workgroup each, every workgroup summing a quarter per wave.  Pieces are
 * 2048, 4096 or 8192 tokens: the smallest that keeps B * chunks at or below
 * 256 workgroups (one per CU), else 8192; never more than 256 chunks per row
 * (longer rows take larger pieces).  Host arithmetic only; no device memory is touched.
 * Returns EAGLE31_ERR_SHAPE for the shapes eagle31_verify_accept rejects
 * (B must be >= 1 here), EAGLE31_ERR_NULL for a NULL output pointer.
 */
int eagle31_verify_chunking(int64_t B, int64_t N, int64_t V, int32_t* chunks, int32_t* tokens_per_chunk);

/* Human-readable name of a status code (static string). */
const char* eagle31_status_string(int status);

/* HIP error code behind the calling thread's last EAGLE31_ERR_HIP (0 if none). */
int eagle31_last_hip_error(void);

/* Free the library-owned scratch memory of every device.  Not to be called
 * while work that uses it is still queued. */
int eagle31_release(void);

/*
 * eagle31_debug_stats_recompute - test hook for the folded decode path
 * (eagle31_fuse_folded with 2 <= M <= 64, and up to 128 tokens at the widths
 * where the column-split decode kernel takes the call; calls of up to six tokens
 * at d = 2048 and 4096, of one token at d = 8192 and of one or two at the other
 * widths up to 4096 compute the statistics in every workgroup and hand nothing
 * over, so the hook does not change them).  That kernel computes each
 * token's statistics once and hands
 * them between workgroups through the workspace;
 * a reader waits a bounded time for them and, if they are not there, computes
 * the rows itself with the same arithmetic.  With on != 0 every reader takes
 * that fallback at once, so a test can check that it gives the same bits.
 * Process-wide; applies to calls enqueued after it returns; always returns
 * EAGLE31_OK.  Slower, and never needed in production.
 */
int eagle31_debug_stats_recompute(int on);

/*
 * eagle31_debug_fail_workspace_zero - test hook: while on != 0, the zeroing of
 * the counters of a newly allocated library-owned workspace reports a launch
 * failure (the call returns EAGLE31_ERR_HIP) instead of running, and the new
 * buffer is freed, so that a later call never finds a buffer whose counters
 * were not zeroed.  Process-wide; always returns EAGLE31_OK.  Never needed in
 * production.
 */
int eagle31_debug_fail_workspace_zero(int on);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE31_H */
