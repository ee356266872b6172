// Row statistics of the three hidden states: per state s and token m, the
// mean and 1/sqrt(var + eps) of a LayerNorm, or 1/sqrt(mean(x^2) + eps) of
// an RMSNorm (EAGLE 3.1 explainer, llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html,
// section "FC 정규화: EAGLE 3.1의 핵심 수정"; RMS form from the vLLM EAGLE 3.1
// release post, devlery.com/blog/vllm-eagle31-attention-drift, section
// "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다").
//
// One wave64 per (state, token) row; token m reads its source row (an
// index list or m, at the state's leading dimension).  Each lane loads
// 16-byte vectors at a 64-lane stride, so every load instruction of the wave
// covers 1 KiB of the row contiguously.  Up to CACHE vectors per lane stay in registers, which
// makes the variance a true two-pass computation (mean first, then the mean
// of squared deviations) from a single read of HBM; longer rows re-read the
// tail for the second pass.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

template <int NORM, int CACHE>
__global__ __launch_bounds__(256) void row_stats_kernel(const uint16_t* __restrict__ h0,
                                                        const uint16_t* __restrict__ h1,
                                                        const uint16_t* __restrict__ h2, RowView rv, int M,
                                                        int d, float eps, float* __restrict__ mu,
                                                        float* __restrict__ rstd) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= 3 * M) return;
    const int s = row / M;
    const int m = row - s * M;
    bool ok;
    const int src = rv_src(rv, m, ok);  // an invalid index reads row 0 (its output row is zeros)
    (void)ok;
    const uint16_t* base = (s == 0 ? h0 : (s == 1 ? h1 : h2)) + (size_t)src * (size_t)rv_ld(rv, s);
    const uint4* vec = reinterpret_cast<const uint4*>(base);
    const int nvec = d >> 3;

    uint4 cache[CACHE];
    float sum = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
        const int v = lane + 64 * i;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (v < nvec) x = vec[v];
        cache[i] = x;
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf_lo(w[q]), b = bf_hi(w[q]);
            sum += a + b;
            sq += a * a + b * b;
        }
    }
    for (int v = lane + 64 * CACHE; v < nvec; v += 64) {
        const uint4 x = vec[v];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf_lo(w[q]), b = bf_hi(w[q]);
            sum += a + b;
            sq += a * a + b * b;
        }
    }

    const float inv_d = 1.0f / (float)d;
    float mean = 0.f, r = 1.f;
    if (NORM == NORM_LN) {
        mean = wave_sum(sum) * inv_d;
        float dev = 0.f;
#pragma unroll
        for (int i = 0; i < CACHE; ++i) {
            if (lane + 64 * i < nvec) {
                const uint32_t w[4] = {cache[i].x, cache[i].y, cache[i].z, cache[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = bf_lo(w[q]) - mean, b = bf_hi(w[q]) - mean;
                    dev += a * a + b * b;
                }
            }
        }
        for (int v = lane + 64 * CACHE; v < nvec; v += 64) {
            const uint4 x = vec[v];
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = bf_lo(w[q]) - mean, b = bf_hi(w[q]) - mean;
                dev += a * a + b * b;
            }
        }
        const float var = wave_sum(dev) * inv_d;
        r = 1.0f / sqrtf(var + eps);
    } else if (NORM == NORM_RMS) {
        const float ms = wave_sum(sq) * inv_d;
        r = 1.0f / sqrtf(ms + eps);
    }
    if (lane == 0) {
        mu[s * M + m] = mean;
        rstd[s * M + m] = r;
    }
}

template <int NORM>
static hipError_t launch_stats_norm(const uint16_t* h0, const uint16_t* h1, const uint16_t* h2, const RowView& rv,
                                    int M, int d, float eps, float* mu, float* rstd, hipStream_t st) {
    const int nvec = d / 8;
    const int blocks = (3 * M + 3) / 4;
    if (nvec <= 64 * 2)
        row_stats_kernel<NORM, 2><<<blocks, 256, 0, st>>>(h0, h1, h2, rv, M, d, eps, mu, rstd);
    else if (nvec <= 64 * 4)
        row_stats_kernel<NORM, 4><<<blocks, 256, 0, st>>>(h0, h1, h2, rv, M, d, eps, mu, rstd);
    else if (nvec <= 64 * 8)
        row_stats_kernel<NORM, 8><<<blocks, 256, 0, st>>>(h0, h1, h2, rv, M, d, eps, mu, rstd);
    else if (nvec <= 64 * 12)
        row_stats_kernel<NORM, 12><<<blocks, 256, 0, st>>>(h0, h1, h2, rv, M, d, eps, mu, rstd);
    else
        row_stats_kernel<NORM, 16><<<blocks, 256, 0, st>>>(h0, h1, h2, rv, M, d, eps, mu, rstd);
    return hipGetLastError();
}

hipError_t launch_row_stats(const uint16_t* h0, const uint16_t* h1, const uint16_t* h2, const RowView& rv, int M,
                            int d, int norm, float eps, float* mu, float* rstd, hipStream_t st) {
    if (norm == NORM_LN) return launch_stats_norm<NORM_LN>(h0, h1, h2, rv, M, d, eps, mu, rstd, st);
    if (norm == NORM_RMS) return launch_stats_norm<NORM_RMS>(h0, h1, h2, rv, M, d, eps, mu, rstd, st);
    return launch_stats_norm<NORM_NONE>(h0, h1, h2, rv, M, d, eps, mu, rstd, st);
}

}  // namespace e31
