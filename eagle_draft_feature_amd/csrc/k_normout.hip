// Post-norm hidden-state feedback: the drafter's output hidden state [M, d]
// is row-normalised (LayerNorm or RMSNorm with its own gamma / beta) before
// it is fed to the next draft step (vLLM EAGLE 3.1 release post,
// devlery.com/blog/vllm-eagle31-attention-drift, sections "EAGLE 3.1이 바꾼
// 것은 작지만 낮은 계층입니다" and "vLLM main에 들어갔다는 것이 뉴스입니다":
// post-norm hidden-state feedback; the model card it cites calls the layer
// norm_output).
//
// One wave64 per row, rows taken at a grid stride.  A lane holds its P
// 16-byte pieces of the row in registers (pieces lane, lane+64, ...), so the
// LayerNorm variance is two passes (mean, then mean of squared deviations)
// over a single HBM read, and the row is fully loaded before any store: out
// may be x itself.  Every load is unconditional: a lane past the row's end
// re-reads the last piece and its values are masked out of the sums (a
// guarded load would get a wait of its own).  Such a lane also normalises and
// stores that last piece, writing the very bytes its owner writes, so the
// store side has no branch either.  gamma and beta are staged once per
// workgroup into LDS (bfloat16, 4*d bytes) and read from there for every row;
// a missing gamma or beta arrives as a readable stand-in pointer with its flag
// off.  Eight waves per workgroup and at most 128 registers per lane let four
// waves share a SIMD, so 16 rows per CU are in flight: a wave's row is one
// chain (load, reduce, store; the next row's loads wait for the stores'
// completion as well), and the overlap between waves is what keeps HBM busy.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int NR_WAVES = 8;
constexpr int NT = 2;  // buffer instruction cache policy: non-temporal

template <int NORM, int P>
__global__ __launch_bounds__(64 * NR_WAVES) __attribute__((amdgpu_waves_per_eu(4))) void norm_rows_kernel(const uint16_t* x, int M, int d, float eps,
                                                        const uint16_t* __restrict__ gamma, int has_gamma,
                                                        const uint16_t* __restrict__ beta, int has_beta,
                                                        uint16_t* out) {
    extern __shared__ u32x4 gb[];  // [d/8] gamma pieces then [d/8] beta pieces, bfloat16
    const int lane = threadIdx.x & 63;
    const int nvec = d >> 3;
    if (NORM != NORM_NONE) {
        const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}, zeros = {0u, 0u, 0u, 0u};
        for (int i = threadIdx.x; i < nvec; i += 64 * NR_WAVES) {
            const u32x4 gl = reinterpret_cast<const u32x4*>(gamma)[i];
            const u32x4 bl = reinterpret_cast<const u32x4*>(beta)[i];
            gb[i] = has_gamma ? gl : ones;
            gb[nvec + i] = (NORM == NORM_LN && has_beta) ? bl : zeros;
        }
        __syncthreads();
    }
    const float inv_d = 1.0f / (float)d;
    const int nwaves = gridDim.x * NR_WAVES;
    for (int row = blockIdx.x * NR_WAVES + (threadIdx.x >> 6); row < M; row += nwaves) {
        // buffer accesses over the row: one 32-bit offset per piece instead of
        // a 64-bit address (every offset is clamped into the row).  Loads and
        // stores carry the non-temporal hint (cache policy bit 1): every byte
        // is touched once.
        const __amdgpu_buffer_rsrc_t rin =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (size_t)row * d), 0, d * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rout =
            __builtin_amdgcn_make_buffer_rsrc(out + (size_t)row * d, 0, d * 2, 0x00020000);
        u32x4 v[P];
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rin, 16 * min(lane + 64 * i, nvec - 1), 0, NT);
        // Each pass below re-expands the packed pieces: the empty asm hides
        // from the compiler that they are unchanged, so it does not keep 8
        // floats per piece live from one pass to the next (which would not
        // fit the register cap).
        auto refresh = [&]() {
#pragma unroll
            for (int i = 0; i < P; ++i) asm volatile("" : "+v"(v[i]));
        };

        float mean = 0.f, r = 1.f;
        if (NORM == NORM_LN) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                float t = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) t += bf_lo(w[q]) + bf_hi(w[q]);
                s += lane + 64 * i < nvec ? t : 0.f;
            }
            mean = wave_sum(s) * inv_d;
            refresh();
            float dev = 0.f;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                float t = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = bf_lo(w[q]) - mean, b = bf_hi(w[q]) - mean;
                    t += a * a + b * b;
                }
                dev += lane + 64 * i < nvec ? t : 0.f;
            }
            r = 1.0f / sqrtf(wave_sum(dev) * inv_d + eps);
        } else if (NORM == NORM_RMS) {
            float sq = 0.f;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                float t = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = bf_lo(w[q]), b = bf_hi(w[q]);
                    t += a * a + b * b;
                }
                sq += lane + 64 * i < nvec ? t : 0.f;
            }
            r = 1.0f / sqrtf(wave_sum(sq) * inv_d + eps);
        }

        refresh();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int vi = min(lane + 64 * i, nvec - 1);
            if (NORM == NORM_NONE) {
                __builtin_amdgcn_raw_buffer_store_b128(v[i], rout, 16 * vi, 0, NT);
            } else {
                const u32x4 gw = gb[vi], bw = gb[nvec + vi];
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = (bf_lo(w[q]) - mean) * r * bf_lo(gw[q]) + bf_lo(bw[q]);
                    const float hi = (bf_hi(w[q]) - mean) * r * bf_hi(gw[q]) + bf_hi(bw[q]);
                    o[q] = pack_bf2(lo, hi);
                }
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, rout, 16 * vi, 0, NT);
            }
            // one piece at a time: hoisting every piece's gamma / beta reads
            // would not fit the register cap
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Workgroups: enough for every row, at most 512 (two per CU, the four waves
// per SIMD the register cap allows); each wave then takes rows at a stride of
// 8 * grid.  P is the smallest listed piece count that covers the row, exact
// for d = 512 * P.
template <int NORM>
static hipError_t launch_norm_rows_p(const uint16_t* x, int M, int d, float eps, const uint16_t* gamma,
                                     const uint16_t* beta, uint16_t* out, hipStream_t st) {
    // stand-in for a missing parameter: row 0 of x, which holds d values
    const int has_g = gamma != nullptr, has_b = beta != nullptr;
    const uint16_t* gp = has_g ? gamma : x;
    const uint16_t* bp = has_b ? beta : x;
    const int nvec = d / 8;
    const int grid = (int)std::min<int64_t>(((int64_t)M + NR_WAVES - 1) / NR_WAVES, 512);
    const size_t lds = NORM == NORM_NONE ? 0 : (size_t)d * 2 * sizeof(uint16_t);
#define E31_NORM_ROWS(PP) \
    norm_rows_kernel<NORM, PP><<<grid, 64 * NR_WAVES, lds, st>>>(x, M, d, eps, gp, has_g, bp, has_b, out)
    const int need = (nvec + 63) / 64;
    if (need <= 1) E31_NORM_ROWS(1);
    else if (need <= 2) E31_NORM_ROWS(2);
    else if (need <= 3) E31_NORM_ROWS(3);
    else if (need <= 4) E31_NORM_ROWS(4);
    else if (need <= 6) E31_NORM_ROWS(6);
    else if (need <= 8) E31_NORM_ROWS(8);
    else if (need <= 10) E31_NORM_ROWS(10);
    else if (need <= 12) E31_NORM_ROWS(12);
    else if (need <= 14) E31_NORM_ROWS(14);
    else E31_NORM_ROWS(16);
#undef E31_NORM_ROWS
    return hipGetLastError();
}

hipError_t launch_norm_rows(const uint16_t* x, int M, int d, int norm, float eps, const uint16_t* gamma,
                            const uint16_t* beta, uint16_t* out, hipStream_t st) {
    if (d > NORM_ROWS_MAX_D || d % 64 != 0 || M <= 0) return hipErrorInvalidValue;
    if (norm == NORM_LN) return launch_norm_rows_p<NORM_LN>(x, M, d, eps, gamma, beta, out, st);
    if (norm == NORM_RMS) return launch_norm_rows_p<NORM_RMS>(x, M, d, eps, gamma, beta, out, st);
    return launch_norm_rows_p<NORM_NONE>(x, M, d, eps, gamma, beta, out, st);
}

}  // namespace e31
