// Column-block decode kernel of the fused per-state norm + FC (few tokens).
//
// With the norm parameters folded into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the LayerNorm parameters are absorbed
// into the FC), the output is
//     out = sum_s rstd_s * (P_s - mu_s * u_s) + c,   P_s = h_s . W'_s^T,
// so the raw hidden states feed the matrix cores directly; mu and rstd come
// from the row-statistics pass launched just before this kernel.
//
// One workgroup owns 16 output columns over the whole K = 3d: it streams 16
// complete rows of W'^T [d, 3d] (6d contiguous bytes each), so no partial
// sum ever leaves the workgroup: no workspace, no atomics, no cross-workgroup
// fences.  Its 12 waves are 4 per state; a wave takes every 4th k-step of 32
// of its state, so its hidden-state pointer never changes and its hot loop
// is loads and MFMAs only.  Token rows beyond M read row 0: an MFMA output
// row depends on its own A row only, and those rows are never stored.
// The four tiles of a state are summed pairwise in LDS ((w0+w2)+(w1+w3)),
// and the epilogue combines the three states with their statistics: the
// result is deterministic.
//
// Memory pipeline: each lane's B operand is one 16-byte load of W'^T (8
// consecutive k of one column) and its A operands one 16-byte load per 16
// tokens (L2 hits shared by every column block).  Both are prefetched CPF
// steps ahead in a register ring, so the wait before a step's MFMAs covers
// only loads issued CPF steps earlier.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int CWS = 4;               // waves per state
constexpr int CW = 3 * CWS;          // waves per workgroup
constexpr int CTHREADS = 64 * CW;
constexpr int CPF = 8;               // prefetch depth (k-steps per wave)

template <int NORM, int MT, bool INSTATS>
__global__ __launch_bounds__(CTHREADS) void decode_cols_kernel(DecodeColsArgs a) {
    const int M = a.M, d = a.d;
    const int nblk = d >> 4;
    // XCD-aware order: workgroup ids go round robin over the 8 XCDs, so each
    // XCD takes a contiguous range of column blocks
    const int per = (nblk + 7) >> 3;
    const int blk = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (blk >= nblk) return;
    const int n0 = blk * 16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int s = wave / CWS, sub = wave - s * CWS;
    const int TS = d >> 5;  // k-steps per state
    const uint16_t* __restrict__ hs = s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2]);
    // this wave's steps: j = sub + CWS * i inside state s
    const uint16_t* __restrict__ wp =
        a.wt + (size_t)(n0 + cb) * ((size_t)3 * d) + (size_t)s * d + 8 * g + (size_t)sub * 32;
    const uint16_t* ap[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const int m = 16 * tt + cb;
        ap[tt] = hs + (size_t)(m < M ? m : 0) * d + 8 * g + (size_t)sub * 32;
    }
    const int nst = (TS - sub + CWS - 1) / CWS;
    constexpr int STEP = CWS * 32;  // elements between this wave's steps

    // In-kernel statistics (few tokens): every lane accumulates shifted sums
    // S1 = sum (x - K), S2 = sum (x - K)^2 (RMSNorm: sum x^2) of its A
    // fragments; K is one shift per token and state shared by all waves of
    // the workgroup (the mean of the state's first 32 values of that row), so
    // the sums of the 4 waves of a state combine exactly and the variance
    // S2/d - (S1/d)^2 stays well conditioned.
    __shared__ float sh_k[3][DECODE_MAX_M];
    __shared__ float sh_st[3][CWS][2][DECODE_MAX_M];
    float kshift[MT];
    float S1[MT], S2[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) S1[tt] = S2[tt] = kshift[tt] = 0.f;
    if (INSTATS && NORM == NORM_LN) {
        if (tid < 3 * 4 * DECODE_MAX_M) {
            const int q = tid / (4 * DECODE_MAX_M), r = tid - q * 4 * DECODE_MAX_M;
            const int m = r >> 2;
            if (m < M) {
                const uint16_t* hq = q == 0 ? a.h[0] : (q == 1 ? a.h[1] : a.h[2]);
                const uint4 x = *reinterpret_cast<const uint4*>(hq + (size_t)m * d + (r & 3) * 8);
                float v = bf_lo(x.x) + bf_hi(x.x) + bf_lo(x.y) + bf_hi(x.y) + bf_lo(x.z) + bf_hi(x.z) +
                          bf_lo(x.w) + bf_hi(x.w);
                v += __shfl_xor(v, 1, 64);
                v += __shfl_xor(v, 2, 64);
                if ((r & 3) == 0) sh_k[q][m] = v * (1.0f / 32.0f);
            }
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const int m = 16 * tt + cb;
            kshift[tt] = m < M ? sh_k[s][m] : 0.f;
        }
    }
    // padding rows read row 0; their sums are masked out when they are stored
    auto stats = [&](const uint4 (&x)[MT]) {
        if (!INSTATS || NORM == NORM_NONE) return;
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const uint32_t w[4] = {x[tt].x, x[tt].y, x[tt].z, x[tt].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float x0 = bf_lo(w[p]), x1 = bf_hi(w[p]);
                if (NORM == NORM_LN) {
                    x0 -= kshift[tt];
                    x1 -= kshift[tt];
                    S1[tt] += x0 + x1;
                }
                S2[tt] = fmaf(x0, x0, fmaf(x1, x1, S2[tt]));
            }
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 rw[CPF];
    uint4 rx[CPF][MT];
    const int nfull = (nst / CPF) * CPF;
    if (nfull > 0) {
#pragma unroll
        for (int p = 0; p < CPF; ++p) {
            rw[p] = *reinterpret_cast<const uint4*>(wp + (size_t)p * STEP);
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) rx[p][tt] = *reinterpret_cast<const uint4*>(ap[tt] + (size_t)p * STEP);
        }
        for (int i = 0; i < nfull; i += CPF) {
#pragma unroll
            for (int p = 0; p < CPF; ++p) {
                const uint4 w = rw[p];
                uint4 x[MT];
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) x[tt] = rx[p][tt];
                // refill the slot CPF steps ahead; past the end it re-reads a
                // step of this wave, which keeps the loads in flight fixed
                const int in = (i + p + CPF < nfull) ? i + p + CPF : nfull - CPF + p;
                rw[p] = *reinterpret_cast<const uint4*>(wp + (size_t)in * STEP);
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) rx[p][tt] = *reinterpret_cast<const uint4*>(ap[tt] + (size_t)in * STEP);
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) acc[tt] = mfma16x16x32(x[tt], w, acc[tt]);
                stats(x);
            }
        }
    }
    for (int i = nfull; i < nst; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(wp + (size_t)i * STEP);
        uint4 x[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            x[tt] = *reinterpret_cast<const uint4*>(ap[tt] + (size_t)i * STEP);
            acc[tt] = mfma16x16x32(x[tt], w, acc[tt]);
        }
        stats(x);
    }
    if (INSTATS && NORM != NORM_NONE) {
        // per row: the 4 lane groups, then (below) the 4 waves of the state
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const float a1 = group4_sum(S1[tt]);
            const float a2 = group4_sum(S2[tt]);
            const int m = 16 * tt + cb;
            if (g == 0 && m < M) {
                sh_st[s][sub][0][m] = a1;
                sh_st[s][sub][1][m] = a2;
            }
        }
    }

    // ---- per state, sum the 4 wave tiles pairwise: (w0 + w2) + (w1 + w3)
    __shared__ __attribute__((aligned(16))) f32x4 buf[3][2][MT * 64];
#pragma unroll
    for (int half = 2; half >= 1; half >>= 1) {
        if (sub >= half && sub < 2 * half) {
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) buf[s][sub - half][tt * 64 + lane] = acc[tt];
        }
        __syncthreads();
        if (sub < half) {
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) acc[tt] += buf[s][sub][tt * 64 + lane];
        }
        __syncthreads();
    }
    // the leaders of states 1 and 2 hand their tiles to the leader of state 0
    if (sub == 0 && s > 0) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) buf[s][0][tt * 64 + lane] = acc[tt];
    }
    __syncthreads();
    if (wave != 0) return;

    // ---- epilogue (wave 0): lane holds column n0 + cb, rows 16*tt + 4*g + e
    const int n = n0 + cb;
    float us[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN)
#pragma unroll
        for (int q = 0; q < 3; ++q) us[q] = a.u[(size_t)q * d + n];
    const float cn = a.c[n];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const f32x4 p1 = buf[1][0][tt * 64 + lane];
        const f32x4 p2 = buf[2][0][tt * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * tt + 4 * g + e;
            if (m >= M) continue;
            const float P[3] = {acc[tt][e], p1[e], p2[e]};
            float y = cn;
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                float mu = 0.f, r = 1.f;
                if (NORM != NORM_NONE) {
                    if (INSTATS) {
                        const float s1 = (sh_st[q][0][0][m] + sh_st[q][2][0][m]) + (sh_st[q][1][0][m] + sh_st[q][3][0][m]);
                        const float s2 = (sh_st[q][0][1][m] + sh_st[q][2][1][m]) + (sh_st[q][1][1][m] + sh_st[q][3][1][m]);
                        const float inv_d = 1.0f / (float)d;
                        if (NORM == NORM_LN) {
                            const float dm = s1 * inv_d;
                            mu = sh_k[q][m] + dm;
                            r = 1.0f / sqrtf(fmaxf(s2 * inv_d - dm * dm, 0.f) + a.eps);
                        } else {
                            r = 1.0f / sqrtf(s2 * inv_d + a.eps);
                        }
                    } else {
                        r = a.rstd[(size_t)q * M + m];
                        if (NORM == NORM_LN) mu = a.mu[(size_t)q * M + m];
                    }
                }
                y += r * (P[q] - mu * us[q]);
            }
            a.out[(size_t)m * d + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
        }
    }
}

template <int NORM>
static hipError_t launch_cols_n(const DecodeColsArgs& a, hipStream_t st) {
    const int nblk = a.d / 16;
    const int grid = ((nblk + 7) / 8) * 8;
    const int MT = (a.M + 15) / 16;
    if (a.instats) {
        if (MT != 1) return hipErrorInvalidValue;
        decode_cols_kernel<NORM, 1, true><<<grid, CTHREADS, 0, st>>>(a);
        return hipGetLastError();
    }
    switch (MT) {
        case 1: decode_cols_kernel<NORM, 1, false><<<grid, CTHREADS, 0, st>>>(a); break;
        case 2: decode_cols_kernel<NORM, 2, false><<<grid, CTHREADS, 0, st>>>(a); break;
        case 3: decode_cols_kernel<NORM, 3, false><<<grid, CTHREADS, 0, st>>>(a); break;
        case 4: decode_cols_kernel<NORM, 4, false><<<grid, CTHREADS, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_cols(const DecodeColsArgs& a, int norm, hipStream_t st) {
    if (norm == NORM_LN) return launch_cols_n<NORM_LN>(a, st);
    if (norm == NORM_RMS) return launch_cols_n<NORM_RMS>(a, st);
    return launch_cols_n<NORM_NONE>(a, st);
}

}  // namespace e31
