// Decode path of the fused per-state norm + FC (few tokens, M <= 64).
//
// The step is out = [n(h_low) | n(h_mid) | n(h_high)] . W + bias with a
// per-state LayerNorm or RMSNorm n (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정"; RMS form: vLLM EAGLE 3.1 release post,
// devlery.com/blog/vllm-eagle31-attention-drift, section
// "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다").  At small M the cost is
// streaming W [3d, d] from HBM once; the arithmetic still needs the matrix
// cores (a wave64 VALU GEMV at M = 64 would need more than the chip's FP32 rate).
//
// Design (one launch):
//  * Work is split over (column block b of 16*J columns) x (K chunk c); a
//    chunk never crosses a state boundary.  Workgroup (b, c) streams its
//    [chunk, 16*J] slice of W exactly once, in the stored row-major layout.
//    Each lane loads 8 consecutive rows x J consecutive columns and
//    transposes that 8 x J block in registers into J MFMA B operands
//    (8 consecutive k of one column each): half a byte-permute per element.
//  * The A operand is built on the fly from the raw hidden states: LayerNorm
//    needs the row mean before rounding to bf16, which is not known inside a
//    chunk, so the chunk subtracts a provisional shift K_c (mean of the
//    chunk's first 32 values of that row) and multiplies by gamma:
//        a = bf16((x - K_c) * gamma).
//    Rows M and M+1 of the A operand carry gamma and beta themselves, so the
//    same MFMAs also produce U_c = sum_k gamma_k W_kn and C_c = sum_k beta_k W_kn.
//    In exact arithmetic, with mu and rstd the state's statistics,
//        sum_k n(x)_k W_kn = rstd * sum_c (P_c - (mu - K_c) U_c) + sum_c C_c,
//    where P_c = sum_{k in c} (x_k - K_c) gamma_k W_kn.  Subtracting a shift
//    close to the mean before rounding keeps the bf16 rounding error relative
//    to the row's spread, not to its offset.
//  * The chunk statistics come from the same A fragments: shifted sums
//    S1 = sum (x - K_c) and S2 = sum (x - K_c)^2 (RMSNorm: sum x^2), so no
//    extra pass over the hidden states is made.
//  * Partials [rows, 16*J] and chunk statistics go to a workspace; the last
//    workgroup of a column block to arrive (atomic counter) combines the
//    statistics of all chunks (exact shifted-sum algebra in float64), forms
//    mu and rstd, and sums the partials in a fixed chunk order: the result
//    is bitwise reproducible.  It resets the counter for the next call.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int DW = 4;               // waves per workgroup
constexpr int DTHREADS = 64 * DW;
constexpr int DECODE_MAX_KPS = 16;  // K chunks per state segment, at most

template <int J>
struct RowVec;
template <>
struct RowVec<8> {
    typedef uint4 T;
    static __device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
        return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
    }
};
template <>
struct RowVec<4> {
    typedef uint2 T;
    static __device__ __forceinline__ uint32_t dw(const uint2& v, int i) { return i == 0 ? v.x : v.y; }
};

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// rows of the A operand that are stored: tokens, then the gamma and beta rows (LayerNorm)
// rows of the A operand after the tokens: gamma and beta (LayerNorm on the
// stored W; the folded variant gets u and c from the prepare step instead)
template <int NORM, bool FOLDED>
__host__ __device__ constexpr int param_rows() { return (NORM == NORM_LN && !FOLDED) ? 2 : 0; }

// column of MFMA block j for lane column cb inside the block of 16*J columns
template <int J, bool FOLDED>
__device__ __forceinline__ int dcol(int j, int cb) { return FOLDED ? 16 * j + cb : J * cb + j; }

template <int NORM, int J, int MT, bool FOLDED>
__global__ __launch_bounds__(DTHREADS) void decode_kernel(DecodeArgs a) {
    constexpr int NW = 16 * J;
    constexpr int ROWS = 16 * MT;
    typedef typename RowVec<J>::T BT;

    const int nb = a.nb, kps = a.kps, M = a.M, d = a.d;
    const int nchunks = 3 * kps;
    const int b = blockIdx.x % nb;
    const int c = blockIdx.x / nb;
    const int s = c / kps;
    const int cj = c - s * kps;
    const int TS = d >> 5;
    const int t0 = s * TS + (cj * TS) / kps;
    const int t1 = s * TS + ((cj + 1) * TS) / kps;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int n0 = b * NW;
    const int seg_k0 = s * d;
    const uint16_t* __restrict__ hs = a.h[s];
    const uint16_t* __restrict__ gam = a.gamma[s];
    const uint16_t* __restrict__ bet = a.beta[s];
    const uint16_t* __restrict__ W = a.W;

    // wave-combine buffers (2 x ROWS x NW floats), reused by the reducer for mu - K_c
    constexpr int BIG = (2 * ROWS * NW > 3 * DECODE_MAX_KPS * DECODE_MAX_M) ? 2 * ROWS * NW
                                                                             : 3 * DECODE_MAX_KPS * DECODE_MAX_M;
    __shared__ __attribute__((aligned(16))) float sh_big[BIG];
    __shared__ float sh_shift[DECODE_MAX_M];
    __shared__ float sh_s1[DW][DECODE_MAX_M];
    __shared__ float sh_s2[DW][DECODE_MAX_M];
    __shared__ float sh_r[3][DECODE_MAX_M];
    __shared__ float sh_mu[3][DECODE_MAX_M];
    __shared__ int sh_last;

    // ---- provisional shift per token row: mean of the chunk's first 32 values
    if (NORM == NORM_LN) {
        const int m = tid >> 2;
        if (m < M) {
            const uint4 x = *reinterpret_cast<const uint4*>(hs + (size_t)m * d + (t0 * 32 - seg_k0) + (tid & 3) * 8);
            float v = bf_lo(x.x) + bf_hi(x.x) + bf_lo(x.y) + bf_hi(x.y) + bf_lo(x.z) + bf_hi(x.z) + bf_lo(x.w) +
                      bf_hi(x.w);
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            if ((tid & 3) == 0) sh_shift[m] = v * (1.0f / 32.0f);
        }
        __syncthreads();
    }

    // ---- per-lane role of each 16-row tile of the A operand
    float shift[MT];
    int role[MT];  // 0 token, 1 gamma row, 2 beta row, 3 zero
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const int m = 16 * tt + cb;
        shift[tt] = 0.f;
        if (m < M) {
            role[tt] = 0;
            if (NORM == NORM_LN) shift[tt] = sh_shift[m];
        } else if (NORM == NORM_LN && !FOLDED && m == M) {
            role[tt] = 1;
        } else if (NORM == NORM_LN && !FOLDED && m == M + 1) {
            role[tt] = 2;
        } else {
            role[tt] = 3;
        }
    }

    f32x4 acc[MT][J];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float S1[MT], S2[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) S1[tt] = S2[tt] = 0.f;

    const uint4 ONES = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    const uint4 ZERO4 = make_uint4(0u, 0u, 0u, 0u);

    // stored W: 8 rows x J columns per lane; folded W'^T: J columns x 8 k per lane
    typedef typename std::conditional<FOLDED, uint4, BT>::type LT;
    constexpr int NL = FOLDED ? J : 8;
    LT wr[NL];
    uint4 xr[MT];
    uint4 gr, br;

    auto load_step = [&](int t, LT (&w)[NL], uint4 (&x)[MT], uint4& gg, uint4& bb) {
        const int kg = t * 32 + 8 * g;
        const int kl = kg - seg_k0;
        if (FOLDED) {
            const size_t K3 = (size_t)3 * d;
#pragma unroll
            for (int j = 0; j < NL; ++j)
                w[j] = *reinterpret_cast<const LT*>(a.wt + (size_t)(n0 + 16 * j + cb) * K3 + kg);
        } else {
            const uint16_t* wp = W + (size_t)kg * d + n0 + J * cb;
#pragma unroll
            for (int r = 0; r < NL; ++r) w[r] = *reinterpret_cast<const LT*>(wp + (size_t)r * d);
        }
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const int m = 16 * tt + cb;
            x[tt] = ZERO4;
            if (role[tt] == 0) x[tt] = *reinterpret_cast<const uint4*>(hs + (size_t)m * d + kl);
        }
        gg = ONES;
        if (!FOLDED && NORM != NORM_NONE && gam != nullptr) gg = *reinterpret_cast<const uint4*>(gam + kl);
        bb = ZERO4;
        if (!FOLDED && NORM == NORM_LN && bet != nullptr) bb = *reinterpret_cast<const uint4*>(bet + kl);
    };

    int t = t0 + wave;
    if (t < t1) load_step(t, wr, xr, gr, br);
    for (; t < t1; t += DW) {
        LT wn[NL];
        uint4 xn[MT];
        uint4 gn, bn;
        const bool more = (t + DW) < t1;
        if (more) load_step(t + DW, wn, xn, gn, bn);

        // B operands: column j of the 8 x J block, 8 consecutive k
        uint4 bf[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if constexpr (FOLDED) {
                bf[j] = wr[j];
            } else {
                uint32_t q[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t r0 = RowVec<J>::dw(wr[2 * p], j >> 1);
                    const uint32_t r1 = RowVec<J>::dw(wr[2 * p + 1], j >> 1);
                    q[p] = (j & 1) ? ((r0 >> 16) | (r1 & 0xffff0000u)) : ((r0 & 0xffffu) | (r1 << 16));
                }
                bf[j] = make_uint4(q[0], q[1], q[2], q[3]);
            }
        }
        // gamma of this lane's 8 k values
        float gf[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t w = u4get(gr, p);
            gf[2 * p] = bf_lo(w);
            gf[2 * p + 1] = bf_hi(w);
        }
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            uint4 af;
            if (NORM == NORM_NONE) {
                af = xr[tt];
            } else if (FOLDED) {
                // raw x feeds the MFMA; only the statistics are formed here
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t w = u4get(xr[tt], p);
                    float x0 = bf_lo(w), x1 = bf_hi(w);
                    if (NORM == NORM_LN) {
                        x0 -= shift[tt];
                        x1 -= shift[tt];
                        S1[tt] += x0 + x1;
                    }
                    S2[tt] += x0 * x0 + x1 * x1;
                }
                af = xr[tt];
            } else {
                uint32_t q[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t w = u4get(xr[tt], p);
                    float x0 = bf_lo(w), x1 = bf_hi(w);
                    if (NORM == NORM_LN) {
                        x0 -= shift[tt];
                        x1 -= shift[tt];
                        S1[tt] += x0 + x1;
                    }
                    S2[tt] += x0 * x0 + x1 * x1;
                    q[p] = pack_bf2(x0 * gf[2 * p], x1 * gf[2 * p + 1]);
                }
                af = make_uint4(q[0], q[1], q[2], q[3]);
                if (NORM == NORM_LN) {
                    // padding lanes hold x = 0 and shift = 0, so their sums stay 0
                    af = role[tt] == 0 ? af : (role[tt] == 1 ? gr : (role[tt] == 2 ? br : ZERO4));
                }
            }
#pragma unroll
            for (int j = 0; j < J; ++j) acc[tt][j] = mfma16x16x32(af, bf[j], acc[tt][j]);
        }

        if (more) {
#pragma unroll
            for (int r = 0; r < NL; ++r) wr[r] = wn[r];
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) xr[tt] = xn[tt];
            gr = gn;
            br = bn;
        }
    }

    // ---- per-row chunk statistics: sum over the 4 lane groups, then the waves
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const float a1 = group4_sum(S1[tt]);
        const float a2 = group4_sum(S2[tt]);
        const int m = 16 * tt + cb;
        if (g == 0 && m < M) {
            sh_s1[wave][m] = a1;
            sh_s2[wave][m] = a2;
        }
    }
    // ---- sum of the four waves' tiles in a fixed order: (w0 + w2) + (w1 + w3).
    // All waves share the lane <-> element mapping of the MFMA output, so the
    // tiles are exchanged in that "fragment order" with 16-byte LDS accesses.
    constexpr int FR = MT * J;  // f32x4 fragments per lane
    f32x4* buf0 = reinterpret_cast<f32x4*>(sh_big);
    f32x4* buf1 = buf0 + FR * 64;
    if (wave >= 2) {
        f32x4* dst = wave == 2 ? buf0 : buf1;
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int j = 0; j < J; ++j) dst[(tt * J + j) * 64 + lane] = acc[tt][j];
    }
    __syncthreads();
    if (wave < 2) {
        const f32x4* src = wave == 0 ? buf0 : buf1;
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int j = 0; j < J; ++j) acc[tt][j] += src[(tt * J + j) * 64 + lane];
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int j = 0; j < J; ++j) buf0[(tt * J + j) * 64 + lane] = acc[tt][j];
    }
    __syncthreads();

    const int slot = b * nchunks + c;
    f32x4* part = reinterpret_cast<f32x4*>(a.part) + (size_t)slot * FR * 64;
    if (wave == 0) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int j = 0; j < J; ++j) part[(tt * J + j) * 64 + lane] = acc[tt][j] + buf0[(tt * J + j) * 64 + lane];
    }
    if (NORM != NORM_NONE) {
        float* st = a.stats + (size_t)slot * DECODE_MAX_M * 3;
        for (int m = tid; m < M; m += DTHREADS) {
            const float v1 = (sh_s1[0][m] + sh_s1[2][m]) + (sh_s1[1][m] + sh_s1[3][m]);
            const float v2 = (sh_s2[0][m] + sh_s2[2][m]) + (sh_s2[1][m] + sh_s2[3][m]);
            st[3 * m + 0] = NORM == NORM_LN ? sh_shift[m] : 0.f;
            st[3 * m + 1] = v1;
            st[3 * m + 2] = v2;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + b, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (old == nchunks - 1);
    }
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    // ---- last arriver of column block b: statistics of every state, then the sum
    float* sh_delta = sh_big;  // [nchunks][64]: mu_s - K_c (LayerNorm)
    for (int m = tid; m < M; m += DTHREADS) {
        for (int ss = 0; ss < 3; ++ss) {
            double r = 1.0;
            if (NORM == NORM_LN) {
                double sum = 0.0;
                for (int cc = ss * kps; cc < (ss + 1) * kps; ++cc) {
                    const float* st = a.stats + ((size_t)(b * nchunks + cc) * DECODE_MAX_M + m) * 3;
                    const int cjj = cc - ss * kps;
                    const double n_c = 32.0 * (double)(((cjj + 1) * TS) / kps - (cjj * TS) / kps);
                    sum += n_c * (double)st[0] + (double)st[1];
                }
                const double mu = sum / (double)d;
                double m2 = 0.0;
                for (int cc = ss * kps; cc < (ss + 1) * kps; ++cc) {
                    const float* st = a.stats + ((size_t)(b * nchunks + cc) * DECODE_MAX_M + m) * 3;
                    const int cjj = cc - ss * kps;
                    const double n_c = 32.0 * (double)(((cjj + 1) * TS) / kps - (cjj * TS) / kps);
                    const double dl = mu - (double)st[0];
                    m2 += (double)st[2] - 2.0 * dl * (double)st[1] + n_c * dl * dl;
                    sh_delta[cc * DECODE_MAX_M + m] = (float)dl;
                }
                sh_mu[ss][m] = (float)mu;
                r = 1.0 / sqrt(m2 / (double)d + (double)a.eps);
            } else if (NORM == NORM_RMS) {
                double sq = 0.0;
                for (int cc = ss * kps; cc < (ss + 1) * kps; ++cc)
                    sq += (double)a.stats[((size_t)(b * nchunks + cc) * DECODE_MAX_M + m) * 3 + 2];
                r = 1.0 / sqrt(sq / (double)d + (double)a.eps);
            }
            sh_r[ss][m] = (float)r;
        }
    }
    __syncthreads();

    // Each thread takes one fragment (4 consecutive rows of one column) at a
    // time, reading every chunk's partial in a fixed order.
    const f32x4* pbase = reinterpret_cast<const f32x4*>(a.part) + (size_t)b * nchunks * FR * 64;
    // fragment holding (row, column): row = 16*tt + 4*(lane>>4) + e, column = dcol(j, lane&15)
    const int Mu = M, Mc = M + 1;
    const int u_tt = Mu >> 4, u_g = (Mu & 15) >> 2, u_e = Mu & 3;
    const int c_tt = Mc >> 4, c_g = (Mc & 15) >> 2, c_e = Mc & 3;
    for (int f = tid; f < FR * 64; f += DTHREADS) {
        const int tt = f / (J * 64);
        const int j = (f / 64) % J;
        const int ln = f & 63;
        const int row0 = 16 * tt + 4 * (ln >> 4);
        if (row0 >= M) continue;
        const int n = dcol<J, FOLDED>(j, ln & 15);
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        float cterm = 0.f;
        for (int ss = 0; ss < 3; ++ss) {
            float ys[4] = {0.f, 0.f, 0.f, 0.f};
            for (int cc = ss * kps; cc < (ss + 1) * kps; ++cc) {
                const f32x4* p = pbase + (size_t)cc * FR * 64;
                const f32x4 v = p[f];
                if (NORM == NORM_LN && !FOLDED) {
                    const float U = p[(u_tt * J + j) * 64 + 16 * u_g + (ln & 15)][u_e];
                    cterm += p[(c_tt * J + j) * 64 + 16 * c_g + (ln & 15)][c_e];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = row0 + e;
                        const float dl = m < M ? sh_delta[cc * DECODE_MAX_M + m] : 0.f;
                        ys[e] += v[e] - dl * U;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) ys[e] += v[e];
                }
            }
            if (FOLDED && NORM == NORM_LN) {
                const float us = a.u[(size_t)ss * d + n0 + n];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = row0 + e;
                    ys[e] -= (m < M ? sh_mu[ss][m] : 0.f) * us;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = row0 + e;
                const float r = (NORM == NORM_NONE || m >= M) ? 1.f : sh_r[ss][m];
                y[e] += r * ys[e];
            }
        }
        float add = cterm;
        if (FOLDED) {
            add += a.c[n0 + n];
        } else if (a.bias != nullptr) {
            add += bf_one(a.bias[n0 + n]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = row0 + e;
            if (m < M) {
                const float v = y[e] + add;
                a.out[(size_t)m * d + n0 + n] = __builtin_bit_cast(uint16_t, (__bf16)v);
            }
        }
    }
    if (tid == 0) a.counters[b] = 0;
}

DecodePlan plan_decode(int M, int d, int norm, bool folded) {
    DecodePlan p;
    const int rows = M + ((norm == NORM_LN && !folded) ? 2 : 0);
    p.MT = (rows + 15) / 16;
    p.J = p.MT <= 2 ? 8 : 4;
    if (d % (16 * p.J) != 0) p.J = 4;
    p.nb = d / (16 * p.J);
    const int TS = d / 32;
    int kps = (768 + 3 * p.nb - 1) / (3 * p.nb);
    if (kps < 1) kps = 1;
    const int kmax = TS / DW > 0 ? TS / DW : 1;
    if (kps > kmax) kps = kmax;
    if (kps > DECODE_MAX_KPS) kps = DECODE_MAX_KPS;
    p.kps = kps;
    const size_t slots = (size_t)p.nb * 3 * kps;
    p.counters_bytes = ((size_t)p.nb * sizeof(int) + 255) / 256 * 256;
    p.stats_bytes = (slots * DECODE_MAX_M * 3 * sizeof(float) + 255) / 256 * 256;
    p.part_bytes = (slots * (size_t)p.MT * 16 * 16 * p.J * sizeof(float) + 255) / 256 * 256;
    return p;
}

template <int NORM, int J, int MT, bool FOLDED>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    const int grid = a.nb * 3 * a.kps;
    decode_kernel<NORM, J, MT, FOLDED><<<grid, DTHREADS, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM, bool FOLDED>
static hipError_t launch_decode_n(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    switch (p.MT) {
        case 1:
            return p.J == 8 ? launch_decode_t<NORM, 8, 1, FOLDED>(a, st) : launch_decode_t<NORM, 4, 1, FOLDED>(a, st);
        case 2:
            return p.J == 8 ? launch_decode_t<NORM, 8, 2, FOLDED>(a, st) : launch_decode_t<NORM, 4, 2, FOLDED>(a, st);
        case 3: return launch_decode_t<NORM, 4, 3, FOLDED>(a, st);
        case 4: return launch_decode_t<NORM, 4, 4, FOLDED>(a, st);
        case 5: return launch_decode_t<NORM, 4, 5, FOLDED>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool FOLDED>
static hipError_t launch_decode_f(const DecodeArgs& a, int norm, const DecodePlan& p, hipStream_t st) {
    if (norm == NORM_LN) return launch_decode_n<NORM_LN, FOLDED>(a, p, st);
    if (norm == NORM_RMS) return launch_decode_n<NORM_RMS, FOLDED>(a, p, st);
    return launch_decode_n<NORM_NONE, FOLDED>(a, p, st);
}

hipError_t launch_decode(const DecodeArgs& a, int norm, bool folded, const DecodePlan& p, hipStream_t st) {
    return folded ? launch_decode_f<true>(a, norm, p, st) : launch_decode_f<false>(a, norm, p, st);
}

}  // namespace e31
