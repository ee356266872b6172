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
//  * Work is split over (column block b of 16*J columns) x (K chunk c), one
//    8-wave workgroup per pair and about one workgroup per CU.  Workgroup
//    (b, c) streams its [chunk, 16*J] slice of W exactly once, in the stored
//    row-major layout: each lane loads 8 consecutive rows x J consecutive
//    columns and transposes that 8 x J block in registers into J MFMA B
//    operands (8 consecutive k of one column each): half a byte-permute per
//    element.  (The folded weight has its own kernel: its tiles are MFMA
//    operands as loaded.)
//  * A chunk that crosses a state boundary is processed as pieces, one per
//    state; every piece has its own partial tile and statistics.
//  * The A operand is built on the fly from the raw hidden states: LayerNorm
//    needs the row mean before rounding to bf16, which is not known inside a
//    piece, so the piece subtracts a provisional shift K_p (mean of the
//    piece's first 32 values of that row) and multiplies by gamma:
//        a = bf16((x - K_p) * gamma).
//    Rows M and M+1 of the A operand carry gamma and beta themselves, so the
//    same MFMAs also produce U_p = sum_k gamma_k W_kn and C_p = sum_k beta_k W_kn.
//    In exact arithmetic, with mu and rstd the state's statistics,
//        sum_k n(x)_k W_kn = rstd * sum_p (P_p - (mu - K_p) U_p) + sum_p C_p,
//    where P_p = sum_{k in p} (x_k - K_p) gamma_k W_kn.  Subtracting a shift
//    close to the mean before rounding keeps the bf16 rounding error relative
//    to the row's spread, not to its offset.
//  * The piece statistics come from the same A fragments: shifted sums
//    S1 = sum (x - K_p) and S2 = sum (x - K_p)^2 (RMSNorm: sum x^2), so no
//    extra pass over the hidden states is made.
//  * The 8 waves of a workgroup sum their tiles pairwise in LDS in a fixed
//    order; the workgroup writes a compact row-major partial and its piece
//    statistics to the workspace with device-coherent stores.  The last
//    workgroup of a column block to arrive (atomic counter) combines the
//    statistics (exact shifted-sum algebra in float64), issues every
//    partial load of its outputs at once, sums the pieces in a fixed order
//    and resets the counter: the result is bitwise reproducible and the
//    workspace is ready for the next call.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

// A W row piece with the non-temporal hint: the stored weight is read once
// per call (the hidden-state rows, re-read across column groups, are not).
template <typename T>
__device__ __forceinline__ T load_w_nt(const uint16_t* p);
template <>
__device__ __forceinline__ uint4 load_w_nt<uint4>(const uint16_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ uint2 load_w_nt<uint2>(const uint16_t* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
}

constexpr int DW = 8;                           // waves per workgroup
constexpr int DTHREADS = 64 * DW;
constexpr int DECODE_MAX_KS = 8;                // K chunks per column block
constexpr int DECODE_SLOTS = 3;                 // piece slots per chunk
constexpr int PPS = 4;                          // pieces per state, at most (ks <= 8)

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

// rows of the A operand after the tokens: gamma and beta (LayerNorm)
template <int NORM>
__host__ __device__ constexpr int param_rows() { return NORM == NORM_LN ? 2 : 0; }

template <int NORM, int J, int MT>
__global__ __launch_bounds__(DTHREADS) void decode_kernel(DecodeArgs a) {
    constexpr int NW = 16 * J;
    constexpr int ROWS = 16 * MT;
    constexpr int FR = MT * J;            // f32x4 accumulators per lane
    constexpr int TILE = ROWS * NW;       // floats of one wave tile
    constexpr int RG = DTHREADS / NW;     // row groups of the reducer
    constexpr int MAXROWS = ROWS < DECODE_MAX_M ? ROWS : DECODE_MAX_M;
    constexpr int RPT = (MAXROWS + RG - 1) / RG;  // reducer rows per thread
    typedef typename RowVec<J>::T LT;
    constexpr int NL = 8;

    const int nb = a.nb, ks = a.kps, M = a.M, d = a.d;
    const int b = blockIdx.x % nb;
    const int c = blockIdx.x / nb;
    const int TS = d >> 5;
    const int T = 3 * TS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int n0 = b * NW;
    const int Mst = M + param_rows<NORM>();
    const uint16_t* __restrict__ W = a.W;

    // big: 4 wave tiles for the pairwise sums; reused for the row-major tile
    // and, in the reducer, for (mu - K_p) per piece
    constexpr int BIG = 4 * TILE;
    static_assert(BIG >= 3 * PPS * DECODE_MAX_M, "reducer scratch");
    __shared__ __attribute__((aligned(16))) float sh_big[BIG];
    __shared__ float sh_shift[DECODE_MAX_M];
    __shared__ float sh_s1[DW][DECODE_MAX_M];
    __shared__ float sh_s2[DW][DECODE_MAX_M];
    __shared__ float sh_r[3][DECODE_MAX_M];
    __shared__ int sh_last;

    // chunk c covers k-steps [t0c, t1c); piece pi is its part in state s_first + pi
    const int t0c = (c * T) / ks, t1c = ((c + 1) * T) / ks;
    const int s_first = t0c / TS;
    const int npieces = (t1c - 1) / TS - s_first + 1;
    // the tokens' source rows and valid mask (every wave holds all of them)
    const WaveRows wr = rv_wave(a.rv, M);

    for (int pi = 0; pi < npieces; ++pi) {
        const int s = s_first + pi;
        const int tp0 = max(t0c, s * TS), tp1 = min(t1c, (s + 1) * TS);
        const int seg_k0 = s * d;
        const uint16_t* __restrict__ hs = a.h[s];
        const uint16_t* __restrict__ gam = a.gamma[s];
        const uint16_t* __restrict__ bet = a.beta[s];
        const size_t lds = (size_t)rv_ld(a.rv, s);

        // ---- provisional shift per token row: mean of the piece's first 32 values
        const size_t shift_src = (size_t)rv_lane_src(a.rv, wr, (tid >> 2) & 63);  // (every lane, before the branch)
        if (NORM == NORM_LN && tid < 4 * DECODE_MAX_M) {
            const int m = tid >> 2;
            if (m < M) {
                const uint4 x =
                    *reinterpret_cast<const uint4*>(hs + shift_src * lds + (tp0 * 32 - seg_k0) + (tid & 3) * 8);
                float v = bf_lo(x.x) + bf_hi(x.x) + bf_lo(x.y) + bf_hi(x.y) + bf_lo(x.z) + bf_hi(x.z) +
                          bf_lo(x.w) + bf_hi(x.w);
                v = quad_sum(v);
                if ((tid & 3) == 0) sh_shift[m] = v * (1.0f / 32.0f);
            }
        }
        __syncthreads();

        // ---- per-lane role of each 16-row tile of the A operand, as bit masks:
        // token rows take the normalised x, row M gamma, row M+1 beta, others 0.
        // Non-token lanes load row 0 (always valid) and mask it away, so the hot
        // loop has no divergent branches.
        float shift[MT];
        uint32_t tok[MT], gmk[MT], bmk[MT];
        const uint16_t* arow[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const int m = 16 * tt + cb;
            const bool is_tok = m < M;
            tok[tt] = is_tok ? 0xffffffffu : 0u;
            gmk[tt] = (NORM == NORM_LN && m == M) ? 0xffffffffu : 0u;
            bmk[tt] = (NORM == NORM_LN && m == M + 1) ? 0xffffffffu : 0u;
            shift[tt] = (NORM == NORM_LN && is_tok) ? sh_shift[m] : 0.f;
            const size_t src = (size_t)rv_lane_src(a.rv, wr, min(m, 63));
            arow[tt] = hs + (is_tok ? src : 0) * lds - seg_k0 + 8 * g;
        }

        f32x4 acc[MT][J];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int j = 0; j < J; ++j) acc[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        float S1[MT], S2[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) S1[tt] = S2[tt] = 0.f;

        // W: 8 rows x J columns per lane.
        // W (the HBM stream) is prefetched one k-step ahead; the A fragments,
        // gamma and beta are L2 hits, loaded at the top of their own step.
        const uint16_t* wbase = W + (size_t)(8 * g) * d + n0 + J * cb;
        const size_t wstep = (size_t)32 * d;  // elements per k-step
        const size_t wsub = (size_t)d;        // elements between the NL loads
        const bool has_g = NORM != NORM_NONE && gam != nullptr;
        const bool has_b = NORM == NORM_LN && bet != nullptr;
        // missing gamma / beta read a valid row of h instead and are replaced by 1 / 0
        const uint16_t* gptr = (has_g ? gam : hs) - seg_k0 + 8 * g;
        const uint16_t* bptr = (has_b ? bet : hs) - seg_k0 + 8 * g;
        const uint32_t gsel = has_g ? 0xffffffffu : 0u;
        const uint32_t bsel = has_b ? 0xffffffffu : 0u;

        // Per k-step: (1) this step's A, gamma and beta loads (L2 hits);
        // (2) transpose of this step's W, loaded one step earlier; (3) the
        // next step's W, issued unconditionally (the last step re-reads its
        // own rows) so the outstanding-load count is static; (4) normalise
        // A and run the MFMAs, waiting only for (1).
        LT wr[NL];
        int t = tp0 + wave;
        if (t < tp1) {
            const uint16_t* wp = wbase + (size_t)t * wstep;
#pragma unroll
            for (int r = 0; r < NL; ++r) wr[r] = load_w_nt<LT>(wp + (size_t)r * wsub);
        }
        for (; t < tp1; t += DW) {
            const int k = t * 32;
            uint4 xr[MT];
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) xr[tt] = *reinterpret_cast<const uint4*>(arow[tt] + k);
            uint4 gr = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
            uint4 br = make_uint4(0u, 0u, 0u, 0u);
            if (NORM != NORM_NONE) {
                const uint4 gl = *reinterpret_cast<const uint4*>(gptr + k);
                gr = make_uint4((gl.x & gsel) | (0x3F803F80u & ~gsel), (gl.y & gsel) | (0x3F803F80u & ~gsel),
                                (gl.z & gsel) | (0x3F803F80u & ~gsel), (gl.w & gsel) | (0x3F803F80u & ~gsel));
            }
            if (NORM == NORM_LN) {
                const uint4 bl = *reinterpret_cast<const uint4*>(bptr + k);
                br = make_uint4(bl.x & bsel, bl.y & bsel, bl.z & bsel, bl.w & bsel);
            }
            __builtin_amdgcn_sched_barrier(0);

            // B operands: column j of the 8 x J block, 8 consecutive k
            uint4 bf[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                uint32_t q[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t r0 = RowVec<J>::dw(wr[2 * p], j >> 1);
                    const uint32_t r1 = RowVec<J>::dw(wr[2 * p + 1], j >> 1);
                    q[p] = (j & 1) ? ((r0 >> 16) | (r1 & 0xffff0000u)) : ((r0 & 0xffffu) | (r1 << 16));
                }
                bf[j] = make_uint4(q[0], q[1], q[2], q[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
            {
                const int tn = (t + DW) < tp1 ? t + DW : t;
                const uint16_t* wp = wbase + (size_t)tn * wstep;
#pragma unroll
                for (int r = 0; r < NL; ++r) wr[r] = load_w_nt<LT>(wp + (size_t)r * wsub);
            }
            __builtin_amdgcn_sched_barrier(0);

            float gf[8];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w = u4get(gr, p);
                gf[2 * p] = bf_lo(w);
                gf[2 * p + 1] = bf_hi(w);
            }
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) {
                uint32_t q[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t w = u4get(xr[tt], p) & tok[tt];
                    if (NORM == NORM_NONE) {
                        q[p] = w;
                    } else {
                        float x0 = bf_lo(w), x1 = bf_hi(w);
                        if (NORM == NORM_LN) {
                            x0 -= shift[tt];
                            x1 -= shift[tt];
                            S1[tt] += x0 + x1;
                        }
                        S2[tt] += x0 * x0 + x1 * x1;
                        const uint32_t pk = pack_bf2(x0 * gf[2 * p], x1 * gf[2 * p + 1]) & tok[tt];
                        q[p] = pk | (u4get(gr, p) & gmk[tt]) | (u4get(br, p) & bmk[tt]);
                    }
                }
                const uint4 af = make_uint4(q[0], q[1], q[2], q[3]);
#pragma unroll
                for (int j = 0; j < J; ++j) acc[tt][j] = mfma16x16x32(af, bf[j], acc[tt][j]);
            }

        }

        // ---- piece statistics: the 4 lane groups, then the waves (fixed order below)
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

        // ---- pairwise sum of the 8 wave tiles in fragment order:
        //      ((w0 + w4) + (w2 + w6)) + ((w1 + w5) + (w3 + w7))
        f32x4* buf = reinterpret_cast<f32x4*>(sh_big);
#pragma unroll
        for (int half = 4; half >= 1; half >>= 1) {
            if (wave >= half && wave < 2 * half) {
                f32x4* dst = buf + (wave - half) * FR * 64;
#pragma unroll
                for (int tt = 0; tt < MT; ++tt)
#pragma unroll
                    for (int j = 0; j < J; ++j) dst[(tt * J + j) * 64 + lane] = acc[tt][j];
            }
            __syncthreads();
            if (wave < half) {
                const f32x4* src = buf + wave * FR * 64;
#pragma unroll
                for (int tt = 0; tt < MT; ++tt)
#pragma unroll
                    for (int j = 0; j < J; ++j) acc[tt][j] += src[(tt * J + j) * 64 + lane];
            }
            __syncthreads();
        }
        // wave 0 holds the workgroup's tile; lay it out row-major for coalesced stores
        float* rowmaj = sh_big;
        if (wave == 0) {
#pragma unroll
            for (int tt = 0; tt < MT; ++tt)
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rowmaj[(16 * tt + 4 * g + e) * NW + J * cb + j] = acc[tt][j][e];
        }
        __syncthreads();

        const int slot = (b * ks + c) * DECODE_SLOTS + pi;
        float* part = a.part + (size_t)slot * TILE;
        for (int v = tid; v < Mst * NW; v += DTHREADS) store_coherent(part + v, rowmaj[v]);
        if (NORM != NORM_NONE) {
            float* st = a.stats + (size_t)slot * DECODE_MAX_M * 3;
            for (int m = tid; m < M; m += DTHREADS) {
                const float v1 = ((sh_s1[0][m] + sh_s1[4][m]) + (sh_s1[2][m] + sh_s1[6][m])) +
                                 ((sh_s1[1][m] + sh_s1[5][m]) + (sh_s1[3][m] + sh_s1[7][m]));
                const float v2 = ((sh_s2[0][m] + sh_s2[4][m]) + (sh_s2[2][m] + sh_s2[6][m])) +
                                 ((sh_s2[1][m] + sh_s2[5][m]) + (sh_s2[3][m] + sh_s2[7][m]));
                store_coherent(st + 3 * m + 0, NORM == NORM_LN ? sh_shift[m] : 0.f);
                store_coherent(st + 3 * m + 1, v1);
                store_coherent(st + 3 * m + 2, v2);
            }
        }
        __syncthreads();  // LDS is reused by the next piece
    }

    // Publish without cache maintenance: partials and statistics were
    // written with device-coherent (agent-scope atomic) stores; every wave
    // waits until they have completed (the workgroup barrier alone does not
    // wait for them), then thread 0 counts the workgroup in.  The last
    // arriver reads them with device-coherent loads.  (An agent-scope
    // release / acquire would write back / invalidate a whole L2.)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (old == ks - 1);
    }
    __syncthreads();
    if (!sh_last) return;

    // ================= last arriver of column block b =================
    // Pieces of this column block by state: state s is covered by chunks
    // chunk_of(s*TS) .. chunk_of((s+1)*TS - 1), at most PPS of them; every
    // table below is indexed by compile-time (s, q), so it lives in registers.
    auto chunk_of = [&](int tt) { return ((tt + 1) * ks - 1) / T; };
    int pslot[3][PPS], plen[3][PPS];
    bool pval[3][PPS];
#pragma unroll
    for (int ss = 0; ss < 3; ++ss) {
        const int c0 = chunk_of(ss * TS), c1 = chunk_of((ss + 1) * TS - 1);
#pragma unroll
        for (int q = 0; q < PPS; ++q) {
            const int cc = c0 + q;
            const int a0 = (cc * T) / ks, a1 = ((cc + 1) * T) / ks;
            pval[ss][q] = cc <= c1;
            pslot[ss][q] = pval[ss][q] ? (b * ks + cc) * DECODE_SLOTS + (ss - a0 / TS) : 0;
            plen[ss][q] = pval[ss][q] ? 32 * (min(a1, (ss + 1) * TS) - max(a0, ss * TS)) : 0;
        }
    }

    // statistics of every state and token (float64 combination of the pieces)
    float* sh_delta = sh_big;  // [3 * PPS][64]: mu_s - K_p
    for (int m = tid; m < M; m += DTHREADS) {
        // every state's piece records are loaded before any is used (one
        // round trip, not one per state)
        // (unconditional loads: a piece that does not exist reads slot 0,
        // inside the workspace, and its values are dropped; a load under a
        // branch would get a wait of its own)
        float Ka[3][PPS], s1a[3][PPS], s2a[3][PPS];
#pragma unroll
        for (int ss = 0; ss < 3; ++ss)
#pragma unroll
            for (int q = 0; q < PPS; ++q) {
                Ka[ss][q] = s1a[ss][q] = s2a[ss][q] = 0.f;
                if (NORM != NORM_NONE) {
                    const float* st = a.stats + ((size_t)pslot[ss][q] * DECODE_MAX_M + m) * 3;
                    Ka[ss][q] = load_coherent(st);
                    s1a[ss][q] = load_coherent(st + 1);
                    s2a[ss][q] = load_coherent(st + 2);
                }
            }
#pragma unroll
        for (int ss = 0; ss < 3; ++ss)
#pragma unroll
            for (int q = 0; q < PPS; ++q)
                if (!pval[ss][q]) Ka[ss][q] = s1a[ss][q] = s2a[ss][q] = 0.f;
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) {
            const float* K = Ka[ss];
            const float* s1 = s1a[ss];
            const float* s2 = s2a[ss];
            double r = 1.0, mu = 0.0;
            if (NORM == NORM_LN) {
                double sum = 0.0;
#pragma unroll
                for (int q = 0; q < PPS; ++q) sum += (double)plen[ss][q] * (double)K[q] + (double)s1[q];
                mu = sum / (double)d;
                double m2 = 0.0;
#pragma unroll
                for (int q = 0; q < PPS; ++q) {
                    const double dl = mu - (double)K[q];
                    if (pval[ss][q]) m2 += (double)s2[q] - 2.0 * dl * (double)s1[q] + (double)plen[ss][q] * dl * dl;
                    sh_delta[(ss * PPS + q) * DECODE_MAX_M + m] = (float)dl;
                }
                r = 1.0 / sqrt(m2 / (double)d + (double)a.eps);
            } else if (NORM == NORM_RMS) {
                double sq = 0.0;
#pragma unroll
                for (int q = 0; q < PPS; ++q) sq += (double)s2[q];
                r = 1.0 / sqrt(sq / (double)d + (double)a.eps);
            }
            sh_r[ss][m] = (float)r;
        }
    }
    __syncthreads();

    // outputs: thread -> column n, rows rg, rg + RG, ...; every load is issued first
    const int n = tid % NW;
    const int rg = tid / NW;
    float P[3][PPS][RPT];
    float U[3][PPS];
    float add = 0.f;
#pragma unroll
    for (int ss = 0; ss < 3; ++ss)
#pragma unroll
        for (int q = 0; q < PPS; ++q) {
            // unconditional loads (rows clamped, missing pieces read slot 0),
            // the values of rows and pieces that do not exist are dropped
            const float* base = a.part + (size_t)pslot[ss][q] * TILE;
            U[ss][q] = 0.f;
            if (NORM == NORM_LN) {
                const float uv = load_coherent(base + M * NW + n);
                const float av = load_coherent(base + (M + 1) * NW + n);
                U[ss][q] = pval[ss][q] ? uv : 0.f;
                add += pval[ss][q] ? av : 0.f;
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int m = rg + RG * i;
                const float pv = load_coherent(base + min(m, M - 1) * NW + n);
                P[ss][q][i] = (pval[ss][q] && m < M) ? pv : 0.f;
            }
        }
    if (a.bias != nullptr) add += bf_one(a.bias[n0 + n]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int m = rg + RG * i;
        if (m >= M) continue;
        float y = 0.f;
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) {
            float ys = 0.f;
#pragma unroll
            for (int q = 0; q < PPS; ++q) {
                float v = P[ss][q][i];
                if (NORM == NORM_LN) v -= sh_delta[(ss * PPS + q) * DECODE_MAX_M + m] * U[ss][q];
                ys += v;
            }
            y += (NORM == NORM_NONE) ? ys : sh_r[ss][m] * ys;
        }
        a.out[(size_t)m * (size_t)a.rv.ld_out + n0 + n] =
            rv_ok(wr, m) ? __builtin_bit_cast(uint16_t, (__bf16)(y + add)) : (uint16_t)0;
    }
    if (tid == 0) __hip_atomic_store(a.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// =====================================================================
// One token on the stored W: normalise first, then a VALU GEMV
// =====================================================================
//
// With one token the normalised activation is a vector of 3d floats, so it
// is computed exactly (fp32) before the contraction and no state boundary or
// fold is involved: out = xn . W + bias, xn = [n(h_low) | n(h_mid) | n(h_high)].
// Workgroup (group g, chunk c) owns columns [512 g, 512 g + 512) -- 1 KiB of
// every row of W -- and K rows [c R, c R + R).  It computes the three rows'
// statistics itself (shifted sums, one wave per row), writes its xn rows to
// LDS, then wave w takes rows w, w + 8, ...: each load instruction is one
// contiguous 1 KiB piece of a row (lane l: columns 8 l .. 8 l + 7), 8 fp32
// FMAs per row and lane.  The waves' sums are added in wave order and the
// chunks of a group in chunk order by the last to arrive (device-coherent
// partials and counter, as in the other decode kernels): the result is
// bitwise reproducible.
constexpr int ONE_ROWS_MAX = 16384;  // K rows per chunk (64 KiB of fp32 in LDS)
constexpr int ONE_XP = 4;            // xn rows per thread whose values are loaded before the W ring
constexpr int ONE_MAXKC = 72;        // K chunks of a column group, at most (d = 1536 takes 72)

// The row's shift piece and first batch (4096 values), loaded by the caller
// ahead of its other loads (they complete in issue order)
struct OneRowPre {
    uint4 k;
    uint4 x[8];
};
__device__ __forceinline__ void one_row_preload(const uint16_t* row, int d, int lane, OneRowPre& pre) {
    pre.k = *reinterpret_cast<const uint4*>(row + 8 * (lane & 3));
    const int nchunk = d >> 3;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int c = lane + 64 * q;
        pre.x[q] = c < nchunk ? *reinterpret_cast<const uint4*>(row + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void one_row_sums(const uint16_t* row, int d, int lane, bool shift, const OneRowPre& pre,
                                             float& K, float& S1, float& S2) {
    K = 0.f;
    if (shift) {
        const uint4 x = pre.k;
        float v = ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
                  ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
        v = quad_sum(v);
        K = v * (1.0f / 32.0f);
    }
    // chunks lane, lane + 64, ... in order; the 8 loads of a batch are
    // issued before any is used (one round trip per 4096 values; the first
    // batch is the preloaded one)
    float s1 = 0.f, s2 = 0.f;
    const int nchunk = d >> 3;
    auto batch = [&](const uint4 (&x)[8], int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (c0 + lane + 64 * q >= nchunk) continue;
            const uint32_t w4[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = bf_lo(w4[e]) - K, x1 = bf_hi(w4[e]) - K;
                s1 += x0 + x1;
                s2 = fmaf(x0, x0, fmaf(x1, x1, s2));
            }
        }
    };
    batch(pre.x, 0);
    for (int c0 = 512; c0 < nchunk; c0 += 512) {
        uint4 x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = c0 + lane + 64 * q;
            x[q] = c < nchunk ? *reinterpret_cast<const uint4*>(row + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
        }
        batch(x, c0);
    }
    S1 = wave_sum(s1);
    S2 = wave_sum(s2);
}

template <int NORM>
__global__ __launch_bounds__(512) void decode_one_kernel(DecodeArgs a) {
    constexpr int R = 8;  // load ring (one 8-row x 128-byte load per step)
    __shared__ float xn[ONE_ROWS_MAX];
    __shared__ float st[3][2];       // mu, rstd per state
    __shared__ float red[8][512];
    __shared__ int sh_last;
    const int d = a.d, ngroups = a.nb, nkc = a.kps;
    const int rows = 3 * d / nkc;    // a multiple of 64 (8 waves x an 8-row ring)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per = (ngroups * nkc + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (lin >= ngroups * nkc) return;
    const int grp = lin / nkc, kc = lin - grp * nkc;
    const int n0 = 512 * grp, k0 = kc * rows;

    // the token's source row (an invalid index reads row 0; the output is zeros)
    bool tok_ok;
    const size_t src0 = (size_t)rv_src(a.rv, 0, tok_ok);
    // Loads complete in issue order, so the ones waited on first go out
    // first: the statistics rows (waves 0..2), this chunk's token values and
    // their gamma and beta (rows tid + 512 j, clamped: a load under a branch
    // would wait for itself), and the bias; then the W ring.
    OneRowPre pre;
    if (NORM != NORM_NONE && wave < 3) one_row_preload(a.h[wave] + src0 * (size_t)rv_ld(a.rv, wave), d, lane, pre);
    uint16_t xh[ONE_XP], xg[ONE_XP], xb[ONE_XP];
#pragma unroll
    for (int j = 0; j < ONE_XP; ++j) {
        const int k = k0 + min(tid + 512 * j, rows - 1), s = k / d, kk = k - s * d;
        xh[j] = ((s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2])) + src0 * (size_t)rv_ld(a.rv, s))[kk];
        xg[j] = xb[j] = 0;
        if (NORM != NORM_NONE) {
            const uint16_t* gs = s == 0 ? a.gamma[0] : (s == 1 ? a.gamma[1] : a.gamma[2]);
            xg[j] = gs ? gs[kk] : (uint16_t)0x3f80;  // bf16 1.0
            if (NORM == NORM_LN) {
                const uint16_t* bs = s == 0 ? a.beta[0] : (s == 1 ? a.beta[1] : a.beta[2]);
                xb[j] = bs ? bs[kk] : (uint16_t)0;
            }
        }
    }
    const float bias_n = a.bias ? bf_one(a.bias[n0 + tid]) : 0.f;

    // this wave's W rows: k0 + wave + 8 i, columns n0 + 8 lane .. + 7
    const uint16_t* __restrict__ wp = a.W + (size_t)(k0 + wave) * d + n0 + 8 * lane;
    const size_t wstep = (size_t)8 * d;
    const int nsteps = rows / 8;     // a multiple of R
    uint4 rw[R];
#pragma unroll
    for (int p = 0; p < R; ++p) rw[p] = load_w_nt<uint4>(wp + (size_t)p * wstep);

    // statistics of the three rows (waves 0..2)
    if (NORM != NORM_NONE && wave < 3) {
        float K, S1, S2;
        one_row_sums(a.h[wave] + src0 * (size_t)rv_ld(a.rv, wave), d, lane, NORM == NORM_LN, pre, K, S1, S2);
        if (lane == 0) {
            const float inv_d = 1.0f / (float)d;
            float mu = 0.f, rstd;
            if (NORM == NORM_LN) {
                const float dm = S1 * inv_d;
                mu = K + dm;
                rstd = 1.0f / sqrtf(fmaxf(S2 * inv_d - dm * dm, 0.f) + a.eps);
            } else {
                rstd = 1.0f / sqrtf(S2 * inv_d + a.eps);
            }
            st[wave][0] = mu;
            st[wave][1] = rstd;
        }
    }
    __syncthreads();
    // xn of this chunk's rows, in fp32: the first ONE_XP rows per thread from
    // the values loaded up front, any further ones loaded here
#pragma unroll
    for (int j = 0; j < ONE_XP; ++j) {
        const int r = tid + 512 * j;
        if (r >= rows) break;
        const int s = (k0 + r) / d;
        float x = bf_one(xh[j]);
        if (NORM != NORM_NONE) {
            x = (x - st[s][0]) * st[s][1] * bf_one(xg[j]);
            if (NORM == NORM_LN) {
                const uint16_t* bs = s == 0 ? a.beta[0] : (s == 1 ? a.beta[1] : a.beta[2]);
                if (bs) x += bf_one(xb[j]);
            }
        }
        xn[r] = x;
    }
    for (int r = tid + 512 * ONE_XP; r < rows; r += 512) {
        const int k = k0 + r, s = k / d, kk = k - s * d;
        const uint16_t* hs = (s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2])) + src0 * (size_t)rv_ld(a.rv, s);
        float x = bf_one(hs[kk]);
        if (NORM != NORM_NONE) {
            const uint16_t* gs = s == 0 ? a.gamma[0] : (s == 1 ? a.gamma[1] : a.gamma[2]);
            const float gm = gs ? bf_one(gs[kk]) : 1.f;
            x = (x - st[s][0]) * st[s][1] * gm;
            if (NORM == NORM_LN) {
                const uint16_t* bs = s == 0 ? a.beta[0] : (s == 1 ? a.beta[1] : a.beta[2]);
                if (bs) x += bf_one(bs[kk]);
            }
        }
        xn[r] = x;
    }
    __syncthreads();

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const float* xr = xn + wave;
    auto fma_row = [&](const uint4& w, float x) __attribute__((always_inline)) {
        const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaf(x, bf_lo(w4[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(x, bf_hi(w4[e]), acc[2 * e + 1]);
        }
    };
    int i = 0;
    for (; i < nsteps - R; i += R) {
#pragma unroll
        for (int p = 0; p < R; ++p) {
            fma_row(rw[p], xr[(i + p) * 8]);
            rw[p] = load_w_nt<uint4>(wp + (size_t)(i + p + R) * wstep);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int p = 0; p < R; ++p) fma_row(rw[p], xr[(i + p) * 8]);

#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][8 * lane + e] = acc[e];
    __syncthreads();
    // thread t < 512: column n0 + t, the waves' sums in wave order
    float* part = a.part + ((size_t)grp * nkc + kc) * 512;
    {
        float v = red[0][tid];
#pragma unroll
        for (int w = 1; w < 8; ++w) v += red[w][tid];
        store_coherent(part + tid, v);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (old == nkc - 1);
    }
    __syncthreads();
    if (!sh_last) return;
    {
        // chunks summed in order; every chunk's load is issued before any is
        // used (indexes past nkc re-read the last chunk and are dropped), so
        // the sum costs one round trip
        const float* gp = a.part + (size_t)grp * nkc * 512 + tid;
        float y = 0.f;
        auto sum_chunks = [&](auto nmax) __attribute__((always_inline)) {
            constexpr int NK = decltype(nmax)::value;
            float v[NK];
#pragma unroll
            for (int q = 0; q < NK; ++q) v[q] = load_coherent(gp + (size_t)min(q, nkc - 1) * 512);
#pragma unroll
            for (int q = 0; q < NK; ++q)
                if (q < nkc) y += v[q];
        };
        if (nkc <= 16)
            sum_chunks(std::integral_constant<int, 16>());
        else if (nkc <= 32)
            sum_chunks(std::integral_constant<int, 32>());
        else if (nkc <= 48)
            sum_chunks(std::integral_constant<int, 48>());
        else
            sum_chunks(std::integral_constant<int, ONE_MAXKC>());
        if (a.bias) y += bias_n;
        a.out[n0 + tid] = tok_ok ? (uint16_t)(pack_bf2(y, 0.f) & 0xffffu) : (uint16_t)0;
    }
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

DecodePlan plan_decode(int M, int d, int norm) {
    DecodePlan p;
    // one token: the VALU kernel, 512-column groups x K chunks, the most
    // workgroups up to one per CU, each wave a multiple of 8 load steps
    if (M == 1 && d % 512 == 0) {
        const int ngroups = d / 512;
        int best = 0;
        for (int nkc = 1; nkc <= 256 && ngroups * nkc <= 256; ++nkc) {
            if ((3 * d) % (nkc * 64) != 0) continue;  // rows per chunk: 8 waves x a multiple of 8 steps
            if (3 * d / nkc > ONE_ROWS_MAX) continue;
            if (nkc > ONE_MAXKC) break;
            best = nkc;
        }
        if (best) {
            p.one = 1;
            p.nb = ngroups;
            p.kps = best;
            p.counters_bytes = ((size_t)ngroups * sizeof(int) + 255) / 256 * 256;
            p.stats_bytes = 256;
            p.part_bytes = ((size_t)ngroups * best * 512 * sizeof(float) + 255) / 256 * 256;
            return p;
        }
    }
    const int rows = M + (norm == NORM_LN ? 2 : 0);
    p.MT = (rows + 15) / 16;
    p.J = p.MT <= 2 ? 8 : 4;
    if (d % (16 * p.J) != 0) p.J = 4;
    p.nb = d / (16 * p.J);
    const int T = 3 * (d / 32);
    // about one 8-wave workgroup per CU, each wave at least two k-steps per chunk
    int ks = (256 + p.nb / 2) / p.nb;
    if (ks < 1) ks = 1;
    if (ks > DECODE_MAX_KS) ks = DECODE_MAX_KS;
    while (ks > 1 && T / ks < 2 * DW) --ks;
    p.kps = ks;
    const size_t slots = (size_t)p.nb * ks * DECODE_SLOTS;
    p.counters_bytes = ((size_t)p.nb * sizeof(int) + 255) / 256 * 256;
    p.stats_bytes = (slots * DECODE_MAX_M * 3 * sizeof(float) + 255) / 256 * 256;
    p.part_bytes = (slots * (size_t)p.MT * 16 * 16 * p.J * sizeof(float) + 255) / 256 * 256;
    return p;
}

template <int NORM, int J, int MT>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    const int grid = a.nb * a.kps;
    decode_kernel<NORM, J, MT><<<grid, DTHREADS, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM>
static hipError_t launch_decode_n(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    switch (p.MT) {
        case 1: return p.J == 8 ? launch_decode_t<NORM, 8, 1>(a, st) : launch_decode_t<NORM, 4, 1>(a, st);
        case 2: return p.J == 8 ? launch_decode_t<NORM, 8, 2>(a, st) : launch_decode_t<NORM, 4, 2>(a, st);
        case 3: return launch_decode_t<NORM, 4, 3>(a, st);
        case 4: return launch_decode_t<NORM, 4, 4>(a, st);
        case 5: return launch_decode_t<NORM, 4, 5>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NORM>
static hipError_t launch_one(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    const int grid = ((p.nb * p.kps + 7) / 8) * 8;
    decode_one_kernel<NORM><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int norm, const DecodePlan& p, hipStream_t st) {
    if (p.one) {
        if (a.M != 1 || a.nb != p.nb || a.kps != p.kps || a.d != 512 * p.nb || (3 * a.d) % (p.kps * 64) ||
            3 * a.d / p.kps > ONE_ROWS_MAX || p.kps > ONE_MAXKC)
            return hipErrorInvalidValue;
        if (norm == NORM_LN) return launch_one<NORM_LN>(a, p, st);
        if (norm == NORM_RMS) return launch_one<NORM_RMS>(a, p, st);
        return launch_one<NORM_NONE>(a, p, st);
    }
    if (norm == NORM_LN) return launch_decode_n<NORM_LN>(a, p, st);
    if (norm == NORM_RMS) return launch_decode_n<NORM_RMS>(a, p, st);
    return launch_decode_n<NORM_NONE>(a, p, st);
}

}  // namespace e31
