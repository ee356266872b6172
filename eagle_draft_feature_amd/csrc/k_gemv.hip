// Decode path of the fused per-state norm + FC on the folded weight (M <= 64).
//
// With the norm parameters folded into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the LayerNorm parameters are absorbed
// into the FC), the output is
//     out = sum_s rstd_s * (P_s - mu_s * u_s) + c,   P_s = h_s . W'_s,
// so the raw hidden states feed the matrix cores and the step is one pass
// over W' (3d x d bf16): HBM-bound for few tokens.
//
// W' is stored as 1 KiB tiles in MFMA B-fragment order (16 columns x 32 k,
// lane l's 8 values at bytes [16 l, 16 l + 16)), the tiles of one 16-column
// block consecutive along k.
//
// Work split: workgroup (g, c) owns the 64 columns of column group g (four
// column blocks) and K chunk c, a piece of one state: a state's d/32 k-steps
// are cut into kps chunks.  Wave w of NW (8, fewer for small d) takes the
// chunk's steps w, w + NW, ...;
// at each step it loads four W' tiles (one per column block, each a
// contiguous 1 KiB) and the A fragments of its 16*MT token rows, and runs
// 4*MT MFMAs, so every A fragment serves 64 columns from registers.  W' is
// prefetched R steps ahead, A RA steps ahead, in register rings with static
// slots (the chunk is one state, so every pointer is fixed per wave).
//
// Statistics come from the same A fragments: each lane keeps shifted sums
// S1 = sum (x - K), S2 = sum (x - K)^2 (RMSNorm: sum x^2), with K one shift
// per token and chunk (the mean of the chunk's first 32 values of that row,
// equal in every wave), so the chunk's sums combine exactly and no separate
// statistics pass is needed.
//
// Each workgroup sums its waves' tiles pairwise in LDS in a fixed order and
// writes a row-major fp32 partial and its chunk statistics to the workspace.
// The last workgroup of a column group to arrive (atomic counter) combines
// the statistics of each state in float64 (exact shifted-sum algebra), sums
// the chunk partials in a fixed order, applies rstd_s, mu_s u_s and c,
// stores bf16 and resets the counter: the result is bitwise reproducible and
// the workspace is ready for the next call.  Token rows beyond M read row
// M-1 and are never stored.
//
// Cross-workgroup handoff without cache maintenance: the L2 of an XCD is
// not coherent with the others, and an agent-scope release / acquire fence
// writes back / invalidates a whole L2, a cost of microseconds per
// workgroup.  Instead every value handed over (partials, statistics) is
// written and read with agent-scope atomic (relaxed) stores and loads, which
// go to the device coherence point; the writer waits for its stores to
// complete (s_waitcnt) before the workgroup barrier and the counter
// increment, and the reader issues its loads only after it has seen the
// final count.
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int GV_WAVES = 8;          // waves per workgroup, at most
constexpr int GV_THREADS = 64 * GV_WAVES;
constexpr int GV_NB = 4;             // column blocks per workgroup (64 columns)

template <int NORM, int MT, int R, int RA>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(GemvArgs a) {
    constexpr int ROWS = 16 * MT;
    constexpr int TILE_F4 = GV_NB * MT * 64;  // f32x4 per wave tile
    const int M = a.M, d = a.d;
    const int ngroups = d >> 6;
    const int nchunks = 3 * a.kps;
    const int nwg = ngroups * nchunks;
    // XCD-aware order: consecutive workgroup ids go round robin over the 8
    // XCDs; each XCD takes a contiguous range of (group, chunk) pairs, so the
    // chunks of a column group tend to share an L2
    const int per = (nwg + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (lin >= nwg) return;
    const int grp = lin / nchunks, ch = lin - grp * nchunks;
    const int s = ch / a.kps, q = ch - s * a.kps;
    const int T3 = d >> 5;                 // k-steps per state
    const int TC = T3 / a.kps;             // k-steps per chunk
    const int tc0 = q * TC;                // first step of the chunk inside the state
    const int NW = a.waves;                // waves of this workgroup
    const int nw = TC / NW;                // this wave's steps (a multiple of R)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const uint16_t* __restrict__ hs = s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2]);

    // W' tiles of column block 4 grp + b, k-step s T3 + tc0 + wave + NW i
    const uint4* __restrict__ wp = reinterpret_cast<const uint4*>(a.wp) +
                                   ((size_t)(GV_NB * grp) * 3 * T3 + (size_t)s * T3 + tc0 + wave) * 64 + lane;
    const size_t wblk = (size_t)3 * T3 * 64;       // uint4 between column blocks
    const size_t wstep = (size_t)NW * 64;          // uint4 between a wave's steps
    // A fragments: row 16 tt + cb (clamped), k = (tc0 + wave + NW i) * 32 + 8 g
    const uint16_t* ap[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const int m = min(16 * tt + cb, M - 1);
        ap[tt] = hs + (size_t)m * d + (size_t)(tc0 + wave) * 32 + 8 * g;
    }
    const int ASTEP = NW * 32;  // elements between a wave's steps

    // shift per token row: mean of the chunk's first 32 values
    float kshift[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        kshift[tt] = 0.f;
        if (NORM == NORM_LN) {
            const int m = min(16 * tt + cb, M - 1);
            const uint4 x = *reinterpret_cast<const uint4*>(hs + (size_t)m * d + (size_t)tc0 * 32 + 8 * g);
            const float v = ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
                            ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
            kshift[tt] = group4_sum(v) * (1.0f / 32.0f);
        }
    }
    float S1[MT], S2[MT];
    f32x4 acc[GV_NB][MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        S1[tt] = S2[tt] = 0.f;
#pragma unroll
        for (int b = 0; b < GV_NB; ++b) acc[b][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    uint4 rw[R][GV_NB];
    uint4 rx[RA][MT];
    auto wload = [&](int i, uint4 (&w)[GV_NB]) {
#pragma unroll
        for (int b = 0; b < GV_NB; ++b) w[b] = wp[(size_t)b * wblk + (size_t)i * wstep];
    };
    auto aload = [&](int i, uint4 (&x)[MT]) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) x[tt] = *reinterpret_cast<const uint4*>(ap[tt] + (size_t)i * ASTEP);
    };
    // prologue in the steady-state issue order (as if steps -R .. -1 had
    // run), so the waits at the loop head equal those inside the loop
#pragma unroll
    for (int p = 0; p < R; ++p) {
        wload(p, rw[p]);
        if (p >= R - RA) aload(p - (R - RA), rx[p - (R - RA)]);
        __builtin_amdgcn_sched_barrier(0);
    }

    auto consume = [&](int p) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int b = 0; b < GV_NB; ++b) acc[b][tt] = mfma16x16x32(rx[p % RA][tt], rw[p][b], acc[b][tt]);
        if (NORM != NORM_NONE) {
#pragma unroll
            for (int tt = 0; tt < MT; ++tt) {
                const uint4 xv = rx[p % RA][tt];
                const uint32_t v[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x0 = bf_lo(v[e]), x1 = bf_hi(v[e]);
                    if (NORM == NORM_LN) {
                        x0 -= kshift[tt];
                        x1 -= kshift[tt];
                        S1[tt] += x0 + x1;
                    }
                    S2[tt] = fmaf(x0, x0, fmaf(x1, x1, S2[tt]));
                }
            }
        }
    };
    // full blocks refill their slots R / RA steps ahead; the last block
    // issues only the refills that stay inside the chunk
    int i = 0;
    for (; i < nw - R; i += R) {
#pragma unroll
        for (int p = 0; p < R; ++p) {
            consume(p);
            wload(i + p + R, rw[p]);
            aload(i + p + RA, rx[p % RA]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int p = 0; p < R; ++p) {
        consume(p);
        if (p + RA < R) aload(i + p + RA, rx[p % RA]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- chunk statistics per token row: 4 lane groups, then the waves
    __shared__ float sh_k[ROWS];
    __shared__ float sh_s[GV_WAVES][2][ROWS];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const float t1 = group4_sum(S1[tt]);
        const float t2 = group4_sum(S2[tt]);
        if (g == 0) {
            sh_s[wave][0][16 * tt + cb] = t1;
            sh_s[wave][1][16 * tt + cb] = t2;
            if (wave == 0) sh_k[16 * tt + cb] = kshift[tt];
        }
    }

    // ---- pairwise sum of the wave tiles, e.g. for 8 waves
    //      ((w0+w4)+(w2+w6))+((w1+w5)+(w3+w7))
    __shared__ __attribute__((aligned(16))) f32x4 buf[GV_WAVES / 2][TILE_F4];
    for (int half = NW / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int b = 0; b < GV_NB; ++b)
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) buf[wave - half][(b * MT + tt) * 64 + lane] = acc[b][tt];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int b = 0; b < GV_NB; ++b)
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) acc[b][tt] += buf[wave][(b * MT + tt) * 64 + lane];
        }
        __syncthreads();
    }
    // wave 0 lays the tile out row-major [ROWS][64] for coalesced stores
    // (a single wave has not passed a barrier yet: make the stats visible)
    if (NW == 1) __syncthreads();
    __shared__ __attribute__((aligned(16))) float rowmaj[ROWS * 64];
    if (wave == 0) {
#pragma unroll
        for (int b = 0; b < GV_NB; ++b)
#pragma unroll
            for (int tt = 0; tt < MT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) rowmaj[(16 * tt + 4 * g + e) * 64 + 16 * b + cb] = acc[b][tt][e];
    }
    __syncthreads();

    const size_t slot = (size_t)grp * nchunks + ch;
    float* part = a.part + slot * (size_t)ROWS * 64;
    const int nthreads = 64 * NW;
    for (int v = tid; v < M * 64; v += nthreads) store_coherent(part + v, rowmaj[v]);
    if (NORM != NORM_NONE) {
        float* st = a.stats + slot * (size_t)DECODE_MAX_M * 3;
        for (int m = tid; m < M; m += nthreads) {
            float v1 = 0.f, v2 = 0.f;
            for (int w = 0; w < NW; ++w) {
                v1 += sh_s[w][0][m];
                v2 += sh_s[w][1][m];
            }
            store_coherent(st + 3 * m + 0, sh_k[m]);
            store_coherent(st + 3 * m + 1, v1);
            store_coherent(st + 3 * m + 2, v2);
        }
    }

    // Publish: every wave waits until its coherent stores have completed
    // (the workgroup barrier alone does not wait for them), then thread 0
    // counts the workgroup in.
    __shared__ int sh_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (old == nchunks - 1);
    }
    __syncthreads();
    if (!sh_last) return;

    // ================= last arriver of column group grp =================
    // statistics of every state and token (float64 combination of the chunks)
    __shared__ float sh_r[3][DECODE_MAX_M];
    __shared__ float sh_mu[3][DECODE_MAX_M];
    const int kps = a.kps;
    const double clen = 32.0 * (double)TC;  // values per chunk
    for (int m = tid; m < M; m += nthreads) {
        for (int ss = 0; ss < 3; ++ss) {
            const float* st0 = a.stats + ((size_t)grp * nchunks + ss * kps) * DECODE_MAX_M * 3 + 3 * m;
            double r = 1.0, mu = 0.0;
            if (NORM == NORM_LN) {
                double sum = 0.0;
                for (int qq = 0; qq < kps; ++qq) {
                    const float* st = st0 + (size_t)qq * DECODE_MAX_M * 3;
                    sum += clen * (double)load_coherent(st) + (double)load_coherent(st + 1);
                }
                mu = sum / (double)d;
                double m2 = 0.0;
                for (int qq = 0; qq < kps; ++qq) {
                    const float* st = st0 + (size_t)qq * DECODE_MAX_M * 3;
                    const double dl = mu - (double)load_coherent(st);
                    m2 += (double)load_coherent(st + 2) - 2.0 * dl * (double)load_coherent(st + 1) + clen * dl * dl;
                }
                r = 1.0 / sqrt(m2 / (double)d + (double)a.eps);
            } else if (NORM == NORM_RMS) {
                double sq = 0.0;
                for (int qq = 0; qq < kps; ++qq) sq += (double)load_coherent(st0 + (size_t)qq * DECODE_MAX_M * 3 + 2);
                r = 1.0 / sqrt(sq / (double)d + (double)a.eps);
            }
            sh_r[ss][m] = (float)r;
            sh_mu[ss][m] = (float)mu;
        }
    }
    __syncthreads();

    // outputs: thread -> column n (64 per group), rows rg, rg + NW, ...
    const int nl = tid & 63, rg = tid >> 6;
    const int n = grp * 64 + nl;
    float us[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN)
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) us[ss] = a.u[(size_t)ss * d + n];
    const float cn = a.c[n];
    for (int m = rg; m < M; m += NW) {
        float y = cn;
        for (int ss = 0; ss < 3; ++ss) {
            float ps = 0.f;
            for (int qq = 0; qq < kps; ++qq)
                ps += load_coherent(a.part + ((size_t)grp * nchunks + ss * kps + qq) * (size_t)ROWS * 64 +
                                    (size_t)m * 64 + nl);
            if (NORM == NORM_LN) ps -= sh_mu[ss][m] * us[ss];
            y += (NORM == NORM_NONE) ? ps : sh_r[ss][m] * ps;
        }
        a.out[(size_t)m * d + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
    }
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- host side
GemvPlan plan_gemv(int M, int d) {
    GemvPlan p;
    p.MT = (M + 15) / 16;
    const int T3 = d / 32;
    const int ngroups = d / 64;
    // the most waves (8, 4, 2, 1) that split a chunk evenly; then the chunks
    // per state that bring the workgroup count nearest one per CU, each wave
    // taking a multiple of the ring depth (4, else 2, else 1) of steps
    int best = -1;
    for (int waves : {8, 4, 2, 1}) {
        for (int kps : {1, 2, 4, 8}) {
            if (T3 % (kps * waves)) continue;
            const int nw = T3 / (kps * waves);
            const int ring = nw % 4 == 0 ? 4 : (nw % 2 == 0 ? 2 : 1);
            const int grid = ngroups * 3 * kps;
            const int score = std::abs(grid - 256) + (ring < 4 ? 64 : 0);
            if (best < 0 || score < best) {
                best = score;
                p.kps = kps;
                p.ring = ring;
                p.waves = waves;
            }
        }
        if (best >= 0) break;
    }
    p.grid = ngroups * 3 * p.kps;
    p.counters_bytes = ((size_t)ngroups * sizeof(int) + 255) / 256 * 256;
    const size_t slots = (size_t)ngroups * 3 * p.kps;
    p.stats_bytes = (slots * DECODE_MAX_M * 3 * sizeof(float) + 255) / 256 * 256;
    p.part_bytes = (slots * (size_t)p.MT * 16 * 64 * sizeof(float) + 255) / 256 * 256;
    return p;
}

template <int NORM, int MT, int R>
static hipError_t launch_g(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    // A ring: as deep as W's, but two steps for three or four token tiles
    // (registers)
    constexpr int RA = (MT >= 3 && R > 2) ? 2 : R;
    const int grid = ((p.grid + 7) / 8) * 8;
    gemv_kernel<NORM, MT, R, RA><<<grid, 64 * p.waves, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM, int MT>
static hipError_t launch_gr(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.ring) {
        case 4: return launch_g<NORM, MT, 4>(a, p, st);
        case 2: return launch_g<NORM, MT, 2>(a, p, st);
        case 1: return launch_g<NORM, MT, 1>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NORM>
static hipError_t launch_gn(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.MT) {
        case 1: return launch_gr<NORM, 1>(a, p, st);
        case 2: return launch_gr<NORM, 2>(a, p, st);
        case 3: return launch_gr<NORM, 3>(a, p, st);
        case 4: return launch_gr<NORM, 4>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const GemvArgs& a, int norm, const GemvPlan& p, hipStream_t st) {
    if (p.kps < 1 || a.kps != p.kps || a.waves != p.waves || a.M < 1 || a.M > DECODE_MAX_M)
        return hipErrorInvalidValue;
    if (norm == NORM_LN) return launch_gn<NORM_LN>(a, p, st);
    if (norm == NORM_RMS) return launch_gn<NORM_RMS>(a, p, st);
    return launch_gn<NORM_NONE>(a, p, st);
}

}  // namespace e31
