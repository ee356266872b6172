// Prefill path of the fused per-state norm + FC (many tokens): a bf16 MFMA
// GEMM on the raw hidden states and the folded weight W'.
//
// With the norm parameters folded into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the parameters are absorbed by the FC),
//     out = sum_s rstd_s * (h_s . W'_s^T - mu_s * u_s) + c,
// so the main loop is a plain GEMM over the three states in turn, and the normalisation is a per-row rescale of the
// accumulator at each state boundary:
//     acc <- (acc - mu_s * u_s) * rstd_s / rstd_{s+1},
// finished by acc <- (acc - mu_2 * u_2) * rstd_2 + c.  The statistics come
// from the row-statistics pass that runs first.
//
// Tiling for gfx950: 256 x 256 output tile, BK = 64, 512 threads (8 waves as
// 2 x 4, each wave 128 x 64 = 8 x 4 MFMA 16x16x32 blocks), operand tiles
// double-buffered in LDS (2 x 64 KiB).  A (hidden states, row-major) is
// staged with a 16-byte XOR swizzle so the 16 lanes reading one k-chunk of
// 16 rows hit distinct banks; W' arrives as 1 KiB MFMA B-fragment tiles
// (16 columns x 32 k, lane l's operand at bytes [16 l, 16 l + 16)), copied
// to LDS as they are, so a B operand is one conflict-free 16-byte read.  Tiles are
// walked in groups of 4 M-tiles, and consecutive workgroup ids are spread so
// that each XCD (workgroup id mod 8) takes a contiguous run of that order:
// the 32 tiles an XCD runs at once share A and B tiles in its L2.
// Few tiles (small M) split K by chunks that never cross a state; partials go
// to a workspace and the last workgroup of a tile sums them in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int PBM = 256, PBN = 256, PBK = 64, PTH = 512;
constexpr int PGM = 4;  // M-tiles per raster group
constexpr int STAGE_U4 = (PBM + PBN) * PBK / 8;  // uint4 per LDS stage (A then B)

struct TileCoord {
    int mt, nt, chunk;
    bool valid;
};

__device__ __forceinline__ TileCoord map_tile(int bid, int TM, int TN, int splits) {
    TileCoord tc;
    const int NI = TM * TN * splits;
    const int P = (NI + 7) / 8;
    const int L = (bid % 8) * P + bid / 8;
    tc.valid = L < NI;
    const int tile = L / splits;
    tc.chunk = L - tile * splits;
    const int group = tile / (PGM * TN);
    const int first_m = group * PGM;
    const int gsz = min(TM - first_m, PGM);
    const int within = tile - group * PGM * TN;
    tc.mt = first_m + within % gsz;
    tc.nt = within / gsz;
    return tc;
}

template <bool SPLIT, int NORM>
__global__ __launch_bounds__(PTH, 1) void prefill_kernel(PrefillArgs a, int TM, int TN) {
    __shared__ __attribute__((aligned(16))) uint4 lds[2 * STAGE_U4];
    // per-row factors of the tile: mu_0, rstd_0/rstd_1, mu_1, rstd_1/rstd_2, mu_2, rstd_2
    // per-column factors: u_0, u_1, u_2, c
    __shared__ float rowf[6][PBM];
    __shared__ float colf[4][PBN];

    const TileCoord tc = map_tile(blockIdx.x, TM, TN, SPLIT ? a.splits : 1);
    if (!tc.valid) return;
    const int M = a.M, d = a.d;
    const size_t K3 = (size_t)3 * d;
    const int m0 = tc.mt * PBM, n0 = tc.nt * PBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int KTS = d / PBK;  // k-tiles per state
    int kt0 = 0, kt1 = 3 * KTS;
    if (SPLIT) {
        const int kps = a.splits / 3;
        const int s = tc.chunk / kps, j = tc.chunk - s * kps;
        kt0 = s * KTS + (j * KTS) / kps;
        kt1 = s * KTS + ((j + 1) * KTS) / kps;
    }

    // A loader role: row lr (+64 i), 16-byte chunk lq of the 128-byte k slice.
    // B loader role: 16-byte piece tid + 512 i of the k-tile's 16 column
    // blocks x 2 tiles (each column block's two tiles are one 2 KiB run).
    const int lr = tid >> 3, lq = tid & 7;
    const int T = (int)(K3 / 32);  // tiles per column block
    const uint4* __restrict__ wt4 = reinterpret_cast<const uint4*>(a.wt);
    uint4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const int s = kt / KTS;
        const int kl = kt * PBK - s * d + 8 * lq;
        const uint16_t* hs = a.h[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + lr + 64 * i;
            ra[i] = make_uint4(0u, 0u, 0u, 0u);
            if (m < M) ra[i] = *reinterpret_cast<const uint4*>(hs + (size_t)m * d + kl);
            const int p = tid + PTH * i;
            const int nb = (n0 >> 4) + (p >> 7);
            rb[i] = make_uint4(0u, 0u, 0u, 0u);
            if (nb < (d >> 4)) rb[i] = wt4[((size_t)nb * T + 2 * kt) * 64 + (p & 127)];
        }
    };
    auto lstore = [&](int stage) {
        uint4* A = lds + stage * STAGE_U4;
        uint4* B = A + PBM * PBK / 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = lr + 64 * i;
            A[r * 8 + (lq ^ (r & 7))] = ra[i];
            B[tid + PTH * i] = rb[i];
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};


    if (tid < PBM) {
        const int m = m0 + tid;
        float f[6] = {0.f, 1.f, 0.f, 1.f, 0.f, 1.f};
        if (m < M && NORM != NORM_NONE) {
            const float r0 = a.rstd[m], r1 = a.rstd[(size_t)M + m], r2 = a.rstd[(size_t)2 * M + m];
            if (NORM == NORM_LN) {
                f[0] = a.mu[m];
                f[2] = a.mu[(size_t)M + m];
                f[4] = a.mu[(size_t)2 * M + m];
            }
            f[1] = SPLIT ? r0 : r0 / r1;
            f[3] = SPLIT ? r1 : r1 / r2;
            f[5] = r2;
        }
#pragma unroll
        for (int q = 0; q < 6; ++q) rowf[q][tid] = f[q];
    } else if (tid < PBM + PBN) {
        const int cl = tid - PBM;
        const int n = n0 + cl;
        float f[4] = {0.f, 0.f, 0.f, 0.f};
        if (n < d) {
            if (NORM == NORM_LN) {
                f[0] = a.u[n];
                f[1] = a.u[(size_t)d + n];
                f[2] = a.u[(size_t)2 * d + n];
            }
            f[3] = a.c[n];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) colf[q][cl] = f[q];
    }
    // (visible to all after the first barrier of the main loop)

    // acc <- (acc - mu_s u_s) * factor_s, per row (factor: rstd ratio, or rstd_2 at the end)
    auto rescale = [&](int s) {
        float uc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) uc[j] = colf[s][wn * 64 + 16 * j + cb];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wm * 128 + 16 * i + 4 * g + e;
                const float mu = rowf[2 * s][r], fac = rowf[2 * s + 1][r];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j][e] = (acc[i][j][e] - mu * uc[j]) * fac;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto body = [&](int kt) {
        const int stage = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) gload(kt + 1);
        const uint4* A = lds + stage * STAGE_U4;
        const uint4* B = A + PBM * PBK / 8;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int q = 4 * kk + g;
            uint4 bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = B[((wn * 4 + j) * 2 + kk) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + 16 * i + cb;
                const uint4 af = A[r * 8 + (q ^ (r & 7))];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af, bfr[j], acc[i][j]);
            }
        }
        if (more) lstore(stage ^ 1);
        __syncthreads();
    };

    gload(kt0);
    lstore(0);
    __syncthreads();
    // one loop per state so the boundary rescale stays out of the hot loop
    for (int s = kt0 / KTS; s < 3 && s * KTS < kt1; ++s) {
        const int ka = max(kt0, s * KTS), kb = min(kt1, (s + 1) * KTS);
        for (int kt = ka; kt < kb; ++kt) body(kt);
        if (!SPLIT && NORM != NORM_NONE && s < 2) rescale(s);
    }

    if (SPLIT) {
        // partial of this chunk in fragment order, then the last arriver sums
        const int splits = a.splits;
        const int tile = tc.mt * TN + tc.nt;
        const size_t frag_per_wg = (size_t)PTH * 32;  // f32x4 per (tile, chunk)
        f32x4* part = reinterpret_cast<f32x4*>(a.part);
        f32x4* mine = part + ((size_t)tile * splits + tc.chunk) * frag_per_wg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (m0 + wm * 128 + 16 * i >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) mine[((size_t)(i * 4 + j) * 8 + wave) * 64 + lane] = acc[i][j];
        }
        __threadfence();
        __syncthreads();
        __shared__ int sh_last;
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            sh_last = (old == splits - 1);
        }
        __syncthreads();
        if (!sh_last) return;
        __threadfence();
        const int kps = splits / 3;
        // fragment by fragment: y = sum_s rstd_s * (sum_{chunks of s} P - mu_s u_s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
                if (m0 + wm * 128 + 16 * i < M) {
                    for (int s = 0; s < 3; ++s) {
                        f32x4 ss = f32x4{0.f, 0.f, 0.f, 0.f};
                        for (int ch = s * kps; ch < (s + 1) * kps; ++ch)
                            ss += part[((size_t)tile * splits + ch) * frag_per_wg + ((size_t)(i * 4 + j) * 8 + wave) * 64 +
                                       lane];
                        const float uc = colf[s][wn * 64 + 16 * j + cb];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = wm * 128 + 16 * i + 4 * g + e;
                            const float mu = rowf[2 * s][rr], r = rowf[2 * s + 1][rr];
                            y[e] += (ss[e] - mu * uc) * r;
                        }
                    }
                }
                acc[i][j] = y;
            }
        }
        if (tid == 0) a.counters[tile] = 0;
    } else {
        // last state: acc <- (acc - mu_2 u_2) * rstd_2
        if (NORM != NORM_NONE) rescale(2);
    }

    // + c, round to bf16, stage the wave's 128 x 64 tile in LDS, store 16-byte rows
    float cc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cc[j] = colf[3][wn * 64 + 16 * j + cb];
    uint16_t* st = reinterpret_cast<uint16_t*>(lds) + (size_t)wave * 128 * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * i + 4 * g + e, col = 16 * j + cb;
                st[r * 64 + col] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][j][e] + cc[j]));
            }
    __syncthreads();
#pragma unroll 4
    for (int v = lane; v < 128 * 8; v += 64) {
        const int r = v >> 3, q = v & 7;
        const int m = m0 + wm * 128 + r;
        const int n = n0 + wn * 64 + 8 * q;
        if (m < M && n < d)
            *reinterpret_cast<uint4*>(a.out + (size_t)m * d + n) = *reinterpret_cast<const uint4*>(st + r * 64 + 8 * q);
    }
}

PrefillPlan plan_prefill(int M, int d) {
    PrefillPlan p;
    p.tiles_m = (M + PBM - 1) / PBM;
    p.tiles_n = (d + PBN - 1) / PBN;
    const int tiles = p.tiles_m * p.tiles_n;
    p.splits = 1;
    if (tiles < 192) {
        // split K into chunks inside states until the grid covers the chip
        int kps = 1;
        const int KTS = d / PBK;
        while (tiles * 3 * kps < 256 && kps * 2 <= KTS && kps < 8) kps *= 2;
        p.splits = 3 * kps;
    }
    if (p.splits > 1) {
        p.counters_bytes = ((size_t)tiles * sizeof(int) + 255) / 256 * 256;
        p.part_bytes = (size_t)tiles * p.splits * PTH * 32 * sizeof(f32x4);
    }
    return p;
}

template <bool SPLIT, int NORM>
static hipError_t launch_prefill_t(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st) {
    const int items = p.tiles_m * p.tiles_n * (SPLIT ? p.splits : 1);
    const int grid = ((items + 7) / 8) * 8;
    prefill_kernel<SPLIT, NORM><<<grid, PTH, 0, st>>>(a, p.tiles_m, p.tiles_n);
    return hipGetLastError();
}

template <bool SPLIT>
static hipError_t launch_prefill_s(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st) {
    if (a.norm == NORM_LN) return launch_prefill_t<SPLIT, NORM_LN>(a, p, st);
    if (a.norm == NORM_RMS) return launch_prefill_t<SPLIT, NORM_RMS>(a, p, st);
    return launch_prefill_t<SPLIT, NORM_NONE>(a, p, st);
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st) {
    return p.splits > 1 ? launch_prefill_s<true>(a, p, st) : launch_prefill_s<false>(a, p, st);
}

}  // namespace e31
