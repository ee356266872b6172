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
// Tiling for gfx950: 256 x 256 output tile, BK = 64, 256 threads (4 waves
// as 2 x 2, each wave 128 x 128 = 8 x 8 MFMA 16x16x32 blocks, whose 256
// accumulator registers the compiler keeps in AGPRs).  Operands go from
// global memory straight to LDS (16-byte LDS-DMA loads, no register
// staging), double-buffered: the loads of k-tile t+1 are issued before the
// MFMAs of k-tile t.  A (hidden states, row-major) lands 8 rows x 128 bytes
// per wave load; its 16-byte chunks are XOR-swizzled by (row / 2) mod 8 on
// the global side, so the 16 rows of a fragment read hit distinct banks.
// W' arrives as 1 KiB MFMA B-fragment tiles (16 columns x 32 k, lane l's
// operand at bytes [16 l, 16 l + 16)), copied to LDS as they are, so a B
// operand is one conflict-free 16-byte read.  Tiles are walked in groups
// of 4 M-tiles, and consecutive workgroup ids are spread so that each XCD
// (workgroup id mod 8) takes a contiguous run of that order: the tiles an
// XCD runs at once share A and B tiles in its L2.
// Few tiles (small M) split K by chunks that never cross a state; partials go
// to a workspace and the last workgroup of a tile sums them in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int PBM = 256, PBN = 256, PBK = 64, PTH = 256;
constexpr int PGM = 4;  // M-tiles per raster group
constexpr int PFD = 4;  // L2 prefetch distance in k-tiles
constexpr int PFW = 2;  // prefetch loads per thread and k-tile
// s_waitcnt immediate: vmcnt <= n, lgkmcnt = 0, expcnt not waited for
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_VMPF = wait_vm(PFW);         // all but the prefetch just issued
constexpr int WAIT_VMPF16 = wait_vm(PFW + 16);  // ... and one stage of LDS-DMA loads
constexpr int WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt = 0 only
constexpr int STAGE_A = PBM * PBK * 2;           // bytes of an A stage (32 KiB)
constexpr int STAGE_BYTES = (PBM + PBN) * PBK * 2;  // A then B (64 KiB)

struct TileCoord {
    int mt, nt, chunk, gsz;  // gsz: M-tiles in the raster group of the tile
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
    tc.gsz = gsz;
    return tc;
}

template <bool SPLIT, int NORM>
__global__ __launch_bounds__(PTH, 1) void prefill_kernel(PrefillArgs a, int TM, int TN) {
    // two stages in separate arrays: with static stage indices the compiler
    // can tell the LDS-DMA writes of one stage from the reads of the other
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE_BYTES];
    // per-row factors of the tile: mu_0, rstd_0/rstd_1, mu_1, rstd_1/rstd_2, mu_2, rstd_2
    // per-column factors: u_0, u_1, u_2, c
    __shared__ float rowf[6][PBM];
    __shared__ float colf[4][PBN];

    const TileCoord tc = map_tile(blockIdx.x, TM, TN, SPLIT ? a.splits : 1);
    if (!tc.valid) return;
    const int M = a.M, d = a.d;
    const size_t K3 = (size_t)3 * d;
    const int m0 = tc.mt * PBM, n0 = tc.nt * PBN;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave bases stay scalar
    const int wm = wave >> 1, wn = wave & 1;
    const int KTS = d / PBK;  // k-tiles per state
    int kt0 = 0, kt1 = 3 * KTS;
    if (SPLIT) {
        const int kps = a.splits / 3;
        const int s = tc.chunk / kps, j = tc.chunk - s * kps;
        kt0 = s * KTS + (j * KTS) / kps;
        kt1 = s * KTS + ((j + 1) * KTS) / kps;
    }

    // Loader roles (per stage, 32 A blocks and 32 B tiles of 1 KiB; wave w
    // issues A blocks and B tiles 8 w .. 8 w + 7):
    //  A block ab: rows 8 ab + lane / 8, LDS chunk lane % 8 holds global
    //  chunk (lane % 8) ^ ((row / 2) % 8); rows past M re-read row M - 1.
    //  B tile bt: column block n0 / 16 + bt / 2 (clamped), k-step 2 kt + bt % 2.
    // Addresses are a wave-uniform base plus a 32-bit per-lane byte offset.
    const int T = (int)(K3 / 32);  // tiles per column block
    const int nblk = d >> 4;
    uint32_t aoff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = 8 * (8 * wave + q) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        aoff[q] = (uint32_t)((min(m0 + r, M - 1) - m0) * d + 8 * c) * 2u;  // < 512 d bytes
    }
    const char* wbase = reinterpret_cast<const char*>(a.wt);
    const uint32_t boff = (uint32_t)lane * 16u;
    auto issue = [&](int kt, char* sa) __attribute__((always_inline)) {
        const int s = kt / KTS;
        const char* hs = reinterpret_cast<const char*>((s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2])) +
                                                       (size_t)m0 * d + (kt * PBK - s * d));
        char* sb = sa + STAGE_A;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_global_load_lds(hs + aoff[q], sa + (8 * wave + q) * 1024, 16, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int bt = 8 * wave + q;
            const int nb = min((n0 >> 4) + (bt >> 1), nblk - 1);
            const char* src = wbase + (((size_t)nb * T + 2 * kt + (bt & 1)) << 10);
            __builtin_amdgcn_global_load_lds(src + boff, sb + bt * 1024, 16, 0, 0);
        }
    };

    // One of the wave's 16 LDS-DMA loads of a stage (c < 8: A block 8 w + c,
    // else B tile 8 w + c - 8); hs: the A source of the k-tile (see issue).
    auto issue_one = [&](int kt, const char* hs, char* sa, int c) __attribute__((always_inline)) {
        if (c < 8) {
            __builtin_amdgcn_global_load_lds(hs + aoff[c], sa + (8 * wave + c) * 1024, 16, 0, 0);
        } else {
            const int bt = 8 * wave + (c - 8);
            const int nb = min((n0 >> 4) + (bt >> 1), nblk - 1);
            const char* src = wbase + (((size_t)nb * T + 2 * kt + (bt & 1)) << 10);
            __builtin_amdgcn_global_load_lds(src + boff, sa + STAGE_A + bt * 1024, 16, 0, 0);
        }
    };
    auto a_src = [&](int kt) __attribute__((always_inline)) {
        const int s = kt / KTS;
        return reinterpret_cast<const char*>((s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2])) + (size_t)m0 * d +
                                             (kt * PBK - s * d));
    };

    // L2 prefetch of k-tile kt + PFD.  Every CU of an XCD asks for the same new
    // k-slice at about the same time, so without it each k-tile pays the
    // latency of memory, which one stage of lookahead cannot hide.  A
    // prefetch is one dword load per 128-byte line.  The workgroups an XCD
    // runs together (a run of the raster order: up to 4 M-tiles x 8 N-tiles)
    // share their A rows along N and their B lines along M, so each one
    // touches only its share: A rows r with r = nt (mod amod), B lines with
    // line = mt (mod bmod).  Split-K workgroups share nothing and touch their
    // whole slice.  Lines are dealt round-robin over the waves, two per lane;
    // lanes without one repeat the first line of their wave (one request).
    // The loaded words are kept until a later wait has covered them.
    int amod = 1, bmod = 1;
    if (!SPLIT) {
        const int na = min(TN, 8), nbm = tc.gsz;
        amod = na >= 8 ? 8 : (na >= 4 ? 4 : (na >= 2 ? 2 : 1));
        bmod = nbm >= 4 ? 4 : (nbm >= 2 ? 2 : 1);
    }
    bool pf_isa[PFW];
    uint64_t pf_off[PFW];
#pragma unroll
    for (int h = 0; h < PFW; ++h) {
        const int nA = PBM / amod, nT = nA + (16 * (PBN / 16)) / bmod;
        int q = wave + 4 * lane + 256 * h;
        if (q >= nT) q = wave;
        if (q < nA) {
            const int r = amod * q + tc.nt % amod;
            pf_isa[h] = true;
            pf_off[h] = (uint64_t)(min(m0 + r, M - 1) - m0) * (uint64_t)d * 2u;
        } else {
            const int L = bmod * (q - nA) + tc.mt % bmod;  // line of the B slice: 16 per column block
            const int nb = min((n0 >> 4) + (L >> 4), nblk - 1);
            pf_isa[h] = false;
            pf_off[h] = ((uint64_t)nb * T << 10) + (uint64_t)(L & 15) * 128u;
        }
    }
    auto prefetch = [&](int kt, uint32_t (&w)[PFW]) __attribute__((always_inline)) {
        const int kp = min(kt + PFD, kt1 - 1);
        const int s = kp / KTS;
        const char* ab = reinterpret_cast<const char*>((s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2])) +
                                                       (size_t)m0 * d + (kp * PBK - s * d));
        const char* bb = wbase + ((size_t)kp << 11);
#pragma unroll
        for (int h = 0; h < PFW; ++h)
            w[h] = __hip_atomic_load(reinterpret_cast<const uint32_t*>((pf_isa[h] ? ab : bb) + pf_off[h]),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    // fragment reads: A row wm 128 + 16 i + lane % 16, chunk 4 kk + lane / 16;
    // the swizzle (row / 2) % 8 is the same for the 8 row blocks, so one base
    // per kk and an immediate offset of 2048 i bytes
    uint32_t aread[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int r = wm * 128 + cb;
        aread[kk] = (uint32_t)(r * 128 + 16 * ((4 * kk + g) ^ ((r >> 1) & 7)));
    }
    const uint32_t bread = (uint32_t)(STAGE_A + wn * 16384) + (uint32_t)lane * 16u;

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        const int n = n0 + tid;
        float h4[4] = {0.f, 0.f, 0.f, 0.f};
        if (n < d) {
            if (NORM == NORM_LN) {
                h4[0] = a.u[n];
                h4[1] = a.u[(size_t)d + n];
                h4[2] = a.u[(size_t)2 * d + n];
            }
            h4[3] = a.c[n];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) colf[q][tid] = h4[q];
    }
    // (visible to all after the first barrier below)

    // acc <- (acc - mu_s u_s) * factor_s, per row (factor: rstd ratio, or rstd_2 at the end)
    auto rescale = [&](int s) __attribute__((always_inline)) {
        float uc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) uc[j] = colf[s][wn * 128 + 16 * j + cb];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wm * 128 + 16 * i + 4 * g + e;
                const float mu = rowf[2 * s][r], fac = rowf[2 * s + 1][r];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j][e] = (acc[i][j][e] - mu * uc[j]) * fac;
            }
        }
    };

    // Fragments of one k-step (kk) of a stage: 8 B and 8 A operands (64 VGPRs).
    auto read_frags = [&](const char* sa, int kk, u32x4 (&fa)[8], u32x4 (&fb)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j] = *reinterpret_cast<const u32x4*>(sa + bread + (2 * j + kk) * 1024);
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[i] = *reinterpret_cast<const u32x4*>(sa + aread[kk] + 2048 * i);
    };
    auto mma = [&](const u32x4 (&fa)[8], const u32x4 (&fb)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    };

    // Software pipeline of one state (k-tiles ka .. kb-1), two stages X, Y:
    // step kt (stage cur holds kt, nxt holds kt + 1, F0 = its kk = 0 operands):
    //   64 MFMAs on F0, with the 16 reads of F1 (kk = 1 of cur) between them
    //   wait for this wave's loads of nxt and for its LDS reads; barrier
    //   (every wave is done with cur, nxt has landed)
    //   64 MFMAs on F1, with the 16 LDS-DMA loads of kt + 2 into cur and the 16
    //   reads of F0 of nxt between them; then the L2 prefetch
    // One memory instruction per 4 MFMAs keeps the address and LDS queues
    // short, so the waves never stall at issue with the MFMA pipe idle.  The
    // barrier is a bare s_barrier (the explicit wait above covers the loads it
    // needs): a fence would also wait for the L2 prefetch still in flight.  The
    // prefetch loads are always the last memory instructions before a wait,
    // which leaves them in flight; their words are kept two steps, until a
    // wait that has covered them.  Near the end of a state the loads re-read
    // the last k-tile and the reads fetch a stale stage: harmless, and the
    // loop body stays free of branches.
    u32x4 fa0[8], fb0[8], fa1[8], fb1[8];
    uint32_t keep[2][PFW];
#pragma unroll
    for (int q = 0; q < PFW; ++q) keep[0][q] = keep[1][q] = 0u;
    auto prefetch_keep = [&](int kt) __attribute__((always_inline)) {
        uint32_t w[PFW];
        prefetch(kt, w);
#pragma unroll
        for (int q = 0; q < PFW; ++q) {
            keep[0][q] = keep[1][q];
            keep[1][q] = w[q];
        }
    };
    auto consume = [&](const uint32_t (&k)[PFW]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < PFW; ++q) asm volatile("" ::"v"(k[q]));
    };
    // read c of a k-step's fragments (c < 8: B operand c, else A operand c - 8)
    auto read_one = [&](const char* sa, int kk, u32x4 (&fa)[8], u32x4 (&fb)[8], int c) __attribute__((always_inline)) {
        if (c < 8)
            fb[c] = *reinterpret_cast<const u32x4*>(sa + bread + (2 * c + kk) * 1024);
        else
            fa[c - 8] = *reinterpret_cast<const u32x4*>(sa + aread[kk] + 2048 * (c - 8));
    };
    // MFMAs 4 c .. 4 c + 3 of a k-step: row block c / 2, column blocks 4 (c % 2) ..
    auto mma4 = [&](const u32x4 (&fa)[8], const u32x4 (&fb)[8], int c) __attribute__((always_inline)) {
        const int i = c >> 1;
#pragma unroll
        for (int j = 4 * (c & 1); j < 4 * (c & 1) + 4; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    };
    auto step = [&](int kt, int kb, char* cur, char* nxt) __attribute__((always_inline)) {
        // F0 has landed (it was read during the previous MFMA half)
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            read_one(cur, 1, fa1, fb1, c);
            mma4(fa0, fb0, c);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(WAIT_VMPF);
        asm volatile("s_barrier" ::: "memory");
        consume(keep[0]);  // the prefetch of two steps ago has landed
        const int kn = min(kt + 2, kb - 1);
        const char* hs = a_src(kn);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            issue_one(kn, hs, cur, c);
            read_one(nxt, 0, fa0, fb0, c);
            mma4(fa1, fb1, c);
            __builtin_amdgcn_sched_barrier(0);
        }
        prefetch_keep(kt);
        __builtin_amdgcn_sched_barrier(0);
    };
    // one pipeline per state, always starting on stage0 (the stage of every
    // access stays static, one copy of the loop); the boundary rescale stays
    // out of the hot loop
    for (int s = kt0 / KTS; s < 3 && s * KTS < kt1; ++s) {
        const int ka = max(kt0, s * KTS), kb = min(kt1, (s + 1) * KTS);
        issue(ka, stage0);
        if (ka + 1 < kb) issue(ka + 1, stage1);
        __builtin_amdgcn_sched_barrier(0);
        prefetch_keep(ka - 1);
        __builtin_amdgcn_sched_barrier(0);
        // stage0 has landed (the loads of stage1 and the prefetch may not have)
        if (ka + 1 < kb)
            __builtin_amdgcn_s_waitcnt(WAIT_VMPF16);
        else
            __builtin_amdgcn_s_waitcnt(WAIT_VMPF);
        asm volatile("s_barrier" ::: "memory");
        read_frags(stage0, 0, fa0, fb0);
        for (int kt = ka; kt < kb; kt += 2) {
            step(kt, kb, stage0, stage1);
            if (kt + 1 < kb) step(kt + 1, kb, stage1, stage0);
        }
        if (!SPLIT && NORM != NORM_NONE && s < 2) rescale(s);
    }
    consume(keep[0]);
    consume(keep[1]);
    // the last steps' loads write the stages the epilogue reuses: all of them
    // land before any wave writes there
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (SPLIT) {
        // partial of this chunk in fragment order, then the last arriver sums
        const int splits = a.splits;
        const int tile = tc.mt * TN + tc.nt;
        const size_t frag_per_wg = (size_t)PTH * 64;  // f32x4 per (tile, chunk)
        f32x4* part = reinterpret_cast<f32x4*>(a.part);
        f32x4* mine = part + ((size_t)tile * splits + tc.chunk) * frag_per_wg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (m0 + wm * 128 + 16 * i >= M) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) mine[((size_t)(i * 8 + j) * 4 + wave) * 64 + lane] = acc[i][j];
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
            for (int j = 0; j < 8; ++j) {
                f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
                if (m0 + wm * 128 + 16 * i < M) {
                    for (int s = 0; s < 3; ++s) {
                        f32x4 ss = f32x4{0.f, 0.f, 0.f, 0.f};
                        for (int ch = s * kps; ch < (s + 1) * kps; ++ch)
                            ss += part[((size_t)tile * splits + ch) * frag_per_wg + ((size_t)(i * 8 + j) * 4 + wave) * 64 +
                                       lane];
                        const float uc = colf[s][wn * 128 + 16 * j + cb];
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

    // + c, round to bf16, stage the wave's 128 x 128 tile in LDS, store 16-byte rows
    float cc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cc[j] = colf[3][wn * 128 + 16 * j + cb];
    uint16_t* st = reinterpret_cast<uint16_t*>(wave < 2 ? stage0 : stage1) + (size_t)(wave & 1) * 128 * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * i + 4 * g + e, col = 16 * j + cb;
                st[r * 128 + col] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][j][e] + cc[j]));
            }
    __syncthreads();
#pragma unroll 4
    for (int v = lane; v < 128 * 16; v += 64) {
        const int r = v >> 4, q = v & 15;
        const int m = m0 + wm * 128 + r;
        const int n = n0 + wn * 128 + 8 * q;
        if (m < M && n < d)
            *reinterpret_cast<uint4*>(a.out + (size_t)m * d + n) = *reinterpret_cast<const uint4*>(st + r * 128 + 8 * q);
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
        p.part_bytes = (size_t)tiles * p.splits * PTH * 64 * sizeof(f32x4);
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
