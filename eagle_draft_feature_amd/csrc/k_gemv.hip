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
// block consecutive along k, so a wave's W' load is one contiguous 1 KiB.
//
// Two kernels:
//  * cols (M <= 8): one workgroup per 16 columns over the whole K, no
//    partial sum leaves it (no workspace, no atomics).  Wave w takes the
//    steps w, w + NW, ... of each state.
//  * split (M > 8): workgroup = 64 columns (four column blocks) x one K
//    chunk inside one state, so each A fragment feeds four MFMAs from
//    registers; the last workgroup of a column group to arrive reduces the
//    chunks in a fixed order.
// W' tiles are prefetched R steps ahead and A fragments RA steps ahead in
// register rings whose slots, pointers and waits are all static.
//
// A operands.  An MFMA A fragment puts 16 token rows in 16 consecutive
// lanes, so loading it directly makes every lane a separate cache access.
// Instead each 16-row tile is loaded coalesced (4 consecutive lanes read one
// row's 64 contiguous bytes), written lane-linear into a wave-private LDS
// tile and read back in fragment order; the chunk order inside a row is
// XOR-swizzled by the row's quarter so that both the lane-linear writes and
// the fragment reads are free of bank conflicts.
//
// Statistics are computed once per call, not once per workgroup: the
// first 3M workgroups each reduce one (state, token) row of the hidden
// states (one wave, coalesced 1 KiB loads; shifted sums S1 = sum (x - K),
// S2 = sum (x - K)^2 with K the mean of the row's first 32 values, RMSNorm
// sum x^2) and publish it; the workgroups that need the statistics (every
// cols workgroup, the last arriver of each split column group) read them
// at their epilogue, long after they were published.  The wait is bounded
// (real-time clock): should it expire, the reader computes every row itself
// with the same function, so the result is the same and every wave exits.
// The handoff uses device-coherent stores and loads (see the split kernel):
// a row's record carries the id of the call that wrote it, so stale records
// of earlier calls are never mistaken for new ones and nothing is reset.
//
// Token rows beyond M read row M-1 and are never stored.  Partial results
// are combined in a fixed order: the output is bitwise reproducible.
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int GV_WAVES = 8;          // waves per workgroup, at most
constexpr int GV_THREADS = 64 * GV_WAVES;
constexpr int GV_NB = 4;             // column blocks per split workgroup (64 columns)
constexpr uint32_t BF16_ONE2 = 0x3F803F80u;  // two bfloat16 ones

// Coalesced load of a 16-row A tile: lane l reads row l / 4, 16-byte chunk
// coal_chunk(l) of the 64-byte k-step; it lands in LDS slot l.
__device__ __forceinline__ int coal_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }
// LDS slot holding chunk g of row r: 4 r + (g ^ (r / 4 mod 4)); MFMA lane L
// needs row L % 16, chunk L / 16.
__device__ __forceinline__ int frag_slot(int lane) {
    const int r = lane & 15, g = lane >> 4;
    return 4 * r + (g ^ ((r >> 2) & 3));
}

// Shifted sums of one hidden-state row, by one wave: K = mean of the row's
// first 32 values, S1 = sum (x - K), S2 = sum (x - K)^2 (RMSNorm: K = 0,
// S2 = sum x^2).  Eight coalesced 1 KiB loads per pass; every lane returns
// the totals.  Deterministic: fixed per-lane order, fixed butterfly.
template <int NORM>
__device__ __forceinline__ void row_sums(const uint16_t* row, int d, int lane, float& K, float& S1, float& S2) {
    K = 0.f;
    if (NORM == NORM_LN) {
        const uint4 x = *reinterpret_cast<const uint4*>(row + 8 * (lane & 3));
        float v = ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
                  ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        K = v * (1.0f / 32.0f);
    }
    float s1 = 0.f, s2 = 0.f;
    auto acc = [&](const uint4& x) __attribute__((always_inline)) {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x0 = bf_lo(w[e]), x1 = bf_hi(w[e]);
            if (NORM == NORM_LN) {
                x0 -= K;
                x1 -= K;
                s1 += x0 + x1;
            }
            s2 = fmaf(x0, x0, fmaf(x1, x1, s2));
        }
    };
    const int nchunk = d >> 3, nfull = nchunk & ~511;
    for (int base = 0; base < nfull; base += 512) {
        uint4 x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = *reinterpret_cast<const uint4*>(row + 8 * (base + lane + 64 * q));
#pragma unroll
        for (int q = 0; q < 8; ++q) acc(x[q]);
    }
    for (int c = nfull + lane; c < nchunk; c += 64) acc(*reinterpret_cast<const uint4*>(row + 8 * c));
    S1 = wave_sum(s1);
    S2 = wave_sum(s2);
}

// Producer side (one wave): rows first, first + stride, ... of the 3M
// (state, token) rows, published as the record (K, S1, S2, call id): the
// three sums are stored first, then, once they have completed, the id.
template <int NORM>
__device__ void stats_produce(const GemvArgs& a, int first, int stride, int lane) {
    const int need = 3 * a.M;
    for (int it = first; it < need; it += stride) {
        const int s = it / a.M, m = it - s * a.M;
        float K, S1, S2;
        row_sums<NORM>(a.h[s] + (size_t)m * a.d, a.d, lane, K, S1, S2);
        if (lane == 0) {
            uint32_t* rec = a.rstats + 4 * it;
            store_coherent_u32(rec + 0, __float_as_uint(K));
            store_coherent_u32(rec + 1, __float_as_uint(S1));
            store_coherent_u32(rec + 2, __float_as_uint(S2));
            __builtin_amdgcn_s_waitcnt(0);
            store_coherent_u32(rec + 3, a.call_id);
        }
    }
}

// Reader side (one wave): all 3M rows into out[it][3] once every record
// carries this call's id; waits at most about 200 us, then computes the
// rows itself with the same function (same result).
template <int NORM>
__device__ void stats_gather(const GemvArgs& a, int lane, float (*out)[3]) {
    const int need = 3 * a.M;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ready = false;
    for (;;) {
        bool mine = true;
        for (int it = lane; it < need; it += 64) mine &= load_coherent_u32(a.rstats + 4 * it + 3) == a.call_id;
        if (__all(mine)) {
            ready = true;
            break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > 20000) break;  // 100 MHz clock
        __builtin_amdgcn_s_sleep(2);
    }
    if (ready) {
        for (int i = lane; i < 3 * need; i += 64) {
            const int it = i / 3, j = i - 3 * it;
            (&out[0][0])[i] = __uint_as_float(load_coherent_u32(a.rstats + 4 * it + j));
        }
    } else {
        for (int it = 0; it < need; ++it) {
            const int s = it / a.M, m = it - s * a.M;
            float K, S1, S2;
            row_sums<NORM>(a.h[s] + (size_t)m * a.d, a.d, lane, K, S1, S2);
            if (lane == 0) {
                out[it][0] = K;
                out[it][1] = S1;
                out[it][2] = S2;
            }
        }
    }
}

// mu and rstd of one row from its published sums
template <int NORM>
__device__ __forceinline__ void row_norm(const float (&st)[3], int d, float eps, float& mu, float& rstd) {
    mu = 0.f;
    rstd = 1.f;
    const float inv_d = 1.0f / (float)d;
    if (NORM == NORM_LN) {
        const float dm = st[1] * inv_d;
        mu = st[0] + dm;
        rstd = 1.0f / sqrtf(fmaxf(st[2] * inv_d - dm * dm, 0.f) + eps);
    } else if (NORM == NORM_RMS) {
        rstd = 1.0f / sqrtf(st[2] * inv_d + eps);
    }
}

// =====================================================================
// cols kernel: M <= 8, one workgroup per 16 columns, whole K
// =====================================================================
//
// Waves 0 .. NW-1 stream W' and run one MFMA per k-step, nothing else in
// their loop.  With a norm, wave NW handles the statistics: it reduces the
// workgroup's share of the rows (if any), then gathers all of them into LDS
// while the others stream.
constexpr int GV_COLS_MAX_THREADS = 64 * (GV_WAVES + 1);

template <int NORM, int R>
__global__ __launch_bounds__(GV_COLS_MAX_THREADS) void gemv_cols_kernel(GemvArgs a) {
    const int M = a.M, d = a.d;
    const int nblk = d >> 4;
    const int NW = a.waves;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const bool stat_wave = NORM != NORM_NONE && wave == NW;
    // wave 0 opens the gate when it reaches the last state: the statistics
    // wave reads the records only from then on (by that time they are long
    // published), so 256 waves do not poll them throughout
    __shared__ int sh_gate;
    if (tid == 0) sh_gate = 0;
    __syncthreads();
    // statistics rows are produced by workgroup ids 0, 1, ... whatever
    // their column block
    if (stat_wave) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane);
    // XCD-aware order: workgroup ids go round robin over the 8 XCDs, so each
    // XCD takes a contiguous range of column blocks
    const int per = (nblk + 7) >> 3;
    const int blk = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (blk >= nblk) return;
    const int T3 = d >> 5;        // k-steps per state
    const int n3 = T3 / NW;       // a streaming wave's steps per state (a multiple of R)

    __shared__ float sh_row[48][3];  // (K, S1, S2) of row (state, token) = s M + m
    __shared__ __attribute__((aligned(16))) f32x4 buf[GV_WAVES][64];
    __shared__ __attribute__((aligned(16))) uint4 lds_a[GV_WAVES][64];
    f32x4 acc[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int n = blk * 16 + cb;
    float cn = 0.f, us[3] = {0.f, 0.f, 0.f};

    if (wave < NW) {
        // epilogue constants first (wave 0): their latency hides under the stream
        if (wave == 0) {
            cn = a.c[n];
            if (NORM == NORM_LN)
#pragma unroll
                for (int s = 0; s < 3; ++s) us[s] = a.u[(size_t)s * d + n];
        }
        const uint4* __restrict__ wp =
            reinterpret_cast<const uint4*>(a.wp) + ((size_t)blk * 3 * T3 + wave) * 64 + lane;
        const size_t wstride = (size_t)NW * 64;  // uint4 between a wave's tiles
        const int aoff = min(lane >> 2, M - 1) * d + wave * 32 + 8 * coal_chunk(lane);
        const int astride = NW * 32;
        const uint16_t* const hp[3] = {a.h[0], a.h[1], a.h[2]};
        auto aload = [&](auto S_, int i) __attribute__((always_inline)) -> uint4 {
            constexpr int S = decltype(S_)::value;
            return *reinterpret_cast<const uint4*>(hp[S] + aoff + (size_t)i * astride);
        };
        uint4* la = lds_a[wave];
        const int fslot = frag_slot(lane);

        uint4 rw[R], rx[R];
        // prologue in the steady-state issue order (as if steps -R .. -1 had run)
#pragma unroll
        for (int p = 0; p < R; ++p) {
            rw[p] = wp[(size_t)p * wstride];
            rx[p] = aload(std::integral_constant<int, 0>(), p);
            __builtin_amdgcn_sched_barrier(0);
        }
        auto consume = [&](auto S_, int p) __attribute__((always_inline)) {
            constexpr int S = decltype(S_)::value;
            la[lane] = rx[p];
            acc[S] = mfma16x16x32(la[fslot], rw[p], acc[S]);
        };
        // Per state: full blocks refill inside the state; the last block's
        // refills belong to the next state (none after the last one).
        auto state_loop = [&](auto S_) __attribute__((always_inline)) {
            constexpr int S = decltype(S_)::value;
            auto Sc = std::integral_constant<int, S>();
            auto Sn = std::integral_constant<int, (S < 2 ? S + 1 : 2)>();
            if (S == 2 && wave == 0 && lane == 0)
                __hip_atomic_store(&sh_gate, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            int i = 0;
            for (; i < n3 - R; i += R) {
                const size_t j0 = (size_t)S * n3 + i;
#pragma unroll
                for (int p = 0; p < R; ++p) {
                    consume(Sc, p);
                    rw[p] = wp[(j0 + p + R) * wstride];
                    rx[p] = aload(Sc, i + p + R);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            const size_t j0 = (size_t)S * n3 + i;
#pragma unroll
            for (int p = 0; p < R; ++p) {
                consume(Sc, p);
                if (S < 2) {
                    rw[p] = wp[(j0 + p + R) * wstride];
                    rx[p] = aload(Sn, p);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        state_loop(std::integral_constant<int, 0>());
        state_loop(std::integral_constant<int, 1>());
        state_loop(std::integral_constant<int, 2>());
    } else if (stat_wave) {
        // gate (bounded like every wait here: about 1 ms of the 100 MHz clock)
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(&sh_gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 &&
               __builtin_amdgcn_s_memrealtime() - t0 < 100000)
            __builtin_amdgcn_s_sleep(8);
        stats_gather<NORM>(a, lane, sh_row);
    }
    __syncthreads();

    // ---- this wave's share sum_s rstd_s P_s (rows 4 g + e), summed over the
    //      waves in order (the statistics wave only takes part in the barrier)
    float rs[3][4], mu[3][4];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = min(4 * g + e, M - 1);
            float st[3] = {0.f, 0.f, 0.f};
            if (NORM != NORM_NONE) {
                st[0] = sh_row[s * M + m][0];
                st[1] = sh_row[s * M + m][1];
                st[2] = sh_row[s * M + m][2];
            }
            row_norm<NORM>(st, d, a.eps, mu[s][e], rs[s][e]);
        }
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = rs[0][e] * acc[0][e] + rs[1][e] * acc[1][e] + rs[2][e] * acc[2][e];
    if (wave < NW) buf[wave][lane] = y;
    __syncthreads();
    if (wave != 0) return;
    y = buf[0][lane];
    for (int w = 1; w < NW; ++w) y += buf[w][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m >= M) continue;
        float v = cn + y[e];
        if (NORM == NORM_LN)
#pragma unroll
            for (int s = 0; s < 3; ++s) v -= rs[s][e] * mu[s][e] * us[s];
        a.out[(size_t)m * d + n] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
}

// =====================================================================
// split kernel: 8 < M <= 64, 64 columns x one K chunk per workgroup
// =====================================================================
//
// Cross-workgroup handoff without cache maintenance: the L2 of an XCD is
// not coherent with the others, and an agent-scope release / acquire fence
// writes back / invalidates a whole L2, a cost of microseconds per
// workgroup.  Instead every value handed over (partials, statistics) is
// written and read with agent-scope atomic (relaxed) stores and loads, which
// go to the device coherence point; the writer waits for its stores to
// complete (s_waitcnt) before the workgroup barrier and the counter
// increment, and the reader issues its loads only after it has seen the
// final count.  The last arriver of a column group sums the chunk partials
// in a fixed order, applies rstd_s, mu_s u_s and c, stores bf16 and resets
// the group's counter, so the workspace is ready for the next call.
template <int NORM, int MT, int R, int RA>
__global__ __launch_bounds__(GV_THREADS) void gemv_split_kernel(GemvArgs a) {
    constexpr int ROWS = 16 * MT;
    constexpr int TILE_F4 = GV_NB * MT * 64;  // f32x4 per wave tile
    const int M = a.M, d = a.d;
    const int ngroups = d >> 6;
    const int nchunks = 3 * a.kps;
    const int nwg = ngroups * nchunks;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    // XCD-aware order: each XCD takes a contiguous range of (group, chunk)
    // pairs, so the chunks of a column group tend to share an L2
    const int per = (nwg + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (lin >= nwg) {
        if (NORM != NORM_NONE && wave == 0) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane);
        return;
    }
    const int grp = lin / nchunks, ch = lin - grp * nchunks;
    const int s = ch / a.kps, q = ch - s * a.kps;
    const int T3 = d >> 5;                 // k-steps per state
    const int TC = T3 / a.kps;             // k-steps per chunk
    const int tc0 = q * TC;                // first step of the chunk inside the state
    const int NW = a.waves;
    const int nw = TC / NW;                // this wave's steps (a multiple of R)
    const uint16_t* __restrict__ hs = s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2]);

    // W' tiles of column block 4 grp + b, k-step s T3 + tc0 + wave + NW i
    const u32x4* __restrict__ wp = reinterpret_cast<const u32x4*>(a.wp) +
                                   ((size_t)(GV_NB * grp) * 3 * T3 + (size_t)s * T3 + tc0 + wave) * 64 + lane;
    const size_t wblk = (size_t)3 * T3 * 64;       // uint4 between column blocks
    const size_t wstep = (size_t)NW * 64;          // uint4 between a wave's steps
    // coalesced A loads: tile tt, row 16 tt + lane / 4 (clamped)
    const uint16_t* ap[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const int m = min(16 * tt + (lane >> 2), M - 1);
        ap[tt] = hs + (size_t)m * d + (size_t)(tc0 + wave) * 32 + 8 * coal_chunk(lane);
    }
    const int ASTEP = NW * 32;

    u32x4 rw[R][GV_NB];
    u32x4 rx[RA][MT];
    auto wload = [&](int i, u32x4 (&w)[GV_NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < GV_NB; ++b) w[b] = wp[(size_t)b * wblk + (size_t)i * wstep];
    };
    auto aload = [&](int i, u32x4 (&x)[MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) x[tt] = *reinterpret_cast<const u32x4*>(ap[tt] + (size_t)i * ASTEP);
    };
    // prologue in the steady-state issue order (as if steps -R .. -1 had run)
#pragma unroll
    for (int p = 0; p < R; ++p) {
        wload(p, rw[p]);
        if (p >= R - RA) aload(p - (R - RA), rx[p - (R - RA)]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // statistics rows of this workgroup id, while the ring fills
    if (NORM != NORM_NONE && wave == 0) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane);

    __shared__ __attribute__((aligned(16))) u32x4 lds_a[GV_WAVES][MT * 64];
    u32x4* la = lds_a[wave];
    const int fslot = frag_slot(lane);

    f32x4 acc[GV_NB][MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
        for (int b = 0; b < GV_NB; ++b) acc[b][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) la[tt * 64 + lane] = rx[p % RA][tt];
        u32x4 af[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) af[tt] = la[tt * 64 + fslot];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int b = 0; b < GV_NB; ++b) acc[b][tt] = mfma16x16x32(af[tt], rw[p][b], acc[b][tt]);
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
    __shared__ float sh_row[3 * DECODE_MAX_M][3];  // (K, S1, S2) of row s M + m
    if (NORM != NORM_NONE && wave == 0) stats_gather<NORM>(a, lane, sh_row);
    __syncthreads();

    // outputs: thread -> column n (64 per group), rows rg, rg + NW, ...
    const int kps = a.kps;
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
            float mu = 0.f, r = 1.f;
            if (NORM != NORM_NONE) {
                const float st[3] = {sh_row[ss * M + m][0], sh_row[ss * M + m][1], sh_row[ss * M + m][2]};
                row_norm<NORM>(st, d, a.eps, mu, r);
            }
            float ps = 0.f;
            for (int qq = 0; qq < kps; ++qq)
                ps += load_coherent(a.part + ((size_t)grp * nchunks + ss * kps + qq) * (size_t)ROWS * 64 +
                                    (size_t)m * 64 + nl);
            if (NORM == NORM_LN) ps -= mu * us[ss];
            y += (NORM == NORM_NONE) ? ps : r * ps;
        }
        a.out[(size_t)m * d + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
    }
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- host side
GemvPlan plan_gemv(int M, int d, int norm) {
    GemvPlan p;
    p.MT = (M + 15) / 16;
    const int T3 = d / 32;
    if (M <= GEMV_COLS_MAX_M) {
        // cols: the most waves (<= 8) splitting a state's steps evenly with a
        // ring of 8, else 4, else 2 steps
        p.kind = GEMV_COLS;
        p.grid = d / 16;
        // one statistics wave beside the streaming ones (none without a norm)
        p.stat_waves = norm == NORM_NONE ? 0 : 1;
        for (int ring : {8, 4, 2}) {
            for (int nw = GV_WAVES; nw >= 1 && p.waves == 0; --nw)
                if (T3 % nw == 0 && (T3 / nw) % ring == 0) p.waves = nw, p.ring = ring;
            if (p.waves) break;
        }
        return p;
    }
    p.kind = GEMV_SPLIT;
    const int ngroups = d / 64;
    // the most waves (8, 4, 2, 1) that split a chunk evenly; then the chunks
    // per state that bring the workgroup count nearest one per CU, each wave
    // taking a multiple of the ring depth (4, else 2, else 1) of steps
    int best = -1;
    for (int waves : {8, 4, 2, 1}) {
        for (int kps : {1, 2, 4, 8}) {
            if (T3 % (kps * waves)) continue;
            const int nw = T3 / (kps * waves);
            // (three or four token tiles keep two steps in flight: registers)
            const int rmax = p.MT >= 3 ? 2 : 4;
            const int ring = (rmax == 4 && nw % 4 == 0) ? 4 : (nw % 2 == 0 ? 2 : 1);
            const int grid = ngroups * 3 * kps;
            const int score = std::abs(grid - 256) + (ring < rmax ? 64 : 0);
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
    p.part_bytes = (slots * (size_t)p.MT * 16 * 64 * sizeof(float) + 255) / 256 * 256;
    return p;
}

template <int NORM, int R>
static hipError_t launch_cols(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    const int grid = ((p.grid + 7) / 8) * 8;
    gemv_cols_kernel<NORM, R><<<grid, 64 * (p.waves + p.stat_waves), 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM, int MT, int R>
static hipError_t launch_split(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    // A ring: as deep as W's, but two steps for three or four token tiles
    // (registers)
    constexpr int RA = (MT >= 3 && R > 2) ? 2 : R;
    const int grid = ((p.grid + 7) / 8) * 8;
    gemv_split_kernel<NORM, MT, R, RA><<<grid, 64 * p.waves, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM, int MT>
static hipError_t launch_split_r(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.ring) {
        case 4: return launch_split<NORM, MT, 4>(a, p, st);
        case 2: return launch_split<NORM, MT, 2>(a, p, st);
        case 1: return launch_split<NORM, MT, 1>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NORM>
static hipError_t launch_gn(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    if (p.kind == GEMV_COLS) {
        switch (p.ring) {
            case 8: return launch_cols<NORM, 8>(a, p, st);
            case 4: return launch_cols<NORM, 4>(a, p, st);
            case 2: return launch_cols<NORM, 2>(a, p, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.MT) {
        case 1: return launch_split_r<NORM, 1>(a, p, st);
        case 2: return launch_split_r<NORM, 2>(a, p, st);
        case 3: return launch_split_r<NORM, 3>(a, p, st);
        case 4: return launch_split_r<NORM, 4>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const GemvArgs& a, int norm, const GemvPlan& p, hipStream_t st) {
    if (p.waves < 1 || p.waves > GV_WAVES || a.waves != p.waves || a.M < 1 || a.M > DECODE_MAX_M)
        return hipErrorInvalidValue;
    if (p.kind == GEMV_COLS && (a.M > GEMV_COLS_MAX_M || a.stat_waves != p.stat_waves || p.stat_waves > 1))
        return hipErrorInvalidValue;
    if (p.kind == GEMV_SPLIT && (p.kps < 1 || a.kps != p.kps)) return hipErrorInvalidValue;
    if (norm == NORM_LN) return launch_gn<NORM_LN>(a, p, st);
    if (norm == NORM_RMS) return launch_gn<NORM_RMS>(a, p, st);
    return launch_gn<NORM_NONE>(a, p, st);
}

}  // namespace e31
