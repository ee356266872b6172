// Decode path of the fused per-state norm + FC on the folded weight (M <= 64,
// and up to 128 tokens in the column-split kernel).
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
// W' is read once per call, so its loads carry the non-temporal hint; the
// hidden-state tiles, re-read by every column group, are ordinary loads.
//
// Work split: workgroup = 64 or 128 columns (4 or 8 column blocks) x one K
// chunk inside one state, so each A fragment feeds 4 or 8 MFMAs from
// registers (the wider tile from 17 tokens on halves the re-reads of A); the
// last workgroup of a column group to arrive reduces the chunks in a fixed
// order.  Wave w of NW takes the chunk's k-steps w, w + NW, ...  W' tiles
// are prefetched R steps ahead and A fragments RA steps ahead in register
// rings whose slots, pointers and waits are all static.
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
// sum x^2) and publish it; the workgroups that need the statistics read them
// after their main loop, long after they were published.  The wait is
// bounded (real-time clock): should it expire, the reader computes every row
// itself with the same function, so the result is the same and every wave
// exits.  The handoff uses device-coherent stores and loads (see the split
// kernel): each of a record's three values is one 64-bit word that carries
// the id of the call that wrote it, so stale records of earlier calls are
// never mistaken for new ones, nothing is reset, and the writer never waits.
//
// Two kernels share this: the column-split kernel (waves own column blocks,
// chunks may cross states; the default from two tokens on where its grid
// fills at least half the chip) and the split kernel (waves share a column
// group's K chunk, chunks inside one state) for the other shapes.
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

// 16-byte accesses to the split-K partials at the device coherence point
// (buffer instructions with agent scope, sc1): the partials of one column
// group are written by workgroups on other XCDs, whose L2s are not
// coherent with this one.  The resource covers [base, base + bytes); an
// access outside it reads 0 / is dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_coherent16(__amdgpu_buffer_rsrc_t rs, int off, const u32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 16);
}
__device__ __forceinline__ u32x4 load_coherent16(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16);
}

// Coalesced load of a 16-row A tile: lane l reads row l / 4, 16-byte chunk
// coal_chunk(l) of the 64-byte k-step; it lands in LDS slot l.
__device__ __forceinline__ int coal_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }
// LDS slot holding chunk g of row r: 4 r + (g ^ (r / 4 mod 4)); MFMA lane L
// needs row L % 16, chunk L / 16.
__device__ __forceinline__ int frag_slot(int lane) {
    const int r = lane & 15, g = lane >> 4;
    return 4 * r + (g ^ ((r >> 2) & 3));
}

// Two k-steps of a 16-row A tile as 128-byte row pieces: 16-byte chunk c
// of row r sits in LDS slot 8 r + (c ^ pair_swz(r)), r the row's index in its
// 16-row block.  The 16 rows of a fragment read then hit distinct banks
// whether a 16-byte LDS access is served 8 or 16 lanes at a time.
__device__ __forceinline__ int pair_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Shifted sums of one hidden-state row, by one wave: K = mean of the row's
// first 32 values, S1 = sum (x - K), S2 = sum (x - K)^2 (RMSNorm: K = 0,
// S2 = sum x^2).  Eight coalesced 1 KiB loads per pass; every lane returns
// the totals.  Deterministic: fixed per-lane order, fixed butterfly.  The
// first pass (and the shift's values) can be loaded ahead (RowPre), so a
// producer wave overlaps it with other loads.
struct RowPre {
    uint4 k;     // 16 bytes of the row's first 32 values (lane % 4 picks which)
    uint4 x[8];  // first pass: chunks lane + 64 q (rows of at least 4096 values)
};

__device__ __forceinline__ void row_preload(const uint16_t* row, int d, int lane, RowPre& pre) {
    pre.k = *reinterpret_cast<const uint4*>(row + 8 * (lane & 3));
    if ((d >> 3) >= 512)
#pragma unroll
        for (int q = 0; q < 8; ++q) pre.x[q] = *reinterpret_cast<const uint4*>(row + 8 * (lane + 64 * q));
}

template <int NORM>
__device__ __forceinline__ void row_sums_pre(const uint16_t* row, int d, int lane, const RowPre& pre, float& K,
                                             float& S1, float& S2) {
    K = 0.f;
    if (NORM == NORM_LN) {
        const uint4 x = pre.k;
        float v = ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
                  ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
        v = quad_sum(v);
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
    int base = 0;
    if (nfull > 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc(pre.x[q]);
        base = 512;
    }
    for (; base < nfull; base += 512) {
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

template <int NORM>
__device__ __forceinline__ void row_sums(const uint16_t* row, int d, int lane, float& K, float& S1, float& S2) {
    RowPre pre;
    row_preload(row, d, lane, pre);
    row_sums_pre<NORM>(row, d, lane, pre, K, S1, S2);
}

// (state, token) row it = s M + m: token m's source row of state s
__device__ __forceinline__ const uint16_t* stats_row(const GemvArgs& a, int it, const WaveRows& wr) {
    const int s = it / a.M, m = it - s * a.M;
    const uint16_t* hs = s == 0 ? a.h[0] : (s == 1 ? a.h[1] : a.h[2]);
    return hs + (size_t)rv_lane_src(a.rv, wr, m) * (size_t)rv_ld(a.rv, s);
}

// A statistics record: the three sums of a row, each published as one
// 64-bit word (value bits, call id << 32) with a single atomic store, so
// that a reader holding all three words with this call's id holds the
// values, and the writer need not wait between stores.
__device__ __forceinline__ void rec_store(uint64_t* p, float v, uint32_t id) {
    __hip_atomic_store(p, (uint64_t)__float_as_uint(v) | ((uint64_t)id << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t rec_load(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Producer side (one wave): rows first, first + stride, ... of the 3M
// (state, token) rows, each published as a record (K, S1, S2).  `pre` holds
// the preloaded start of row `first` (if first < 3M).
template <int NORM>
__device__ void stats_produce(const GemvArgs& a, int first, int stride, int lane, const RowPre& pre,
                              const WaveRows& wr) {
    const int need = 3 * a.M;
    for (int it = first; it < need; it += stride) {
        float K, S1, S2;
        if (it == first) row_sums_pre<NORM>(stats_row(a, it, wr), a.d, lane, pre, K, S1, S2);
        else row_sums<NORM>(stats_row(a, it, wr), a.d, lane, K, S1, S2);
        if (lane == 0) {
            uint64_t* rec = a.rstats + 4 * it;
            rec_store(rec + 0, K, a.call_id);
            rec_store(rec + 1, S1, a.call_id);
            rec_store(rec + 2, S2, a.call_id);
        }
    }
}

// Reader side (one wave): all 3M rows into out[it][3] once every record
// carries this call's id; waits at most about 200 us, then computes the
// rows itself with the same function (same result).  Every load of a round
// is issued before the first is used, and the round that finds every id
// also holds the values.
template <int NORM>
__device__ void stats_gather(const GemvArgs& a, int lane, float (*out)[3], const WaveRows& wr) {
    constexpr int MAXR = 3 * DECODE_MAX_M;  // rows, at most
    constexpr int J = MAXR / 64;           // rows per lane, at most
    const int need = 3 * a.M;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ready = false;
    uint64_t w[J][3];
    // (every load below is unconditional, its row clamped to the last one:
    // loads under a branch would each get a wait of their own)
    for (; !a.stats_recompute;) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int k = 0; k < 3; ++k) w[j][k] = rec_load(a.rstats + 4 * min(lane + 64 * j, need - 1) + k);
        bool mine = true;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int k = 0; k < 3; ++k) mine &= (uint32_t)(w[j][k] >> 32) == a.call_id;
        if (__all(mine)) {
            ready = true;
            break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > 20000) break;  // 100 MHz clock
        __builtin_amdgcn_s_sleep(2);
    }
    if (ready) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int it = lane + 64 * j;
            if (it < need)
#pragma unroll
                for (int k = 0; k < 3; ++k) out[it][k] = __uint_as_float((uint32_t)w[j][k]);
        }
    } else {
        for (int it = 0; it < need; ++it) {
            float K, S1, S2;
            row_sums<NORM>(stats_row(a, it, wr), a.d, lane, K, S1, S2);
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

// Reader side for one wave's share of the rows: row first + lane (below
// 3M) as (mu, rstd) into out[row] once its record carries this call's id
// (the same bounded wait and the same fallback as stats_gather, so the same
// bits).  One round trip when the records are there.
// PRE: the caller loaded row it's three words earlier (p0, p1, p2); they
// are enough when all carry this call's id, and otherwise the wait below runs.
template <int NORM, bool PRE>
__device__ void stats_gather_rows(const GemvArgs& a, int lane, int first, float (*out)[2], const WaveRows& wr,
                                  uint64_t p0, uint64_t p1, uint64_t p2) {
    const int need = 3 * a.M;
    const int it = min(first + lane, need - 1);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ready = false;
    uint64_t w[3];
    if constexpr (PRE) {
        w[0] = p0;
        w[1] = p1;
        w[2] = p2;
        bool mine = !a.stats_recompute;
#pragma unroll
        for (int k = 0; k < 3; ++k) mine &= (uint32_t)(w[k] >> 32) == a.call_id;
        ready = __all(mine);
    }
    if (!ready) for (; !a.stats_recompute;) {
#pragma unroll
        for (int k = 0; k < 3; ++k) w[k] = rec_load(a.rstats + 4 * it + k);
        bool mine = true;
#pragma unroll
        for (int k = 0; k < 3; ++k) mine &= (uint32_t)(w[k] >> 32) == a.call_id;
        if (__all(mine)) {
            ready = true;
            break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > 20000) break;  // 100 MHz clock
        __builtin_amdgcn_s_sleep(2);
    }
    float st[3];
    if (ready) {
#pragma unroll
        for (int k = 0; k < 3; ++k) st[k] = __uint_as_float((uint32_t)w[k]);
    } else {
        // the wave recomputes its rows one by one; lane r keeps row first + r
        const int last = min(first + 64, need);
        for (int r = first; r < last; ++r) {
            float K, S1, S2;
            row_sums<NORM>(stats_row(a, r, wr), a.d, lane, K, S1, S2);
            if (r == it) {
                st[0] = K;
                st[1] = S1;
                st[2] = S2;
            }
        }
    }
    if (first + lane < need) row_norm<NORM>(st, a.d, a.eps, out[it][0], out[it][1]);
}

// =====================================================================
// 64 or 128 columns x one K chunk per workgroup
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
template <int NORM, int MT, int NB, int R, int RA>
__global__ __launch_bounds__(GV_THREADS) void gemv_split_kernel(GemvArgs a) {
    constexpr int ROWS = 16 * MT;
    constexpr int NCOL = 16 * NB;            // columns per workgroup
    constexpr int TILE_F4 = NB * MT * 64;    // f32x4 of a wave tile
    const int M = a.M, d = a.d;
    const int ngroups = d / NCOL;
    const int nchunks = 3 * a.kps;
    const int nwg = ngroups * nchunks;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    // XCD-aware order: each XCD takes a contiguous range of (group, chunk)
    // pairs, so the chunks of a column group tend to share an L2
    const int per = (nwg + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    // every wave: the tokens' source rows and valid mask
    const WaveRows wr = rv_wave(a.rv, M);
    // the statistics row of this workgroup id (if any): its start is loaded
    // first, so its latency overlaps the W' ring fill
    const bool producer = NORM != NORM_NONE && wave == 0 && (int)blockIdx.x < 3 * M;
    RowPre pre;
    if (producer) row_preload(stats_row(a, blockIdx.x, wr), d, lane, pre);
    if (lin >= nwg) {
        if (producer) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane, pre, wr);
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
    const size_t lds = (size_t)rv_ld(a.rv, s);

    // W' tiles of column block NB grp + b, k-step s T3 + tc0 + wave + NW i
    const u32x4* __restrict__ wp = reinterpret_cast<const u32x4*>(a.wp) +
                                   ((size_t)(NB * grp) * 3 * T3 + (size_t)s * T3 + tc0 + wave) * 64 + lane;
    const size_t wblk = (size_t)3 * T3 * 64;       // uint4 between column blocks
    const size_t wstep = (size_t)NW * 64;          // uint4 between a wave's steps
    // coalesced A loads: tile tt, row 16 tt + lane / 4 (clamped)
    const uint16_t* ap[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
        const int m = min(16 * tt + (lane >> 2), M - 1);
        ap[tt] = hs + (size_t)rv_lane_src(a.rv, wr, m) * lds + (size_t)(tc0 + wave) * 32 + 8 * coal_chunk(lane);
    }
    const int ASTEP = NW * 32;

    u32x4 rw[R][NB];
    u32x4 rx[RA][MT];
    auto wload = [&](int i, u32x4 (&w)[NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) w[b] = __builtin_nontemporal_load(&wp[(size_t)b * wblk + (size_t)i * wstep]);
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
    if (producer) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane, pre, wr);

    // LDS: during the loop the waves' A transpose tiles, afterwards the
    // pairwise-reduction buffers, then the row-major tile
    constexpr int LDS_A = GV_WAVES * MT * 64 * 16;
    constexpr int LDS_RED = (GV_WAVES / 2) * TILE_F4 * 16;  // at most 4 x 32 KiB
    constexpr int LDS_ROW = ROWS * NCOL * 4;
    constexpr int LDS_BYTES = LDS_A > LDS_RED ? (LDS_A > LDS_ROW ? LDS_A : LDS_ROW) : (LDS_RED > LDS_ROW ? LDS_RED : LDS_ROW);
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    u32x4* la = reinterpret_cast<u32x4*>(smem) + wave * MT * 64;
    const int fslot = frag_slot(lane);

    f32x4 acc[NB][MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) la[tt * 64 + lane] = rx[p % RA][tt];
        u32x4 af[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) af[tt] = la[tt * 64 + fslot];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b][tt] = mfma16x16x32(af[tt], rw[p][b], acc[b][tt]);
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
    __syncthreads();  // every wave is done with its A tile area

    // ---- pairwise sum of the wave tiles, e.g. for 8 waves
    //      ((w0+w4)+(w2+w6))+((w1+w5)+(w3+w7)): whole tiles, one round per level
    f32x4* buf = reinterpret_cast<f32x4*>(smem);
    for (int half = NW / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) buf[(wave - half) * TILE_F4 + (b * MT + tt) * 64 + lane] = acc[b][tt];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) acc[b][tt] += buf[wave * TILE_F4 + (b * MT + tt) * 64 + lane];
        }
        __syncthreads();
    }
    // wave 0 lays the tile out row-major [ROWS][NCOL] for coalesced stores
    float* rowmaj = reinterpret_cast<float*>(smem);
    if (wave == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int tt = 0; tt < MT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) rowmaj[(16 * tt + 4 * g + e) * NCOL + 16 * b + cb] = acc[b][tt][e];
    }
    __syncthreads();

    // the tile's first M rows go to this chunk's slot with 16-byte stores at
    // the device coherence point (buffer stores with agent scope, sc1)
    const size_t slot = (size_t)grp * nchunks + ch;
    const int nthreads = 64 * NW;
    {
        const __amdgpu_buffer_rsrc_t rs = part_rsrc(a.part + slot * (size_t)ROWS * NCOL, ROWS * NCOL * 4);
        const u32x4* src4 = reinterpret_cast<const u32x4*>(rowmaj);
        for (int v = tid; v < M * NCOL / 4; v += nthreads) store_coherent16(rs, v * 16, src4[v]);
    }

    // Wave 0 gathers the statistics records now (every workgroup; they were
    // published long before), so their loads share the round trip of the
    // partial stores and the last arriver does not wait for them.
    __shared__ float sh_row[3 * DECODE_MAX_M][3];  // (K, S1, S2) of row s M + m
    if (NORM != NORM_NONE && wave == 0) stats_gather<NORM>(a, lane, sh_row, wr);

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
    // each row's (mu, rstd) once, from the gathered sums
    __shared__ float sh_mr[3 * DECODE_MAX_M][2];
    if (NORM != NORM_NONE) {
        for (int it = tid; it < 3 * M; it += blockDim.x) {
            const float st[3] = {sh_row[it][0], sh_row[it][1], sh_row[it][2]};
            row_norm<NORM>(st, d, a.eps, sh_mr[it][0], sh_mr[it][1]);
        }
        __syncthreads();
    }
    // outputs: thread -> 4 consecutive columns (c4), rows rg, rg + rstep, ...
    // Each pass covers 4 rows x 3 states x 2 chunks: its 24 16-byte loads are
    // all issued before the first is used.  Chunks are summed in their order.
    const int kps = a.kps;
    constexpr int CQ = NCOL / 4;
    const int c4 = tid % CQ, rg = tid / CQ, rstep = nthreads / CQ;
    const int n = grp * NCOL + 4 * c4;
    const __amdgpu_buffer_rsrc_t rg_rs = part_rsrc(a.part + (size_t)grp * nchunks * ROWS * NCOL, nchunks * ROWS * NCOL * 4);
    auto load_pass = [&](int m0, int qq, u32x4 (&v)[4][3][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int ss = 0; ss < 3; ++ss)
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    const int m = m0 + rstep * r4;
                    const int off = (((ss * kps + qq + q2) * ROWS + m) * NCOL + 4 * c4) * 4;
                    v[r4][ss][q2] = (m < M && qq + q2 < kps) ? load_coherent16(rg_rs, off) : u32x4{0u, 0u, 0u, 0u};
                }
    };

    float us[3][4], cn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        cn[e] = a.c[n + e];
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) us[ss][e] = NORM == NORM_LN ? a.u[(size_t)ss * d + n + e] : 0.f;
    }
    if (rg < rstep) {
        for (int m0 = rg; m0 < M; m0 += 4 * rstep) {
            f32x4 ps[4][3];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
                for (int ss = 0; ss < 3; ++ss) ps[r4][ss] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int qq = 0; qq < kps; qq += 2) {
                u32x4 v[4][3][2];
                load_pass(m0, qq, v);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
                    for (int ss = 0; ss < 3; ++ss)
#pragma unroll
                        for (int q2 = 0; q2 < 2; ++q2) ps[r4][ss] += __builtin_bit_cast(f32x4, v[r4][ss][q2]);
            }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int m = m0 + rstep * r4;
                if (m >= M) continue;
                float y[4] = {cn[0], cn[1], cn[2], cn[3]};
#pragma unroll
                for (int ss = 0; ss < 3; ++ss) {
                    float mu = 0.f, r = 1.f;
                    if (NORM != NORM_NONE) {
                        mu = sh_mr[ss * M + m][0];
                        r = sh_mr[ss * M + m][1];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float pv = ps[r4][ss][e];
                        if (NORM == NORM_LN) pv -= mu * us[ss][e];
                        y[e] += (NORM == NORM_NONE) ? pv : r * pv;
                    }
                }
                const uint2 w = rv_ok(wr, m) ? make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])) : make_uint2(0u, 0u);
                *reinterpret_cast<uint2*>(a.out + (size_t)m * (size_t)a.rv.ld_out + n) = w;
            }
        }
    }
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// =====================================================================
// One or two tokens: one 16-column block x the whole K per workgroup
// =====================================================================
//
// With one or two tokens the hidden states are small (24 KiB per token at
// d = 4096), so every workgroup copies them into LDS once, computes their
// statistics itself (the same shifted sums as the split kernel's, from LDS),
// and walks the whole K for one 16-column block of W': no split-K partials,
// no counters, nothing handed between workgroups (d = 4096 gives 256
// workgroups, one per CU).  Wave w of 8 takes the k-steps w, w + 8, ... of
// each state in turn, one accumulator per state, with an R-step W' ring; the
// A fragment of a step is one LDS read (token rows padded by 64 bytes, so
// that the distinct rows fall in different banks).  The waves' per-state
// tiles are summed in LDS in wave order, and wave 0 applies
// sum_s rstd_s (P_s - mu_s u_s) + c.  Measured: with four tokens the 96 KiB
// staged per workgroup before the loop costs more than the column-split
// kernel's hand-off.
constexpr int WH_MAXM = 2;
constexpr int WH_A_BYTES = WH_MAXM * (6 * 4096 + 64);  // token rows in LDS, at most
constexpr int WH_WAVES = 8;

template <int NORM, int R, int MM>
__global__ __launch_bounds__(64 * WH_WAVES) void gemv_whole_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) char la[MM * (6 * 4096 + 64)];
    __shared__ f32x4 red[WH_WAVES][3][16];  // the tiles' first row group (rows 0..3 hold the tokens)
    __shared__ float sst[3 * MM][3];
    const int M = a.M, d = a.d;
    const int T3 = d >> 5, JS = T3 / WH_WAVES;  // k-steps per state and wave
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = blockIdx.x;
    if (grp >= (d >> 4)) return;
    const int rstride = 6 * d + 64;

    // The tokens' rows into LDS, states concatenated (row m: k = 0 .. 3d-1).
    // Their loads are issued before the W' ring's, every one of them (a
    // thread's surplus chunks wrap round to chunks already taken, spread
    // over the rows), so the LDS writes wait for these loads alone and the
    // ring stays in flight across the staging barrier.
    constexpr int ACH = MM * (3 * 4096 / 8) / (64 * WH_WAVES);  // 16-byte chunks per thread
    const int cpr = (3 * d) >> 3, cps = d >> 3;  // 16-byte chunks per row / per state
    const int nchunk = M * cpr;
    const WaveRows wr = rv_wave(a.rv, M);
    u32x4 av[ACH];
    int aoff[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        int v = tid + i * 64 * WH_WAVES;
        v = v < nchunk ? v : v % nchunk;
        const int m = v / cpr, c = v - m * cpr;
        const int st = (c >= cps) + (c >= 2 * cps);
        const size_t srow = (size_t)rv_lane_src(a.rv, wr, m);
        const uint16_t* base = st == 0 ? a.h[0] + srow * (size_t)a.rv.ld[0]
                                       : (st == 1 ? a.h[1] + srow * (size_t)a.rv.ld[1] : a.h[2] + srow * (size_t)a.rv.ld[2]);
        av[i] = *reinterpret_cast<const u32x4*>(base + 8 * (c - st * cps));
        aoff[i] = m * rstride + c * 16;
    }
    __builtin_amdgcn_sched_barrier(0);

    // W' tiles of column block grp: this wave's local step j is k-step
    // wave + WH_WAVES j
    const u32x4* __restrict__ wp = reinterpret_cast<const u32x4*>(a.wp) + ((size_t)grp * 3 * T3 + wave) * 64 + lane;
    constexpr int WSTEP = WH_WAVES * 64;  // uint4 between a wave's steps
    u32x4 rw[R];
#pragma unroll
    for (int p = 0; p < R; ++p) rw[p] = __builtin_nontemporal_load(&wp[(size_t)p * WSTEP]);
    __builtin_amdgcn_sched_barrier(0);
    // c and u of this lane's column, needed at the end only: behind the ring
    const int n = 16 * grp + cb;
    const float cn = a.c[n];
    float un[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN)
#pragma unroll
        for (int q = 0; q < 3; ++q) un[q] = a.u[(size_t)q * d + n];

#pragma unroll
    for (int i = 0; i < ACH; ++i)
        if (tid + i * 64 * WH_WAVES < nchunk) *reinterpret_cast<u32x4*>(la + aoff[i]) = av[i];
    __syncthreads();

    // statistics of the 3M (state, token) rows: wave w takes rows w, w + 8
    if (NORM != NORM_NONE) {
        for (int it = wave; it < 3 * M; it += WH_WAVES) {
            const int st = it / M, m = it - st * M;
            const char* row = la + m * rstride + st * d * 2;
            float K = 0.f;
            if (NORM == NORM_LN) {
                const uint4 x = *reinterpret_cast<const uint4*>(row + 16 * (lane & 3));
                float v = ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
                          ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
                v = quad_sum(v);
                K = v * (1.0f / 32.0f);
            }
            float s1 = 0.f, s2 = 0.f;
            for (int c = lane; c < (d >> 3); c += 64) {
                const uint4 x = *reinterpret_cast<const uint4*>(row + 16 * c);
                const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x0 = bf_lo(w4[e]), x1 = bf_hi(w4[e]);
                    if (NORM == NORM_LN) {
                        x0 -= K;
                        x1 -= K;
                        s1 += x0 + x1;
                    }
                    s2 = fmaf(x0, x0, fmaf(x1, x1, s2));
                }
            }
            const float S1 = wave_sum(s1), S2 = wave_sum(s2);
            if (lane == 0) {
                sst[it][0] = K;
                sst[it][1] = S1;
                sst[it][2] = S2;
            }
        }
    }

    // MFMA lane L: token row L % 16 (clamped to M - 1), 16-byte chunk L / 16 of the step
    const char* abase = la + min(cb, M - 1) * rstride + 16 * g;
    f32x4 acc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one state: its ring blocks refill R steps ahead (the last block of the
    // last state does not); slot = local step % R, static
    auto run_state = [&](f32x4& ac, int j0, bool last) __attribute__((always_inline)) {
        int i = 0;
        const int nfull = last ? JS - R : JS;
        for (; i < nfull; i += R) {
#pragma unroll
            for (int p = 0; p < R; ++p) {
                const int jj = j0 + i + p;
                const u32x4 af = *reinterpret_cast<const u32x4*>(abase + (wave + WH_WAVES * jj) * 64);
                ac = mfma16x16x32(af, rw[p], ac);
                rw[p] = __builtin_nontemporal_load(&wp[(size_t)(jj + R) * WSTEP]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (last) {
#pragma unroll
            for (int p = 0; p < R; ++p) {
                const int jj = j0 + i + p;
                const u32x4 af = *reinterpret_cast<const u32x4*>(abase + (wave + WH_WAVES * jj) * 64);
                ac = mfma16x16x32(af, rw[p], ac);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // each state's tile rows 0..3 (lanes 0..15) to LDS as soon as it is done
    run_state(acc[0], 0, false);
    if (g == 0) red[wave][0][lane] = acc[0];
    run_state(acc[1], JS, false);
    if (g == 0) red[wave][1][lane] = acc[1];
    run_state(acc[2], 2 * JS, true);
    if (g == 0) red[wave][2][lane] = acc[2];
    __syncthreads();
    if (wave != 0) return;

    // wave 0, every LDS read issued before any is used: lane (g, cb) reads
    // waves 2 g, 2 g + 1 of the rows e < MM (a fixed tree over the waves
    // with the cross-row sums below); lane MM q + m turns the sums of
    // (state q, token m) into (mu, rstd) (lanes past 3 MM take state 2's, unused)
    static_assert(WH_WAVES == 8, "the tree takes two waves per 16-lane row");
    float tv[3][2][MM];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
            for (int e = 0; e < MM; ++e) tv[q][w][e] = reinterpret_cast<const float*>(&red[2 * g + w][q][cb])[e];
    float stl[3] = {0.f, 0.f, 0.f};
    if (NORM != NORM_NONE) {
        const int it = min(lane / MM, 2) * M + min(lane % MM, M - 1);
#pragma unroll
        for (int k = 0; k < 3; ++k) stl[k] = sst[it][k];
    }
    __builtin_amdgcn_sched_barrier(0);
    float mu = 0.f, rs = 1.f;
    if (NORM != NORM_NONE) row_norm<NORM>(stl, d, a.eps, mu, rs);
    float P[3][MM];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int e = 0; e < MM; ++e) P[q][e] = xor32_sum(xor16_sum(tv[q][0][e] + tv[q][1][e]));
    // lane (0, cb): rows e, column n; (mu, rstd) of a row read from its lane
#pragma unroll
    for (int e = 0; e < MM; ++e) {
        float y = cn;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            float muq = 0.f, rq = 1.f;
            if (NORM != NORM_NONE) {
                muq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), MM * q + e));
                rq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), MM * q + e));
            }
            float pv = P[q][e];
            if (NORM == NORM_LN) pv -= muq * un[q];
            y += (NORM == NORM_NONE) ? pv : rq * pv;
        }
        if (g == 0 && e < M)
            a.out[(size_t)e * (size_t)a.rv.ld_out + n] = rv_ok(wr, e) ? (uint16_t)(pack_bf2(y, 0.f) & 0xffffu) : (uint16_t)0;
    }
}

// =====================================================================
// Up to 6 tokens, packed token blocks: one 16-column block x the whole K
// =====================================================================
//
// The MFMA's 16 A rows hold at most 6 tokens here, so the rows past the
// tokens are spare.  A wave's token loads use them: lane (g, cb) of a
// "packed block" holds token row cb % MP (MP = 16 / SB, a power of two at
// or above M) of the wave's k-step t0 + cb / MP, 16 bytes of k-group g.  One
// 16-byte load per lane thus brings SB of the wave's k-steps for every
// token (SB = 16 at one token, 2 at five or six), and the A fragment of
// k-step t0 + j is the block moved j * MP lanes down each 16-lane row (a DPP
// row shift; rows past the tokens then hold junk whose MFMA rows are never
// read).  Each lane feeds its block's values once to the row statistics
// (shifted sums; shift K = mean of the row's first 32 values), so the
// statistics cost one pass over the tokens' values per workgroup, spread
// through the loop, and no token bytes are staged before it.  Otherwise as
// the whole-K kernel: one 16-column block of W' per workgroup (d = 4096: 256
// workgroups), wave w of 8 takes the k-steps w, w + 8, ... of each state in
// turn with an 8- or 16-step W' ring.  Each wave publishes a state's tile
// rows that can hold tokens and its per-token statistics to LDS as soon as
// the state is done (lane sums by DPP and gfx950 permlane swaps, no LDS round
// trip); after one barrier wave 0 issues all its LDS reads at once, sums the
// waves in a fixed tree, broadcasts (mu, rstd) by readlane and applies
// sum_s rstd_s (P_s - mu_s u_s) + c.
// Measured: from seven tokens on, every workgroup's pass over all the
// tokens' values costs as much as the column-split kernel's hand-off.
constexpr int PK_MAXM = 6;
constexpr int PK_WAVES = 8;
constexpr int PK_R = 8;  // W' ring depth, and the least k-steps per wave and state
// One token at d <= 4096 (blocks of 16 k-steps, one workgroup per CU): a
// 16-step ring, which kept the loop fed better (17.7 against 18.1 us at
// d = 4096).  Elsewhere it was as fast or slower: six tokens 20.5 against
// 20.1 us; one token at d = 8192 (two workgroups per CU in turn) 68.0
// against 64.7.
inline int pk_ring(int sb, int d) { return sb == 16 && d <= 4096 ? 16 : PK_R; }

// v moved down by n lanes within each 16-lane row (lane i takes lane i + n;
// lanes past the row's end get 0)
__device__ __forceinline__ uint32_t row_shl_u32(uint32_t v, int n) {
    switch (n) {
        case 0: return v;
        case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xf, 0xf, true);
        case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xf, 0xf, true);
        case 3: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x103, 0xf, 0xf, true);
        case 4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xf, 0xf, true);
        case 5: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x105, 0xf, 0xf, true);
        case 6: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x106, 0xf, 0xf, true);
        case 7: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x107, 0xf, 0xf, true);
        case 8: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x108, 0xf, 0xf, true);
        case 9: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x109, 0xf, 0xf, true);
        case 10: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10a, 0xf, 0xf, true);
        case 11: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10b, 0xf, 0xf, true);
        case 12: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10c, 0xf, 0xf, true);
        case 13: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10d, 0xf, 0xf, true);
        case 14: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10e, 0xf, 0xf, true);
        default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x10f, 0xf, 0xf, true);
    }
}

// sum over the lanes of each 16-lane row whose index is equal modulo MP
// (DPP row rotations by 8, 4, .. MP); every such lane ends with the sum
template <int MP>
__device__ __forceinline__ float row_mod_sum(float v) {
    if (MP <= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
    if (MP <= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
    if (MP <= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
    if (MP <= 1) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
    return v;
}

template <int NORM, int SB, int R>
__global__ __launch_bounds__(64 * PK_WAVES) void gemv_pack_kernel(GemvArgs a) {
    constexpr int MP = 16 / SB, U = SB > R ? SB : R, NBB = U / SB;  // U: steps per body
    constexpr int NG = (MP + 3) / 4;  // 16-lane row groups of a tile that hold token rows
    __shared__ f32x4 red[PK_WAVES][3][16 * NG];
    __shared__ __align__(16) float sred[3][MP][PK_WAVES][2];
    __shared__ float smk[3][MP];
    const int M = a.M, d = a.d;
    const int T3 = d >> 5, JS = T3 / PK_WAVES;  // k-steps per state; per state and wave
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = blockIdx.x;
    if (grp >= (d >> 4)) return;
    const int n = 16 * grp + cb;  // this lane's output column
    const WaveRows wr = rv_wave(a.rv, M);

    // packed-block lane (g, cb): step offset jl = cb / MP, token row rl = cb % MP
    const int jl = cb / MP, rl = cb % MP;
    const bool rvalid = rl < M;
    const size_t brow = (size_t)rv_lane_src(a.rv, wr, min(rl, M - 1));
    // Wave w takes runs of RL consecutive k-steps of each state: its local
    // step l is the state's k-step RL w + 8 RL (l / RL) + l % RL.  With RL =
    // SB a packed block holds SB consecutive k-steps, SB x 64 contiguous bytes
    // of each token row; in the wave-strided order (RL = 1) its pieces are
    // 64 bytes each, 512 bytes apart.  Runs measured faster from four k-steps
    // per block on (d = 8192, one token: 60.5 against 63.6 us) and slower at
    // two (six tokens: eight rows of 128 bytes, 21.3 against 20.3 us).
    // State s's block of the local steps [t, t + SB): bs + 512 t.
    constexpr int RL = SB >= 4 ? SB : 1;
    const int boff = 64 * (RL * wave + (RL == 1 ? PK_WAVES * jl : jl));
    const char* const b0 = reinterpret_cast<const char*>(a.h[0] + brow * (size_t)a.rv.ld[0]) + 16 * g + boff;
    const char* const b1 = reinterpret_cast<const char*>(a.h[1] + brow * (size_t)a.rv.ld[1]) + 16 * g + boff;
    const char* const b2 = reinterpret_cast<const char*>(a.h[2] + brow * (size_t)a.rv.ld[2]) + 16 * g + boff;
    constexpr int BSTEP = 64 * PK_WAVES;  // bytes per local step between blocks

    // shift rows (LayerNorm): lane (g, cb) holds the values 8 g .. of each
    // state's first k-step of its own token row; c and u of this lane's column
    u32x4 kf0 = {0u, 0u, 0u, 0u}, kf1 = kf0, kf2 = kf0;
    if (NORM == NORM_LN) {
        kf0 = *reinterpret_cast<const u32x4*>(a.h[0] + brow * (size_t)a.rv.ld[0] + 8 * g);
        kf1 = *reinterpret_cast<const u32x4*>(a.h[1] + brow * (size_t)a.rv.ld[1] + 8 * g);
        kf2 = *reinterpret_cast<const u32x4*>(a.h[2] + brow * (size_t)a.rv.ld[2] + 8 * g);
    }
    const float cn = a.c[n];
    float un[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN) {
#pragma unroll
        for (int q = 0; q < 3; ++q) un[q] = a.u[(size_t)q * d + n];
    }
    __builtin_amdgcn_sched_barrier(0);

    // rings: the first body's packed blocks, then the W' ring
    u32x4 ab[NBB];
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) ab[bb] = *reinterpret_cast<const u32x4*>(b0 + bb * SB * BSTEP);
    // the W' tile of local step l (over the three states in turn), in uint4
    const u32x4* __restrict__ wp = reinterpret_cast<const u32x4*>(a.wp) + ((size_t)grp * 3 * T3 + RL * wave) * 64 + lane;
    auto woff = [](int l) __attribute__((always_inline)) { return (size_t)(PK_WAVES * RL * (l / RL) + l % RL) * 64; };
    u32x4 rw[R];
#pragma unroll
    for (int p = 0; p < R; ++p) {
        rw[p] = __builtin_nontemporal_load(&wp[woff(p)]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // per-lane shifts of the packed lanes' token rows
    float kb[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN) {
        const u32x4 kf[3] = {kf0, kf1, kf2};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            float v = ((bf_lo(kf[q][0]) + bf_hi(kf[q][0])) + (bf_lo(kf[q][1]) + bf_hi(kf[q][1]))) +
                      ((bf_lo(kf[q][2]) + bf_hi(kf[q][2])) + (bf_lo(kf[q][3]) + bf_hi(kf[q][3])));
            v = xor32_sum(xor16_sum(v));
            const float K = v * (1.0f / 32.0f);  // the shift of token row rl
            if (wave == 0 && g == 0 && cb < MP) smk[q][cb] = K;
            kb[q] = K;
        }
    }

    f32x4 acc[3];
    float s1[3] = {0.f, 0.f, 0.f}, s2[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one body of U steps of state s starting at local step i: per packed
    // block its statistics, its SB fragments and the prefetch of the block U
    // steps on (from anext when that lies in the next state), then SB steps.
    // refill: 0 none, 1 W' and blocks, 2 W' only for steps whose target is
    // still inside the call (the last body of the last state)
    auto body = [&](f32x4& ac, float& x1s, float& x2s, float k, int j0, int i, const char* anext, int nexti,
                    int refill) __attribute__((always_inline)) {
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb) {
            if (NORM != NORM_NONE) {
                float t1 = 0.f, t2 = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x0 = bf_lo(ab[bb][e]), x1 = bf_hi(ab[bb][e]);
                    if (NORM == NORM_LN) {
                        x0 -= k;
                        x1 -= k;
                        t1 += x0 + x1;
                    }
                    t2 = fmaf(x0, x0, fmaf(x1, x1, t2));
                }
                x1s += rvalid ? t1 : 0.f;
                x2s += rvalid ? t2 : 0.f;
            }
            // fragments of steps 1 .. SB-1; step 0 reads the block itself,
            // after which its registers take the block U steps on
            u32x4 fr[SB];
#pragma unroll
            for (int j = 1; j < SB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) fr[j][e] = row_shl_u32(ab[bb][e], j * MP);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int p = bb * SB + j;
                ac = mfma16x16x32(j == 0 ? ab[bb] : fr[j], rw[p % R], ac);
                if (refill == 1 || (refill == 2 && p + R < U))
                    rw[p % R] = __builtin_nontemporal_load(&wp[woff(j0 + i + p + R)]);
                if (j == 0 && refill == 1) ab[bb] = *reinterpret_cast<const u32x4*>(anext + (nexti + bb * SB) * BSTEP);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // one state: JS / U bodies; the last one's prefetches target the next
    // state (or, in the last state, only what is left of it)
    auto run_state = [&](f32x4& ac, float& x1s, float& x2s, float k, int j0, const char* acur, const char* anext,
                         bool last) __attribute__((always_inline)) {
        int i = 0;
        for (; i < JS - U; i += U) body(ac, x1s, x2s, k, j0, i, acur, i + U, 1);
        if (last)
            body(ac, x1s, x2s, k, j0, i, acur, 0, 2);
        else
            body(ac, x1s, x2s, k, j0, i, anext, 0, 1);
    };
    // a state's share for the cross-wave sums, once its steps are done: the
    // tile rows that can hold tokens (row groups below NG), and each token
    // row's statistics summed over its lanes (DPP within the 16-lane rows,
    // then the two cross-row swaps); states 0 and 1 while the next state's
    // loads are in flight
    auto publish = [&](int q) __attribute__((always_inline)) {
        if (g < NG) red[wave][q][lane] = acc[q];
        if (NORM != NORM_NONE) {
            const float x1 = xor32_sum(xor16_sum(row_mod_sum<MP>(s1[q])));
            const float x2 = xor32_sum(xor16_sum(row_mod_sum<MP>(s2[q])));
            if (lane < MP) *reinterpret_cast<float2*>(&sred[q][lane][wave][0]) = make_float2(x1, x2);
        }
    };
    run_state(acc[0], s1[0], s2[0], kb[0], 0, b0, b1, false);
    publish(0);
    run_state(acc[1], s1[1], s2[1], kb[1], JS, b1, b2, false);
    publish(1);
    run_state(acc[2], s1[2], s2[2], kb[2], 2 * JS, b2, b2, true);
    publish(2);
    __syncthreads();
    if (wave != 0) return;

    // wave 0. Lane (g, cb) sums WPL waves' tiles of row group g mod NG (waves
    // WPL (g / NG) ..), and the lanes of one row group are then summed across
    // rows: a fixed tree over the 8 waves. Lane MP q + r turns the sums of
    // (state q, token r) into (mu, rstd) (lanes past 3 MP take state 2's, unused).
    // Every LDS read is issued before any is used: one round trip.
    constexpr int WPL = PK_WAVES * NG / 4;
    const int gg = g % NG, w0 = (g / NG) * WPL;
    const int qs = min(lane / MP, 2), r = lane % MP;
    // only the tile elements that can hold a token are read (rows e < MP),
    // each into registers of its own
    constexpr int EU = MP < 4 ? MP : 4;
    float tv[3][WPL][EU];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int w = 0; w < WPL; ++w)
#pragma unroll
            for (int e = 0; e < EU; ++e) tv[q][w][e] = reinterpret_cast<const float*>(&red[w0 + w][q][16 * gg + cb])[e];
    f32x4 sv[PK_WAVES / 2];  // (S1, S2) of waves 2 i and 2 i + 1
    float kq = 0.f;
    if (NORM != NORM_NONE) {
#pragma unroll
        for (int i = 0; i < PK_WAVES / 2; ++i) sv[i] = reinterpret_cast<const f32x4*>(&sred[qs][r][0][0])[i];
        if (NORM == NORM_LN) kq = smk[qs][r];
    }
    __builtin_amdgcn_sched_barrier(0);
    float P[3][EU];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int e = 0; e < EU; ++e) {
            P[q][e] = tv[q][0][e];
#pragma unroll
            for (int w = 1; w < WPL; ++w) P[q][e] += tv[q][w][e];
        }
    float mu = 0.f, rs = 1.f;
    if (NORM != NORM_NONE) {
        float S1 = 0.f, S2 = 0.f;
#pragma unroll
        for (int i = 0; i < PK_WAVES / 2; ++i) {
            S1 += sv[i][0];
            S2 += sv[i][1];
            S1 += sv[i][2];
            S2 += sv[i][3];
        }
        const float st[3] = {kq, S1, S2};
        row_norm<NORM>(st, d, a.eps, mu, rs);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int e = 0; e < EU; ++e) {
            if (NG == 1) P[q][e] = xor16_sum(P[q][e]);
            P[q][e] = xor32_sum(P[q][e]);
        }
    // lane (g, cb): rows 4 g + e, column n; (mu, rstd) of a row read from
    // its lane (the same for the whole wave)
#pragma unroll
    for (int e = 0; e < EU; ++e) {
        const int m = 4 * g + e;
        float y = cn;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            float muq = 0.f, rq = 1.f;
            if (NORM != NORM_NONE) {
                muq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), MP * q + e));
                rq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), MP * q + e));
                if (NG == 2) {
                    const float mu1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), MP * q + 4 + e));
                    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), MP * q + 4 + e));
                    muq = g == 1 ? mu1 : muq;
                    rq = g == 1 ? r1 : rq;
                }
            }
            float pv = P[q][e];
            if (NORM == NORM_LN) pv -= muq * un[q];
            y += (NORM == NORM_NONE) ? pv : rq * pv;
        }
        if (m < M) a.out[(size_t)m * (size_t)a.rv.ld_out + n] = rv_ok(wr, m) ? (uint16_t)(pack_bf2(y, 0.f) & 0xffffu) : (uint16_t)0;
    }
}

// =====================================================================
// Column split: one 16-column block per wave over a K chunk
// =====================================================================
//
// Workgroup (group, chunk): NW waves, wave w owning column block NW group + w
// over the chunk's k-steps, so no wave's result needs another's and the
// workgroup ends without an LDS reduction.  The A tile of a k-step (MT
// 16-row tiles, loaded coalesced as in the split kernel) is needed by every
// wave, so it is loaded once per workgroup: in a group of NW k-steps wave w
// loads k-step w's tiles into registers two groups ahead and writes them,
// lane-linear, into one of two LDS stages one group ahead; one workgroup
// barrier per group (LDS only) separates the writes of a stage from its
// reads.  W' streams through a per-wave register ring RW k-steps deep.
// Chunks need not align with the states: a chunk that crosses a state
// boundary keeps the part before it in a second accumulator set.  The
// chunk counts make the grid one workgroup per CU.  After its loop a
// workgroup applies the statistics (gathered from the records the first 3M
// workgroups published) to its part(s), so that a chunk leaves one summable
// contribution, stored in fragment order (no re-layout); the last workgroup
// of a column group to arrive adds c and the contributions in chunk order.
constexpr int GN_RW = 8;     // W' ring: k-steps per wave
constexpr int GN_MAXCH = 8;  // K chunks, at most

template <int NORM, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void gemvn_kernel(GemvArgs a) {
    constexpr int ATILE = MT * 1024;   // bytes of one k-step's A tiles
    constexpr int GROUP = NW * ATILE;  // bytes of one group's (NW k-steps)
    constexpr int BODY = GN_RW > 2 * NW ? GN_RW : 2 * NW;  // k-steps per unrolled body: even groups, whole ring
    static_assert(BODY % GN_RW == 0 && BODY % (2 * NW) == 0, "ring and stages must be static in a body");
    __shared__ __attribute__((aligned(16))) char sa[2][GROUP];
    __shared__ float sh_mr[3 * GEMVN_MAX_M][2];  // (mu, rstd) of each (state, token) row
    __shared__ int sh_last;
    const int M = a.M, d = a.d;
    const int TS = d >> 5, T = 3 * TS;
    const int ngroups = d / (16 * NW), nch = a.nch, nwg = ngroups * nch;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware order: each XCD takes a contiguous range of (group, chunk) pairs
    const int per = (nwg + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    const WaveRows wr = rv_wave(a.rv, M);
    const bool producer = NORM != NORM_NONE && wave == 0 && (int)blockIdx.x < 3 * M;
    RowPre pre;
    if (producer) row_preload(stats_row(a, blockIdx.x, wr), d, lane, pre);
    if (lin >= nwg) {
        if (producer) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane, pre, wr);
        return;
    }
    const int grp = lin / nch, ch = lin - grp * nch;
    const int t0 = (ch * T) / nch, nsteps = T / nch;  // the plan makes nsteps a multiple of BODY
    const int s0 = t0 / TS;
    const int tsplit = min(t0 + nsteps, (s0 + 1) * TS);  // first k-step of the next state (or the end)
    const bool spans = tsplit < t0 + nsteps;
    const int n = 16 * (NW * grp + wave) + cb;  // this lane's output column
    const float us0 = NORM == NORM_LN && t0 == s0 * TS ? a.u[(size_t)s0 * d + n] : 0.f;
    const float us1 = NORM == NORM_LN && spans ? a.u[(size_t)(s0 + 1) * d + n] : 0.f;

    // A, by k-step pairs: in a group of NW k-steps wave w loads half
    // w % 2 (rows 8 MT (w % 2) ..) of the 16 MT token rows of pair w / 2, as
    // MT loads of 8 rows x 128 bytes (two k-steps), so that a load touches 8
    // whole cache lines (16 rows x 64 bytes touch 16 and cost the load units
    // about twice as much).  Load q of this lane: row 8 MT (w % 2) + 8 q +
    // lane / 8 (clamped to M - 1), chunk (lane % 8) ^ pair_swz(row); element
    // k of the pair starting at k-step t is at ap[state][q] + 32 t.  A pair
    // never crosses a state: chunks and states start at even k-steps.
    const uint16_t* ap0[MT];
    const uint16_t* ap1[MT];
    {
        const int s1 = min(s0 + 1, 2);
        const uint16_t* h0 = s0 == 0 ? a.h[0] : (s0 == 1 ? a.h[1] : a.h[2]);
        const uint16_t* h1 = s1 == 0 ? a.h[0] : (s1 == 1 ? a.h[1] : a.h[2]);
        const size_t ld0 = (size_t)rv_ld(a.rv, s0), ld1 = (size_t)rv_ld(a.rv, s1);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const int row = 8 * MT * (wave & 1) + 8 * q + (lane >> 3);
            const int c = (lane & 7) ^ pair_swz(row & 15);
            const size_t src = (size_t)rv_lane_src(a.rv, wr, min(row, M - 1));
            ap0[q] = h0 + src * ld0 - (size_t)s0 * d + 8 * c;
            ap1[q] = h1 + src * ld1 - (size_t)s1 * d + 8 * c;
        }
    }
    const int wpair = 2 * (wave >> 1);  // first k-step of this wave's pair in a group
    // this lane's part of the pair starting at k-step t
    auto aload = [&](int t, u32x4 (&x)[MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < MT; ++q)
            x[q] = *reinterpret_cast<const u32x4*>((t < tsplit ? ap0[q] : ap1[q]) + (size_t)32 * t);
    };
    // stage layout: pair p (of the group's NW / 2) at p 2048 MT bytes, row r at
    // + 128 r; each load lands 8 rows (1 KiB) contiguous
    auto awrite = [&](int stage, const u32x4 (&x)[MT]) __attribute__((always_inline)) {
        char* dst = sa[stage] + (wave >> 1) * (2048 * MT) + (8 * MT * (wave & 1)) * 128 + lane * 16;
#pragma unroll
        for (int q = 0; q < MT; ++q) *reinterpret_cast<u32x4*>(dst + q * 1024) = x[q];
    };
    const int ngrp = nsteps / NW;
    // fragment reads: row 16 tt + lane % 16, chunk lane / 16 of the pair's
    // first (aread0) or second (aread1) k-step
    const int aread0 = cb * 128 + 16 * (g ^ pair_swz(cb));
    const int aread1 = cb * 128 + 16 * ((4 + g) ^ pair_swz(cb));
    // prologue: A of groups 0 and 1 first (their writes to the stages wait
    // only for them: loads complete in issue order), then the W' ring, then
    // group 2's A in flight
    u32x4 ra[MT], rb[MT];
    aload(t0 + wpair, ra);
    aload(t0 + NW + wpair, rb);
    // W' tiles of this wave's column block, k-steps t0 ..
    const u32x4* __restrict__ wp = reinterpret_cast<const u32x4*>(a.wp) + ((size_t)(NW * grp + wave) * T + t0) * 64 + lane;
    u32x4 rw[GN_RW];
#pragma unroll
    for (int p = 0; p < GN_RW; ++p) rw[p] = __builtin_nontemporal_load(wp + (size_t)min(p, nsteps - 1) * 64);
    awrite(0, ra);
    awrite(1, rb);
    if (2 < ngrp) aload(t0 + 2 * NW + wpair, ra);
    __syncthreads();
    // the statistics row of this workgroup id, from the row loaded at the
    // start (the record needs no wait; the other waves run ahead to group 0's
    // barrier meanwhile)
    if (producer) stats_produce<NORM>(a, blockIdx.x, gridDim.x, lane, pre, wr);

    f32x4 acc[MT], accs[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) acc[tt] = accs[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // with one or two token tiles the statistics records (published long
    // before) are loaded at the start of the last body, beside its W' loads,
    // so the gather after the loop finds them in registers (measured: no gain
    // with four tiles, where the gather loads them itself)
    uint64_t pw0 = 0, pw1 = 0, pw2 = 0;
    for (int b0 = 0; b0 < nsteps; b0 += BODY) {
        if constexpr (MT <= 2) {
            if (b0 == nsteps - BODY) {
                const uint64_t* rp = a.rstats + 4 * min(64 * wave + lane, 3 * M - 1);
                pw0 = rec_load(rp);
                pw1 = rec_load(rp + 1);
                pw2 = rec_load(rp + 2);
            }
        }
#pragma unroll
        for (int gi = 0; gi < BODY / NW; ++gi) {
            const int G = b0 / NW + gi;  // group index
            const char* stg = sa[gi & 1];
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const int i = G * NW + j;  // step inside the chunk
                const int slot = (gi * NW + j) % GN_RW;
                const u32x4 bw = rw[slot];
                rw[slot] = __builtin_nontemporal_load(wp + (size_t)min(i + GN_RW, nsteps - 1) * 64);
                u32x4 af[MT];
#pragma unroll
                for (int tt = 0; tt < MT; ++tt)
                    af[tt] = *reinterpret_cast<const u32x4*>(stg + (j >> 1) * (2048 * MT) + tt * 2048 +
                                                             ((j & 1) ? aread1 : aread0));
                if (t0 + i == tsplit) {
#pragma unroll
                    for (int tt = 0; tt < MT; ++tt) {
                        accs[tt] = acc[tt];
                        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) acc[tt] = mfma16x16x32(af[tt], bw, acc[tt]);
            }
            // every wave has read this stage: refill it with group G + 2
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            if (G + 2 < ngrp) {
                awrite(gi & 1, ra);
                if (G + 3 < ngrp) aload(t0 + (G + 3) * NW + wpair, ra);
            }
        }
    }

    // statistics (published long before): wave w gathers rows 64 w ..
    // 64 w + 63 and turns each row's sums into (mu, rstd) for the workgroup
    if (NORM != NORM_NONE && 64 * wave < 3 * M)
        stats_gather_rows<NORM, (MT <= 2)>(a, lane, 64 * wave, sh_mr, wr, pw0, pw1, pw2);
    __syncthreads();
    // this wave's contribution of the chunk, sum over its state parts of
    // rstd_s (P - mu_s u_s) (P for no norm), fragment order, stored at the
    // device coherence point.  u_s sums the whole state, so mu_s u_s is
    // subtracted once per state: by the part that starts at the state's
    // first k-step (a part after a boundary always does).
    const bool first0 = t0 == s0 * TS;
    f32x4 y[MT];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = min(16 * tt + 4 * g + e, M - 1);
            float v = spans ? accs[tt][e] : acc[tt][e];
            if (NORM != NORM_NONE) {
                const float mu = sh_mr[s0 * M + m][0], r = sh_mr[s0 * M + m][1];
                v = r * (NORM == NORM_LN && first0 ? v - mu * us0 : v);
            }
            if (spans) {
                float v1 = acc[tt][e];
                if (NORM != NORM_NONE) {
                    const int s1 = s0 + 1;
                    const float mu = sh_mr[s1 * M + m][0], r = sh_mr[s1 * M + m][1];
                    v1 = r * (NORM == NORM_LN ? v1 - mu * us1 : v1);
                }
                v += v1;
            }
            y[tt][e] = v;
        }
    const size_t wtile = (size_t)MT * 64;  // f32x4 of one wave's part
    auto part_base = [&](int c) { return a.part + (((size_t)grp * nch + c) * NW + wave) * wtile * 4; };
    {
        const __amdgpu_buffer_rsrc_t rs = part_rsrc(part_base(ch), (int)(wtile * 16));
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) store_coherent16(rs, (tt * 64 + lane) * 16, __builtin_bit_cast(u32x4, y[tt]));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (old == nch - 1);
    }
    __syncthreads();
    if (!sh_last) return;

    // ================= last arriver of column group grp =================
    // wave w: column block NW grp + w; the chunks' contributions, summed in
    // chunk order, in batches of up to 4 token tiles whose loads are all
    // issued before the first is used (one round trip per batch)
    const float cn = a.c[n];
    constexpr int TB = MT < 4 ? MT : 4;
#pragma unroll
    for (int tb = 0; tb < MT; tb += TB) {
        // (loads unconditional, chunks past nch re-reading the last one and
        // dropped below: a load under a branch would get a wait of its own)
        u32x4 v[GN_MAXCH][TB];
#pragma unroll
        for (int c = 0; c < GN_MAXCH; ++c) {
            const __amdgpu_buffer_rsrc_t rs = part_rsrc(part_base(min(c, nch - 1)), (int)(wtile * 16));
#pragma unroll
            for (int k = 0; k < TB; ++k)
                if (tb + k < MT) v[c][k] = load_coherent16(rs, ((tb + k) * 64 + lane) * 16);
        }
        f32x4 tot[TB];
#pragma unroll
        for (int k = 0; k < TB; ++k) tot[k] = f32x4{cn, cn, cn, cn};
#pragma unroll
        for (int c = 0; c < GN_MAXCH; ++c)
            if (c < nch)
#pragma unroll
                for (int k = 0; k < TB; ++k)
                    if (tb + k < MT) tot[k] += __builtin_bit_cast(f32x4, v[c][k]);
#pragma unroll
        for (int k = 0; k < TB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * (tb + k) + 4 * g + e;
                if (tb + k < MT && m < M)
                    a.out[(size_t)m * (size_t)a.rv.ld_out + n] =
                        rv_ok(wr, m) ? (uint16_t)(pack_bf2(tot[k][e], 0.f) & 0xffffu) : (uint16_t)0;
            }
    }
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- host side
GemvPlan plan_gemv(int M, int d, int norm) {
    (void)norm;
    GemvPlan p;
    p.MT = (M + 15) / 16;
    const int T3 = d / 32;
    // up to 6 tokens where each wave's k-steps per state are a multiple of 8
    // (d = 2048, 4096): the packed-block whole-K kernel; one token also where
    // its grid is whole rounds of the CUs (d = 8192: 64.5 us against 67.9 on
    // the split kernel; from two tokens on the column split is as fast there)
    if (M <= PK_MAXM && d % (32 * PK_WAVES) == 0 && (d <= 4096 || (M == 1 && (d / 16) % 256 == 0)) &&
        (d / 32 / PK_WAVES) % PK_R == 0) {
        const int JS = T3 / PK_WAVES;
        int mp = 1;
        while (mp < M) mp <<= 1;
        p.pack = 1;
        p.sb = std::min(16 / mp, JS);
        p.ring = pk_ring(p.sb, d);
        p.waves = PK_WAVES;
        p.kps = 1;
        p.nb = 1;
        p.grid = d / 16;
        p.counters_bytes = 256;
        p.part_bytes = 256;
        return p;
    }
    // a handful of tokens: the whole-K kernel when its token rows fit in LDS
    // (one workgroup per 16-column block, at most one round of the CUs)
    if (M <= WH_MAXM && d <= 4096 && d % (32 * WH_WAVES) == 0 && M * (6 * d + 64) <= WH_A_BYTES) {
        const int JS = T3 / WH_WAVES;
        int ring = 8;
        while (ring > 1 && (JS % ring || JS < ring)) ring >>= 1;
        if (JS % ring == 0 && JS >= ring) {
            p.whole = 1;
            p.ring = ring;
            p.waves = WH_WAVES;
            p.kps = 1;
            p.nb = 1;
            p.grid = d / 16;
            p.counters_bytes = 256;
            p.part_bytes = 256;
            return p;
        }
    }
    // The column-split kernel: 8 waves (128 columns) per workgroup and the
    // most K chunks that keep the grid at one workgroup per CU, each chunk a
    // whole number of unrolled bodies (k-steps); at least 128 workgroups.
    if (M >= 2 && M <= GEMVN_MAX_M) {
        constexpr int NW = 8;
        const int body = std::max(GN_RW, 2 * NW);
        const int ngroups = d / (16 * NW);
        int best = 0;
        if (d % (16 * NW) == 0)
            for (int nch = 1; nch <= GN_MAXCH && ngroups * nch <= 256; ++nch)
                if (T3 * 3 % (nch * body) == 0) best = nch;
        if (best > 0 && ngroups * best >= 128) {
            p.cols = 1;
            p.nch = best;
            p.waves = NW;
            p.nb = NW;
            p.kps = 1;
            p.grid = ngroups * best;
            p.counters_bytes = ((size_t)ngroups * sizeof(int) + 255) / 256 * 256;
            p.part_bytes = ((size_t)ngroups * best * NW * p.MT * 64 * 16 + 255) / 256 * 256;
            return p;
        }
    }
    if (M > DECODE_MAX_M) return GemvPlan{};  // more tokens: the column split or nothing (prefill)
    // Column blocks per workgroup: 8 (128 columns) from two token tiles on,
    // which halves how often the workgroups re-read the hidden states; the
    // wider tile then keeps fewer k-steps in flight (registers).
    for (int nb : {8, 4}) {
        if (nb == 8 && (p.MT < 2 || d % 128)) continue;
        const int ngroups = d / (16 * nb);
        const int rmax = nb == 4 ? (p.MT >= 3 ? 2 : 4) : (p.MT >= 4 ? 1 : 2);
        // the most waves (8, 4, 2, 1; 128 columns need 2) that split a chunk
        // evenly; then the chunks per state that bring the workgroup count
        // nearest one per CU, each wave taking a multiple of the ring depth
        int best = -1;
        for (int waves : {8, 4, 2, 1}) {
            if (64 * waves < 16 * nb) continue;
            for (int kps : {1, 2, 4, 8}) {
                if (T3 % (kps * waves)) continue;
                const int nw = T3 / (kps * waves);
                int ring = rmax;
                while (nw % ring) ring >>= 1;
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
        if (best < 0) continue;
        p.nb = nb;
        p.grid = ngroups * 3 * p.kps;
        p.counters_bytes = ((size_t)ngroups * sizeof(int) + 255) / 256 * 256;
        const size_t slots = (size_t)ngroups * 3 * p.kps;
        p.part_bytes = (slots * (size_t)p.MT * 16 * 16 * nb * sizeof(float) + 255) / 256 * 256;
        return p;
    }
    return p;
}

template <int NORM, int MT, int NB, int R>
static hipError_t launch_split(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    // A ring: as deep as W's, but two steps for three or four token tiles
    // (registers)
    constexpr int RA = (MT >= 3 && R > 2) ? 2 : R;
    const int grid = ((p.grid + 7) / 8) * 8;
    gemv_split_kernel<NORM, MT, NB, R, RA><<<grid, 64 * p.waves, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM, int MT, int NB>
static hipError_t launch_split_r(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.ring) {
        case 4:
            if constexpr (NB == 4) return launch_split<NORM, MT, NB, 4>(a, p, st);
            return hipErrorInvalidValue;
        case 2: return launch_split<NORM, MT, NB, 2>(a, p, st);
        case 1: return launch_split<NORM, MT, NB, 1>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NORM>
static hipError_t launch_gn(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    if (p.nb == 8) {
        switch (p.MT) {
            case 2: return launch_split_r<NORM, 2, 8>(a, p, st);
            case 3: return launch_split_r<NORM, 3, 8>(a, p, st);
            case 4: return launch_split_r<NORM, 4, 8>(a, p, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.MT) {
        case 1: return launch_split_r<NORM, 1, 4>(a, p, st);
        case 2: return launch_split_r<NORM, 2, 4>(a, p, st);
        case 3: return launch_split_r<NORM, 3, 4>(a, p, st);
        case 4: return launch_split_r<NORM, 4, 4>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

// token-row slots staged per workgroup: 1 or 2 (d <= 4096)
template <int NORM, int R>
static hipError_t launch_whole_mm(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    if (a.M == 1)
        gemv_whole_kernel<NORM, R, 1><<<p.grid, 64 * WH_WAVES, 0, st>>>(a);
    else
        gemv_whole_kernel<NORM, R, 2><<<p.grid, 64 * WH_WAVES, 0, st>>>(a);
    return hipGetLastError();
}

template <int NORM>
static hipError_t launch_whole(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.ring) {
        case 8: return launch_whole_mm<NORM, 8>(a, p, st);
        case 4: return launch_whole_mm<NORM, 4>(a, p, st);
        case 2: return launch_whole_mm<NORM, 2>(a, p, st);
        case 1: return launch_whole_mm<NORM, 1>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NORM>
static hipError_t launch_cols(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    const int grid = ((p.grid + 7) / 8) * 8;
    switch (p.MT) {
        case 1: gemvn_kernel<NORM, 1, 8><<<grid, 512, 0, st>>>(a); break;
        case 2: gemvn_kernel<NORM, 2, 8><<<grid, 512, 0, st>>>(a); break;
        case 3: gemvn_kernel<NORM, 3, 8><<<grid, 512, 0, st>>>(a); break;
        case 4: gemvn_kernel<NORM, 4, 8><<<grid, 512, 0, st>>>(a); break;
        case 5: gemvn_kernel<NORM, 5, 8><<<grid, 512, 0, st>>>(a); break;
        case 6: gemvn_kernel<NORM, 6, 8><<<grid, 512, 0, st>>>(a); break;
        case 7: gemvn_kernel<NORM, 7, 8><<<grid, 512, 0, st>>>(a); break;
        case 8: gemvn_kernel<NORM, 8, 8><<<grid, 512, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int NORM>
static hipError_t launch_pack(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
    switch (p.sb) {
        case 16:
            if (p.ring == 16) gemv_pack_kernel<NORM, 16, 16><<<p.grid, 64 * PK_WAVES, 0, st>>>(a);
            else gemv_pack_kernel<NORM, 16, PK_R><<<p.grid, 64 * PK_WAVES, 0, st>>>(a);
            break;
        case 8: gemv_pack_kernel<NORM, 8, PK_R><<<p.grid, 64 * PK_WAVES, 0, st>>>(a); break;
        case 4: gemv_pack_kernel<NORM, 4, PK_R><<<p.grid, 64 * PK_WAVES, 0, st>>>(a); break;
        case 2: gemv_pack_kernel<NORM, 2, PK_R><<<p.grid, 64 * PK_WAVES, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a, int norm, const GemvPlan& p, hipStream_t st) {
    if (p.pack) {
        // the kernel's fixed shape: k-steps per wave and state a multiple of
        // its ring and of its body (max(sb, ring) steps), every token a row
        // slot (16 / sb of them), one workgroup per 16-column block
        const int JS = a.d / 32 / PK_WAVES, body = std::max(p.sb, p.ring);
        if (a.M < 1 || a.M > PK_MAXM || (a.d > 4096 && (a.M != 1 || (a.d / 16) % 256)) || a.d % (32 * PK_WAVES) || p.sb < 2 || p.sb > 16 ||
            a.M > 16 / p.sb || (p.ring != PK_R && !(p.ring == 16 && p.sb == 16)) || JS % body || p.sb > JS || p.grid != a.d / 16)
            return hipErrorInvalidValue;
        if (norm == NORM_LN) return launch_pack<NORM_LN>(a, p, st);
        if (norm == NORM_RMS) return launch_pack<NORM_RMS>(a, p, st);
        return launch_pack<NORM_NONE>(a, p, st);
    }
    if (p.cols) {
        const int T = 3 * a.d / 32, body = std::max(GN_RW, 16);
        if (p.waves != 8 || a.nch != p.nch || p.nch < 1 || p.nch > GN_MAXCH || a.d % 128 || T % (p.nch * body) ||
            a.M < 2 || a.M > GEMVN_MAX_M || (p.MT - 1) * 16 >= a.M || p.MT * 16 < a.M ||
            (long long)(a.d / 128) * p.nch != p.grid)
            return hipErrorInvalidValue;
        if (norm == NORM_LN) return launch_cols<NORM_LN>(a, p, st);
        if (norm == NORM_RMS) return launch_cols<NORM_RMS>(a, p, st);
        return launch_cols<NORM_NONE>(a, p, st);
    }
    if (p.whole) {
        if (a.M < 1 || a.M > WH_MAXM || a.d > 4096 || a.M * (6 * a.d + 64) > WH_A_BYTES || a.d % (32 * WH_WAVES) ||
            p.grid != a.d / 16 || (a.d / 32 / WH_WAVES) % p.ring || a.d / 32 / WH_WAVES < p.ring)
            return hipErrorInvalidValue;
        if (norm == NORM_LN) return launch_whole<NORM_LN>(a, p, st);
        if (norm == NORM_RMS) return launch_whole<NORM_RMS>(a, p, st);
        return launch_whole<NORM_NONE>(a, p, st);
    }
    if (p.waves < 1 || p.waves > GV_WAVES || a.waves != p.waves || a.M < 1 || a.M > DECODE_MAX_M ||
        64 * p.waves < 16 * p.nb || a.d % (16 * p.nb))
        return hipErrorInvalidValue;
    if (p.kps < 1 || a.kps != p.kps) return hipErrorInvalidValue;
    if (norm == NORM_LN) return launch_gn<NORM_LN>(a, p, st);
    if (norm == NORM_RMS) return launch_gn<NORM_RMS>(a, p, st);
    return launch_gn<NORM_NONE>(a, p, st);
}

}  // namespace e31
