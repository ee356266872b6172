// Prefill path of the fused per-state norm + FC (many tokens): a bf16 MFMA
// GEMM on the raw hidden states and the folded weight W'.
//
// With the norm parameters folded into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the parameters are absorbed by the FC),
//     out = sum_s rstd_s * (h_s . W'_s^T - mu_s * u_s) + c,
// so the main loop is a plain GEMM over the three states in turn.  The
// accumulator is scaled per row by rstd_s / rstd_{s+1} at each state
// boundary, so it ends as sum_s rstd_s h_s . W'_s; the epilogue multiplies by
// rstd_2 and subtracts the rank-3 mean term sum_s (rstd_s mu_s) u_s before
// adding c.  The statistics come from the row-statistics pass that runs
// first.
//
// Tiling for gfx950: 256 x 256 output tile, 256 threads (4 waves as 2 x 2,
// each wave 128 x 128 = 8 x 8 MFMA 16x16x32 blocks, whose 256 accumulator
// registers the compiler keeps in AGPRs), k in sub-tiles of 32 (one MFMA
// k-step) through four 32 KiB LDS stages.  Operands go from global memory
// straight to LDS (16-byte LDS-DMA loads, no register staging).  A (hidden
// states, row-major) lands as 16-row x 64-byte blocks, one per wave load;
// its 16-byte chunks are XOR-swizzled by (row / 4) mod 4 on the global side,
// so the 16 rows of a fragment read hit distinct banks.  W' arrives as 1 KiB
// MFMA B-fragment tiles (16 columns x 32 k, lane l's operand at bytes
// [16 l, 16 l + 16)), copied to LDS as they are, so a B operand is one
// conflict-free 16-byte read.  Each sub-step issues the loads of the
// sub-tile needed 2-3 sub-steps later.  Tiles are walked in groups of 4
// M-tiles, and consecutive workgroup ids are spread so that each XCD
// (workgroup id mod 8) takes a contiguous run of that order: the tiles an
// XCD runs at once share A and B tiles in its L2.
// Few tiles (small M) split K into chunks, each inside one state (or, with 43
// to 64 tiles, four equal chunks across the states, which store one partial
// per state part); the partials go to the workspace and a reduction kernel
// launched next on the stream sums each state's parts in a fixed order and
// applies the statistics.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int PBM = 256, PBN = 256, PBK = 32, PTH = 256;  // PBK: k per sub-tile (one MFMA k-step)
constexpr int PGM = 4;   // M-tiles per raster group
constexpr int STAGE_A = PBM * PBK * 2;              // A part of a stage (16 KiB)
constexpr int STAGE_BYTES = (PBM + PBN) * PBK * 2;  // A then B (32 KiB)
// s_waitcnt immediates: vmcnt <= n with lgkmcnt = 0; lgkmcnt = 0 alone
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// LDS-DMA loads written as inline asm, so that the compiler sees no vector
// memory operation in the main loop: it then inserts no waits of its own
// (its alias analysis cannot always separate the stage a load writes from the
// stage being read), and the explicit waits, derived from the fixed issue
// order, are the only ones.  The asm writes M0, which nothing else in the
// kernel uses.  16 bytes per lane from sbase + voff (sbase wave-uniform) to
// LDS byte lds + 16 lane:
// (readfirstlane pins the wave-uniform operands to scalar registers; the
// compiler drops it where they already are)
__device__ __forceinline__ uint64_t uniform64(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(uniform64(sbase))
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// x >= y ? a : b on the scalar unit (wave-uniform operands): a compare and a
// select, where the compiler would otherwise branch or build a lookup table
__device__ __forceinline__ uint64_t sel_ge(int x, int y, uint64_t a, uint64_t b) {
    uint64_t r;
    asm("s_cmp_ge_i32 %1, %2\n\ts_cselect_b64 %0, %3, %4" : "=s"(r) : "s"(x), "s"(y), "s"(a), "s"(b) : "scc");
    return r;
}

// Stores one lane's part of a 16 x 16 fp32 block as bf16.  Lane (g, cb) holds
// rows row0 + e (e < 4; row0 = block row + 4 g) of column col0 + cb.  Two
// exchanges inside each quad of lanes (cb = 4 k + t; partners t ^ 1, then
// t ^ 2) leave lane t with one row, row0 + (((t & 1) << 1) | (t >> 1)), and
// the quad's 4 columns col0 + 4 k .. + 3: one 8-byte store, no staging
// through LDS.  Rows from M and columns from d on are not stored; output
// rows are ldo elements apart; row row0 + e is stored as zeros unless bit e
// of okbits is set.
__device__ __forceinline__ void store_block_bf16(uint16_t* out, int M, int d, long long ldo, int row0, int col0,
                                                 int cb, uint32_t okbits, float v0, float v1, float v2, float v3) {
    const int t = cb & 3, k4 = cb >> 2;
    const bool odd = (t & 1) != 0, hi = t >= 2;
    auto swap1 = [](float x) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    };
    auto swap2 = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false); };
    // even lanes keep rows 0, 1 and odd lanes rows 2, 3 of the pair's two columns
    const float r0 = swap1(odd ? v0 : v2), r1 = swap1(odd ? v1 : v3);
    const uint32_t P0 = odd ? pack_bf2(r0, v2) : pack_bf2(v0, r0);
    const uint32_t P1 = odd ? pack_bf2(r1, v3) : pack_bf2(v1, r1);
    // then each lane keeps one row of the quad's four columns
    const uint32_t rv = swap2(hi ? P0 : P1);
    const int e = ((t & 1) << 1) | (t >> 1);
    const uint32_t keep = 0u - ((okbits >> e) & 1u);  // all ones, or zero for a token stored as zeros
    const uint2 w0 = hi ? make_uint2(rv, P1) : make_uint2(P0, rv);
    const uint2 w = make_uint2(w0.x & keep, w0.y & keep);
    const int m = row0 + e;
    const int n = col0 + 4 * k4;
    if (m < M && n < d) *reinterpret_cast<uint2*>(out + (size_t)m * (size_t)ldo + n) = w;
}

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

// ULD: the three states share one row pitch, so each lane's A offsets are
// computed once (the same for every state); otherwise they are formed at each
// load from the lane's source row and the pitch of the state being loaded.
template <bool SPLIT, int NORM, bool ULD>
__global__ __launch_bounds__(PTH, 1) void prefill_kernel(PrefillArgs a, int TM, int TN) {
    // four stages in separate arrays: with static stage indices the compiler
    // can tell the LDS-DMA writes of one stage from the reads of another
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st3[STAGE_BYTES];
    // per-row factors of the tile: mu_0, rstd_0/rstd_1, mu_1, rstd_1/rstd_2, mu_2, rstd_2,
    // then 1 / 0 for a token whose output row is stored / zeroed;
    // per-column factors: u_0, u_1, u_2, c
    __shared__ float rowf[7][PBM];
    __shared__ float colf[4][PBN];
    // end of a sub-step: the stage of sub-tile u + 2 has landed, i.e. all but
    // the newest 2 stages of loads (8 per wave each) are complete
    constexpr int WAIT_STAGE = wait_vm(16);

    const TileCoord tc = map_tile(blockIdx.x, TM, TN, SPLIT ? a.chunks : 1);
    if (!tc.valid) return;
    const int M = a.M, d = a.d;
    const int m0 = tc.mt * PBM, n0 = tc.nt * PBN;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cb = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave bases stay scalar
    const int wm = wave >> 1, wn = wave & 1;
    const int KTS = d / PBK;  // sub-tiles per state
    int kt0 = 0, kt1 = 3 * KTS;
    if (SPLIT && a.chunks != a.splits) {
        // four equal chunks across the states (sub-tiles 3 KTS c / 4 ..): each
        // state gets two parts, the first from the state's start
        kt0 = (tc.chunk * 3 * KTS) / 4;
        kt1 = ((tc.chunk + 1) * 3 * KTS) / 4;
    } else if (SPLIT) {
        const int kps = a.splits / 3;
        const int s = tc.chunk / kps, j = tc.chunk - s * kps;
        kt0 = s * KTS + (j * KTS) / kps;
        kt1 = s * KTS + ((j + 1) * KTS) / kps;
    }

    // Loads of a stage (16 A blocks and 16 B tiles of 1 KiB; wave w issues
    // A blocks and B tiles 4 w .. 4 w + 3), one LDS-DMA instruction each:
    //  A block ab: rows 16 ab + lane / 4, LDS chunk lane % 4 holds global
    //  chunk (lane % 4) ^ ((row / 4) % 4); rows past M re-read row M - 1.
    //  B tile bt: column block n0 / 16 + bt (clamped), k-step u.
    // Addresses are a wave-uniform base plus a 32-bit per-lane byte offset:
    // for A, the lane's source row times the state's row pitch (rows relative
    // to the tile's first without an index list, absolute with one) plus its
    // chunk.
    const int T = 3 * KTS;  // tiles per column block
    const int nblk = d >> 4;
    const bool indexed = a.rv.idx != nullptr;
    uint32_t arow[4], acol[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 16 * (4 * wave + q) + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        const int m = min(m0 + r, M - 1);
        bool ok;
        arow[q] = indexed ? (uint32_t)rv_src(a.rv, m, ok) : (uint32_t)(m - m0);
        acol[q] = (uint32_t)(16 * c);
        if (ULD) acol[q] += arow[q] * (uint32_t)(a.rv.ld[0] * 2);  // the whole offset, once
    }
    const char* wbase = reinterpret_cast<const char*>(a.wt);
    const uint32_t boff = (uint32_t)lane * 16u;
    // per-state A bases (the tile's first row, or row 0 with an index list),
    // each less its state's first k, so that sub-tile u of state s starts at
    // base_s + 64 u bytes: two compare-and-selects, no branches
    const uint64_t hb0 = (uint64_t)(uintptr_t)(a.h[0] + (indexed ? 0 : (size_t)m0 * (size_t)a.rv.ld[0]));
    const uint64_t hb1 = (uint64_t)(uintptr_t)(a.h[1] + (indexed ? 0 : (size_t)m0 * (size_t)a.rv.ld[1])) - (uint64_t)d * 2u;
    const uint64_t hb2 = (uint64_t)(uintptr_t)(a.h[2] + (indexed ? 0 : (size_t)m0 * (size_t)a.rv.ld[2])) - (uint64_t)d * 4u;
    auto a_state = [&](int u) __attribute__((always_inline)) { return u >= 2 * KTS ? 2 : (u >= KTS ? 1 : 0); };
    auto a_src = [&](int u) __attribute__((always_inline)) {
        const uint64_t b = sel_ge(u, 2 * KTS, hb2, sel_ge(u, KTS, hb1, hb0));
        return reinterpret_cast<const char*>(b + (uint64_t)u * (PBK * 2));
    };
    // row pitch of sub-tile u's state in bytes (the host keeps the offsets below 2^32)
    auto a_pitch = [&](int u) __attribute__((always_inline)) {
        return ULD ? 0u : (uint32_t)__builtin_amdgcn_readfirstlane((int)(rv_ld(a.rv, a_state(u)) * 2));
    };
    // load c (< 8) of the wave's share of sub-tile u into stage sa; hs = a_src(u), ap = a_pitch(u)
    auto issue_one = [&](int u, const char* hs, uint32_t ap, char* sa, int c) __attribute__((always_inline)) {
        if (c < 4) {
            dma16(hs, ULD ? acol[c] : arow[c] * ap + acol[c], lds_addr(sa + (4 * wave + c) * 1024));
        } else {
            const int bt = 4 * wave + (c - 4);
            const int nb = min((n0 >> 4) + bt, nblk - 1);
            dma16(wbase + (((size_t)nb * T + u) << 10), boff, lds_addr(sa + STAGE_A + bt * 1024));
        }
    };

    // fragment reads: A row wm 128 + 16 i + lane % 16, chunk lane / 16; the
    // swizzle (row / 4) % 4 is the same for the 8 row blocks, so one base and
    // an immediate offset of 1024 i bytes.  B tile wn 8 + j, lane's 16 bytes.
    const uint32_t aread = (uint32_t)((wm * 128 + cb) * 64 + 16 * (g ^ ((cb >> 2) & 3)));
    const uint32_t bread = (uint32_t)(STAGE_A + wn * 8192) + (uint32_t)lane * 16u;

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (tid < PBM) {
        const int m = m0 + tid;
        bool tok_ok = false;
        if (m < M) (void)rv_src(a.rv, m, tok_ok);
        rowf[6][tid] = tok_ok ? 1.f : 0.f;
        float r[3] = {1.f, 1.f, 1.f}, mu[3] = {0.f, 0.f, 0.f};
        if (m < M && NORM != NORM_NONE) {
#pragma unroll
            for (int q = 0; q < 3; ++q) r[q] = a.rstd[(size_t)q * M + m];
            if (NORM == NORM_LN)
#pragma unroll
                for (int q = 0; q < 3; ++q) mu[q] = a.mu[(size_t)q * M + m];
        }
        float f[6];
        if (SPLIT) {
            // mu_0, rstd_0, mu_1, rstd_1, mu_2, rstd_2
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                f[2 * q] = mu[q];
                f[2 * q + 1] = r[q];
            }
        } else {
            // rstd_0/rstd_1, rstd_1/rstd_2, rstd_2, rstd_0 mu_0, rstd_1 mu_1, rstd_2 mu_2
            f[0] = r[0] / r[1];
            f[1] = r[1] / r[2];
            f[2] = r[2];
#pragma unroll
            for (int q = 0; q < 3; ++q) f[3 + q] = r[q] * mu[q];
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

    // Without split-K the accumulator carries sum_s rstd_s h_s . W'_s: at the
    // end of state s (s < 2) it is scaled per row by rstd_s / rstd_{s+1}; the
    // mean terms, sum_s rstd_s mu_s u_s, are subtracted in the epilogue.
    auto rescale = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float fac = rowf[s][wm * 128 + 16 * i + 4 * g + e];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j][e] *= fac;
            }
        }
    };

    // Pipeline of one state (sub-tiles ua .. ub-1) over four stages; stage v
    // (mod 4) of the state holds sub-tile ua + v.  Sub-step u, with F(u) (its
    // 8 A and 8 B operands) already in registers:
    //   64 MFMAs on F(u); between them, the 16 reads of F(u + 1), one per 4
    //   MFMAs, and the 8 loads of sub-tile u + 4 into the stage of u (free:
    //   every wave read F(u) before the last barrier), one per 8; then
    //   wait for the stage of u + 2 and the reads; barrier.
    // A stage is needed 2 to 3 sub-steps after its loads are issued.  The
    // barrier is a bare s_barrier (the explicit wait covers what it needs).
    // Each sub-step issues exactly 8 loads per wave, so one vmcnt bound fits
    // every wait; near the end of a state the loads re-read the last sub-tile
    // and the reads may fetch a stale stage: harmless, and the body has no
    // branches.
    u32x4 fA[2][8], fB[2][8];  // two register sets of operands
    // read c of sub-tile operands (c < 8: B operand c, else A operand c - 8)
    auto read_one = [&](const char* sa, int set, int c) __attribute__((always_inline)) {
        if (c < 8)
            fB[set][c] = *reinterpret_cast<const u32x4*>(sa + bread + c * 1024);
        else
            fA[set][c - 8] = *reinterpret_cast<const u32x4*>(sa + aread + 1024 * (c - 8));
    };
    auto sub_step = [&](int u, int lim, char* cur, char* nxt, int set) __attribute__((always_inline)) {
        // F(u) has landed (read during the previous sub-step)
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
        const int un = min(u + 4, lim - 1);
        const char* hs = a_src(un);
        const uint32_t ap = a_pitch(un);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if ((c & 1) == 0) issue_one(un, hs, ap, cur, c >> 1);
            read_one(nxt, set ^ 1, c);
            const int i = c >> 1;
#pragma unroll
            for (int j = 4 * (c & 1); j < 4 * (c & 1) + 4; ++j)
                acc[i][j] = mfma16x16x32(fA[set][i], fB[set][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(WAIT_STAGE);
        asm volatile("s_barrier" ::: "memory");
    };
    // When every state's sub-tile count is a multiple of 4 (and always for a
    // split-K chunk: one inside a state, or one of four across the states with
    // every part a multiple of 4), the pipeline runs on across the state
    // boundaries: the loads near the end of a state already fetch the next one
    // and each state starts on stage 0 again.  Otherwise it restarts at every
    // state.
    const bool cont = SPLIT || (KTS & 3) == 0;
    // a split chunk's partial of state s's part starting at sub-tile ua, in
    // fragment order (rows from M on are skipped); slot: the chunk, or with
    // chunks across the states 2 s + (0 for the part that starts the state)
    auto store_part = [&](int s, int ua) __attribute__((always_inline)) {
        const int tile = tc.mt * TN + tc.nt;
        const int slot = a.chunks != a.splits ? 2 * s + (ua == s * KTS ? 0 : 1) : tc.chunk;
        const size_t frag_per_wg = (size_t)PTH * 64;  // f32x4 per (tile, slot)
        f32x4* mine = reinterpret_cast<f32x4*>(a.part) + ((size_t)tile * a.splits + slot) * frag_per_wg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (m0 + wm * 128 + 16 * i >= M) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) mine[((size_t)(i * 8 + j) * 4 + wave) * 64 + lane] = acc[i][j];
        }
    };
    for (int s = kt0 / KTS; s < 3 && s * KTS < kt1; ++s) {
        const int ua = max(kt0, s * KTS), ub = min(kt1, (s + 1) * KTS);
        const int lim = cont ? kt1 : ub;  // loads stay below lim
        if (!cont || ua == kt0) {
            // prologue: sub-tiles ua .. ua+3 (clamped) into stages 0..3
            char* const stv[4] = {st0, st1, st2, st3};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int uv = min(ua + v, lim - 1);
                const char* hs = a_src(uv);
                const uint32_t ap = a_pitch(uv);
#pragma unroll
                for (int c = 0; c < 8; ++c) issue_one(uv, hs, ap, stv[v], c);
                __builtin_amdgcn_sched_barrier(0);
            }
            // stages 0 and 1 have landed; F(ua) from stage 0
            __builtin_amdgcn_s_waitcnt(WAIT_STAGE);
            asm volatile("s_barrier" ::: "memory");
#pragma unroll
            for (int c = 0; c < 16; ++c) read_one(st0, 0, c);
            // every wave has its F(ua) before sub-step ua reloads stage 0
            __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
            asm volatile("s_barrier" ::: "memory");
        }
        for (int u = ua; u < ub; u += 4) {
            sub_step(u, lim, st0, st1, 0);
            if (u + 1 < ub) sub_step(u + 1, lim, st1, st2, 1);
            if (u + 2 < ub) sub_step(u + 2, lim, st2, st3, 0);
            if (u + 3 < ub) sub_step(u + 3, lim, st3, st0, 1);
        }
        if (!SPLIT && NORM != NORM_NONE && s < 2) rescale(s);
        if (SPLIT && ub < kt1) {
            // a chunk across the states: this state's part is done
            store_part(s, ua);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // the last sub-steps' loads (re-reads near the end) land before the
    // workgroup can end and its LDS be handed to another
    __builtin_amdgcn_s_waitcnt(0);

    if (SPLIT) {
        // the chunk's (last) partial; the reduction kernel that runs next on
        // the stream sums each state's parts in order
        const int sl = (kt1 - 1) / KTS;
        store_part(sl, max(kt0, sl * KTS));
        return;
    }

    // y = acc rstd_2 - sum_s (rstd_s mu_s) u_s + c, rounded to bf16
    float cc[8], uu[3][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int col = wn * 128 + 16 * j + cb;
        cc[j] = colf[3][col];
#pragma unroll
        for (int q = 0; q < 3; ++q) uu[q][j] = NORM == NORM_LN ? colf[q][col] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float r2[4], rm[3][4];
        uint32_t okbits = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = wm * 128 + 16 * i + 4 * g + e;
            okbits |= rowf[6][rr] > 0.5f ? (1u << e) : 0u;
            r2[e] = NORM != NORM_NONE ? rowf[2][rr] : 1.f;
#pragma unroll
            for (int q = 0; q < 3; ++q) rm[q][e] = NORM == NORM_LN ? rowf[3 + q][rr] : 0.f;
        }
        auto fin = [&](float x, int j, int e) __attribute__((always_inline)) {
            float y = x * r2[e] + cc[j];
            if (NORM == NORM_LN) y -= rm[0][e] * uu[0][j] + rm[1][e] * uu[1][j] + rm[2][e] * uu[2][j];
            return y;
        };
#pragma unroll
        for (int j = 0; j < 8; ++j)
            store_block_bf16(a.out, M, d, a.rv.ld_out, m0 + wm * 128 + 16 * i + 4 * g, n0 + wn * 128 + 16 * j, cb,
                             okbits, fin(acc[i][j][0], j, 0), fin(acc[i][j][1], j, 1), fin(acc[i][j][2], j, 2),
                             fin(acc[i][j][3], j, 3));
    }
}

// Split-K reduction: one wave per fragment group (tile, i, j, wave of the
// main kernel), whose 64 lanes hold the same rows and columns as in the main
// kernel.  y = sum_s rstd_s (sum over the chunks of state s, in their order,
// - mu_s u_s) + c, stored through the same quad exchange.  It runs after the
// main kernel on the stream, so plain loads see the partials.
template <int NORM, int KPS>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs a, int TM, int TN) {
    const int lane = threadIdx.x & 63, g = lane >> 4, cb = lane & 15;
    const int fg = blockIdx.x * 4 + (threadIdx.x >> 6);  // 256 fragment groups per tile
    const int tile = fg >> 8;
    if (tile >= TM * TN) return;
    const int ij = (fg >> 2) & 63, w = fg & 3;
    const int i = ij >> 3, j = ij & 7, wm = w >> 1, wn = w & 1;
    const int mt = tile / TN, nt = tile - mt * TN;
    const int M = a.M, d = a.d;
    const int row0 = mt * PBM + wm * 128 + 16 * i + 4 * g;
    if (mt * PBM + wm * 128 + 16 * i >= M) return;  // whole wave: rows the main kernel did not store
    const int col = nt * PBN + wn * 128 + 16 * j + cb;
    const int splits = a.splits;  // 3 KPS
    const f32x4* part = reinterpret_cast<const f32x4*>(a.part) + (size_t)tile * splits * PTH * 64 + (size_t)(ij * 4 + w) * 64 + lane;
    // Every load goes out before any value is used (a value tested inside
    // the branch of its own load waits for all loads in flight): the row
    // indices, the rows' statistics, c and u, then exactly KPS partials per
    // state; the empty asm statements keep the compiler from sinking a load
    // into the branch of a later use.  Without an index list the index load
    // reads c (a device array here) and is dropped; columns past d read
    // column d - 1 and are not stored.
    const bool has_idx = a.rv.idx != nullptr;
    const int* ip = has_idx ? a.rv.idx : reinterpret_cast<const int*>(a.c);
    int raw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = ip[has_idx ? min(row0 + e, M - 1) : 0];
    float mu_r[3][4], rs_r[3][4];
#pragma unroll
    for (int ss = 0; ss < 3; ++ss)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = min(row0 + e, M - 1);
            mu_r[ss][e] = NORM == NORM_LN ? a.mu[(size_t)ss * M + m] : 0.f;
            rs_r[ss][e] = NORM != NORM_NONE ? a.rstd[(size_t)ss * M + m] : 1.f;
        }
    const bool colok = col < d;
    const int colc = min(col, d - 1);
    const float cl = a.c[colc];
    float ul[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN)
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) ul[ss] = a.u[(size_t)ss * d + colc];
    f32x4 v[3][KPS];
#pragma unroll
    for (int ss = 0; ss < 3; ++ss)
#pragma unroll
        for (int ch = 0; ch < KPS; ++ch) v[ss][ch] = part[(size_t)(ss * KPS + ch) * PTH * 64];
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(raw[e]));
    f32x4 ps[3];
#pragma unroll
    for (int ss = 0; ss < 3; ++ss) {
        ps[ss] = v[ss][0];
#pragma unroll
        for (int ch = 1; ch < KPS; ++ch) ps[ss] += v[ss][ch];
    }
    const float cn = colok ? cl : 0.f;
    float uc[3] = {0.f, 0.f, 0.f};
    if (NORM == NORM_LN && colok)
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) uc[ss] = ul[ss];
    float y[4];
    uint32_t okbits = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = has_idx ? raw[e] : min(row0 + e, M - 1);  // a dense call's row is its own
        const bool ok = r >= 0 && r < a.rv.n_src;
        okbits |= ok ? (1u << e) : 0u;
        float acc = cn;
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) {
            float pv = ps[ss][e];
            if (NORM == NORM_LN) pv -= mu_r[ss][e] * uc[ss];
            acc += NORM == NORM_NONE ? pv : rs_r[ss][e] * pv;
        }
        y[e] = acc;
    }
    store_block_bf16(a.out, M, d, a.rv.ld_out, row0, nt * PBN + wn * 128 + 16 * j, cb, okbits, y[0], y[1], y[2], y[3]);
}

PrefillPlan plan_prefill(int M, int d) {
    PrefillPlan p;
    p.tiles_m = (M + PBM - 1) / PBM;
    p.tiles_n = (d + PBN - 1) / PBN;
    const int tiles = p.tiles_m * p.tiles_n;
    p.splits = 1;
    if (tiles < 192) {
        // split K into chunks inside states: as many chunks per state as keep
        // the grid within one round of the chip (one workgroup per CU).
        // Measured at d=5120, M=128 / 256 and d=8192, M=512: a second round,
        // or a part of one, costs more than the CUs it fills (the partials
        // grow with the chunks); e.g. 4 chunks per state at d=5120, M=256 take
        // 75 us where 8 take 94 us.
        const int KTS = d / PBK;
        const int kps = std::max(1, std::min(std::min(8, KTS), 256 / (3 * tiles)));
        p.splits = 3 * kps;
        p.chunks = p.splits;
        // 43 to 64 tiles: one chunk per state would leave a quarter or more of
        // the CUs idle, two a second round; four equal chunks across the states
        // (two parts per state, each a multiple of 4 sub-tiles) fill up to 256
        if (kps == 1 && 4 * tiles <= 256 && KTS % 16 == 0) {
            p.splits = 6;
            p.chunks = 4;
        }
    }
    if (p.splits > 1) p.part_bytes = (size_t)tiles * p.splits * PTH * 64 * sizeof(f32x4);
    return p;
}

template <bool SPLIT, int NORM>
static hipError_t launch_prefill_t(const PrefillArgs& a, const PrefillPlan& p, hipStream_t st) {
    const int items = p.tiles_m * p.tiles_n * (SPLIT ? p.chunks : 1);
    const int grid = ((items + 7) / 8) * 8;
    if (a.rv.ld[0] == a.rv.ld[1] && a.rv.ld[1] == a.rv.ld[2])
        prefill_kernel<SPLIT, NORM, true><<<grid, PTH, 0, st>>>(a, p.tiles_m, p.tiles_n);
    else
        prefill_kernel<SPLIT, NORM, false><<<grid, PTH, 0, st>>>(a, p.tiles_m, p.tiles_n);
    if (SPLIT) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // 256 fragment groups per tile, 4 per workgroup; the chunks per state
        // (parts per state in the four-chunk mode) are a template argument
        const int rg = p.tiles_m * p.tiles_n * 64;
        switch (a.splits / 3) {
            case 1: prefill_reduce_kernel<NORM, 1><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 2: prefill_reduce_kernel<NORM, 2><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 3: prefill_reduce_kernel<NORM, 3><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 4: prefill_reduce_kernel<NORM, 4><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 5: prefill_reduce_kernel<NORM, 5><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 6: prefill_reduce_kernel<NORM, 6><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 7: prefill_reduce_kernel<NORM, 7><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            case 8: prefill_reduce_kernel<NORM, 8><<<rg, 256, 0, st>>>(a, p.tiles_m, p.tiles_n); break;
            default: return hipErrorInvalidValue;
        }
    }
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
