// Speculative-decoding verify / accept step (the Leviathan rule of the
// speculative-decoding lesson, factory.pai-world.com/.../15-speculative-decoding-eagle3,
// section "불변식: Leviathan 거부 샘플링"): for each sequence b, the N drafts are
// checked left to right; draft d at position i is kept iff
// u_acc * p_i(d) < q_i(d) (float32 product: the keep probability
// min(1, q/p) without a division); at the first rejection j the next token is
// drawn from the residual max(q_j - p_j, 0) (q_j itself when that is all
// zero), else from q_N.  The draw is the inverse CDF in token order, exact:
// the smallest t with w_0 + ... + w_t > u_res * sum(w).
//
// Exactness.  A float32 w in [0, 1] is m * 2^(e) with a 24-bit m and
// e >= -149, so w * 2^149 = m << sh with sh <= 126: an integer below 2^151.
// It is accumulated as five 32-bit digits held in 64-bit sums (a digit sum
// of at most 2^31 terms below 2^32 cannot overflow), so every sum here is
// exact and independent of the order of addition.  The threshold
// floor(u_res * T) is exact too (u_res = m_u * 2^-s, s >= 24), and for an
// integer prefix S_t, S_t > u_res T <=> S_t > floor(u_res T).
//
// Work split (HBM-bound: the sampled row or row pair is read once).  A
// sequence's row is cut into C chunks of L tokens, one workgroup each
// (B * C workgroups, chunks of 8192 tokens or more, at most 256 per row).
// Every workgroup finds j itself (N loads), sums its chunk's weights exactly
// (all of a thread's loads issued before the first is used; per lane into
// four exponent bands of 64-bit sums, one add per token, turned into digits
// at the end), flags invalid values (NaN, above 1)
// and positive ones, and publishes the record; the last workgroup of the
// sequence to arrive (device-scope counter) loads every record at once (one
// per thread), scans them to get the total and each chunk's prefix, forms the
// threshold, picks the first chunk whose prefix exceeds it, and searches that
// chunk: each wave loads its quarter into registers and sums it, then the
// wave whose quarter holds the crossing scans its registers 256 tokens at a
// time with a lane-level inclusive scan of digit sums.  A
// residual that is all zero (only when q_j <= p_j everywhere) makes the last
// arriver sum and search q_j over the whole row itself.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int VF_THREADS = 256;     // 4 waves
constexpr int VF_ND = 5;            // 32-bit digits of w * 2^149 (bits 0..159)
constexpr int VF_NN = 6;            // normalised digits of a sum (192 bits)

struct Dig {
    uint64_t d[VF_ND];
};
struct Nat {
    uint32_t n[VF_NN + 1];
};

__device__ __forceinline__ void dig_zero(Dig& a) {
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) a.d[i] = 0;
}
__device__ __forceinline__ void dig_add(Dig& a, const Dig& b) {
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) a.d[i] += b.d[i];
}
// a += w * 2^149 for a float32 w in [0, 1] (w > 1 would need more digits:
// callers pass valid weights only)
__device__ __forceinline__ void dig_add_w(Dig& a, float w) {
    const uint32_t b = __float_as_uint(w);
    const uint32_t E = (b >> 23) & 0xffu, f = b & 0x7fffffu;
    const uint32_t m = E ? (f | 0x800000u) : f;
    const uint32_t sh = E ? E - 1 : 0;
    const uint32_t k = sh >> 5;
    const uint64_t v = (uint64_t)m << (sh & 31);
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) a.d[i] += (k == (uint32_t)i ? lo : 0u) + (k + 1 == (uint32_t)i ? hi : 0u);
}
// Per-lane accumulation by exponent band: w * 2^149 = v << (32 k) with
// v = m << (sh % 32) < 2^55 and k = sh / 32 in 0..3, so one 64-bit add into
// band k per token (fewer than 2^9 tokens per band before a flush).
struct Band {
    uint64_t b[4];
};
__device__ __forceinline__ void band_zero(Band& a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a.b[i] = 0;
}
__device__ __forceinline__ void band_add_w(Band& a, float w) {
    const uint32_t x = __float_as_uint(w);
    const uint32_t E = (x >> 23) & 0xffu, f = x & 0x7fffffu;
    const uint32_t m = E ? (f | 0x800000u) : f;
    const uint32_t sh = E ? E - 1 : 0;
    const uint32_t k = sh >> 5;
    const uint64_t v = (uint64_t)m << (sh & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) a.b[i] += k == (uint32_t)i ? v : 0ull;
}
// d += bands (band k is v * 2^(32 k)), bands cleared
__device__ __forceinline__ void band_flush(Band& a, Dig& d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d.d[i] += (uint32_t)a.b[i];
        d.d[i + 1] += a.b[i] >> 32;
        a.b[i] = 0;
    }
}
__device__ __forceinline__ Dig dig_shfl_up(const Dig& a, int delta) {
    Dig r;
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) {
        const uint32_t lo = __shfl_up((uint32_t)a.d[i], delta, 64), hi = __shfl_up((uint32_t)(a.d[i] >> 32), delta, 64);
        r.d[i] = ((uint64_t)hi << 32) | lo;
    }
    return r;
}
__device__ __forceinline__ Dig dig_shfl_xor(const Dig& a, int mask) {
    Dig r;
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) {
        const uint32_t lo = __shfl_xor((uint32_t)a.d[i], mask, 64), hi = __shfl_xor((uint32_t)(a.d[i] >> 32), mask, 64);
        r.d[i] = ((uint64_t)hi << 32) | lo;
    }
    return r;
}
__device__ __forceinline__ Dig dig_wave_sum(Dig a) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dig_add(a, dig_shfl_xor(a, o));
    return a;
}
// carry-propagated digits
__device__ __forceinline__ Nat nat_of(const Dig& a) {
    Nat r;
    uint64_t carry = 0;
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) {
        const uint64_t t = a.d[i] + carry;  // a.d[i] < 2^63, carry < 2^32
        r.n[i] = (uint32_t)t;
        carry = t >> 32;
    }
    r.n[VF_ND] = (uint32_t)carry;
    r.n[VF_ND + 1] = (uint32_t)(carry >> 32);
    return r;
}
__device__ __forceinline__ bool nat_gt(const Nat& a, const Nat& b) {
#pragma unroll
    for (int i = VF_NN; i >= 0; --i)
        if (a.n[i] != b.n[i]) return a.n[i] > b.n[i];
    return false;
}
__device__ __forceinline__ bool nat_zero(const Nat& a) {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i <= VF_NN; ++i) o |= a.n[i];
    return o == 0;
}
__device__ __forceinline__ Nat nat_sub(const Nat& a, const Nat& b) {  // a >= b
    Nat r;
    uint64_t borrow = 0;
#pragma unroll
    for (int i = 0; i <= VF_NN; ++i) {
        const uint64_t t = (uint64_t)a.n[i] - b.n[i] - borrow;
        r.n[i] = (uint32_t)t;
        borrow = (t >> 63) & 1;
    }
    return r;
}
// floor(u * T) for a float32 u in [0, 1)
__device__ __forceinline__ Nat nat_mul_u(const Nat& T, float u) {
    const uint32_t b = __float_as_uint(u);
    const uint32_t E = (b >> 23) & 0xffu, f = b & 0x7fffffu;
    const uint64_t m = E ? (f | 0x800000u) : f;
    const int s = E ? 150 - (int)E : 149;  // u = m * 2^-s, s >= 24
    uint32_t P[VF_NN + 3];
    uint64_t carry = 0;
#pragma unroll
    for (int i = 0; i <= VF_NN; ++i) {
        const uint64_t t = (uint64_t)T.n[i] * m + carry;
        P[i] = (uint32_t)t;
        carry = t >> 32;
    }
    P[VF_NN + 1] = (uint32_t)carry;
    P[VF_NN + 2] = 0;
    const int q = s >> 5, r = s & 31;  // q in 0..4
    Nat out;
#pragma unroll
    for (int qq = 0; qq <= 4; ++qq)
        if (q == qq) {
#pragma unroll
            for (int i = 0; i <= VF_NN; ++i) {
                const uint32_t lo = i + qq <= VF_NN + 2 ? P[i + qq] : 0u;
                const uint32_t hi = i + qq + 1 <= VF_NN + 2 ? P[i + qq + 1] : 0u;
                out.n[i] = r ? (lo >> r) | (hi << (32 - r)) : lo;
            }
        }
    return out;
}

// The weight row of a sequence: residual max(q - p, 0) (mode 0) or q (mode 1).
struct WRow {
    const float* q;
    const float* p;
    int mode;
};
// weight of token i (< V); *bad |= invalid (NaN or outside [0, 1]); *pos |= w > 0
__device__ __forceinline__ float wval(const WRow& r, int i, uint32_t& bad, uint32_t& pos) {
    float w;
    if (r.mode == 0) {
        const float dd = r.q[i] - r.p[i];
        if (dd != dd || dd > 1.0f) bad = 1u;
        w = dd > 0.0f ? dd : 0.0f;
    } else {
        w = r.q[i];
        if (!(w >= 0.0f && w <= 1.0f)) bad = 1u;
    }
    if (bad) w = 0.0f;  // keeps the digit sums in range; the row's result is "no token" anyway
    pos |= w > 0.0f ? 1u : 0u;
    return w;
}

// Exact sum of the weights [a, a + len) by the workgroup (every thread gets
// the result); bad / pos OR-reduced.
template <bool VEC>
__device__ void wg_range_sum(const WRow& r, int a, int len, Dig& sum, uint32_t& bad, uint32_t& pos, Dig* sh_dig,
                             uint32_t* sh_flag) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    Dig acc;
    dig_zero(acc);
    Band band;
    band_zero(band);
    uint32_t b = 0, ps = 0;
    int it = 0;
    for (int i = a + 4 * tid; i < a + len; i += 4 * VF_THREADS, ++it) {
        float w[4];
        if (VEC && i + 4 <= a + len) {
            if (r.mode == 0) {
                const f32x4 qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.q + i));
                const f32x4 pv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.p + i));
                const float qq[4] = {qv[0], qv[1], qv[2], qv[3]}, pp[4] = {pv[0], pv[1], pv[2], pv[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dd = qq[e] - pp[e];
                    const uint32_t bb = (dd != dd || dd > 1.0f) ? 1u : 0u;
                    b |= bb;
                    w[e] = (bb || !(dd > 0.0f)) ? 0.0f : dd;
                }
            } else {
                const f32x4 qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.q + i));
                const float qq[4] = {qv[0], qv[1], qv[2], qv[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t bb = !(qq[e] >= 0.0f && qq[e] <= 1.0f) ? 1u : 0u;
                    b |= bb;
                    w[e] = bb ? 0.0f : qq[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ps |= w[e] > 0.0f ? 1u : 0u;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t bb = 0;
                w[e] = i + e < a + len ? wval(r, i + e, bb, ps) : 0.0f;
                b |= bb;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) band_add_w(band, w[e]);
        if ((it & 63) == 63) band_flush(band, acc);  // at most 256 tokens per band between flushes
    }
    band_flush(band, acc);
    acc = dig_wave_sum(acc);
    b = __any(b) ? 1u : 0u;
    ps = __any(ps) ? 1u : 0u;
    if (lane == 0) {
        sh_dig[wave] = acc;
        sh_flag[wave] = b | (ps << 1);
    }
    __syncthreads();
    dig_zero(sum);
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < VF_THREADS / 64; ++w) {
        dig_add(sum, sh_dig[w]);
        f |= sh_flag[w];
    }
    bad = f & 1u;
    pos = (f >> 1) & 1u;
    __syncthreads();
}

constexpr int VF_L = 8192;                    // tokens per chunk (rows up to 256 chunks)
constexpr int VF_SPT = VF_L / (4 * VF_THREADS);  // float4 steps per thread in a chunk
constexpr int VF_QS = VF_L / 4 / 256;          // 256-token steps in a quarter chunk

// weights of 4 consecutive tokens from loaded q (and p) vectors
__device__ __forceinline__ void w4(const WRow& r, const f32x4& qv, const f32x4& pv, float (&w)[4], uint32_t& bad,
                                   uint32_t& pos) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x;
        uint32_t bb;
        if (r.mode == 0) {
            const float dd = qv[e] - pv[e];
            bb = (dd != dd || dd > 1.0f) ? 1u : 0u;
            x = (bb || !(dd > 0.0f)) ? 0.0f : dd;
        } else {
            bb = !(qv[e] >= 0.0f && qv[e] <= 1.0f) ? 1u : 0u;
            x = bb ? 0.0f : qv[e];
        }
        bad |= bb;
        pos |= x > 0.0f ? 1u : 0u;
        w[e] = x;
    }
}

// Exact sum of a whole chunk [a, a + VF_L) of aligned rows: each thread's
// VF_SPT vector loads (of q and p) are issued before any is used.
__device__ void wg_chunk_sum(const WRow& r, int a, Dig& sum, uint32_t& bad, uint32_t& pos, Dig* sh_dig,
                             uint32_t* sh_flag) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4 qv[VF_SPT], pv[VF_SPT];
#pragma unroll
    for (int k = 0; k < VF_SPT; ++k) {
        const int i = a + 4 * tid + 4 * VF_THREADS * k;
        qv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.q + i));
        pv[k] = r.mode == 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.p + i)) : qv[k];
    }
    Band band;
    band_zero(band);
    uint32_t b = 0, ps = 0;
#pragma unroll
    for (int k = 0; k < VF_SPT; ++k) {
        float w[4];
        w4(r, qv[k], pv[k], w, b, ps);
#pragma unroll
        for (int e = 0; e < 4; ++e) band_add_w(band, w[e]);
    }
    Dig acc;
    dig_zero(acc);
    band_flush(band, acc);
    acc = dig_wave_sum(acc);
    b = __any(b) ? 1u : 0u;
    ps = __any(ps) ? 1u : 0u;
    if (lane == 0) {
        sh_dig[wave] = acc;
        sh_flag[wave] = b | (ps << 1);
    }
    __syncthreads();
    dig_zero(sum);
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < VF_THREADS / 64; ++w) {
        dig_add(sum, sh_dig[w]);
        f |= sh_flag[w];
    }
    bad = f & 1u;
    pos = (f >> 1) & 1u;
    __syncthreads();
}

// inclusive scan of Dig over the 64 lanes
__device__ __forceinline__ Dig dig_wave_scan(Dig x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const Dig up = dig_shfl_up(x, o);
        if (lane >= o) dig_add(x, up);
    }
    return x;
}

// LDS slot of chunk token t: one pad word per 32 tokens, so that a lane
// reading 32 contiguous tokens hits distinct banks
__device__ __forceinline__ int vf_slot(int t) { return t + (t >> 5); }
constexpr int VF_SLOTS = VF_L + VF_L / 32;

// Smallest t in [a, a + len), len <= VF_L, whose prefix (from a) exceeds thr.
// The chunk's weights are loaded coalesced into LDS; lane l of wave w then
// owns tokens [32 (64 w + l), +32) and sums them.  The quarter that holds the
// crossing is found from the wave sums, the lane from one scan of that wave's
// lane sums, the token from one scan of that lane's 32 weights.  Every thread
// gets t.
template <bool VEC>
__device__ int wg_search_chunk(const WRow& r, int a, int len, const Nat& thr, Dig* sh_dig, int* sh_int, Nat* sh_nat,
                               float* sh_w) {
    constexpr int TPL = VF_L / VF_THREADS;  // tokens per lane: 32
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (VEC && len == VF_L) {
        f32x4 qv[VF_SPT], pv[VF_SPT];
#pragma unroll
        for (int k = 0; k < VF_SPT; ++k) {
            const int i = a + 4 * tid + 4 * VF_THREADS * k;
            qv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.q + i));
            pv[k] = r.mode == 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.p + i)) : qv[k];
        }
#pragma unroll
        for (int k = 0; k < VF_SPT; ++k) {
            float* dst = sh_w + vf_slot(4 * tid + 4 * VF_THREADS * k);  // 4 tokens, one 32-run
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = r.mode == 0 ? qv[k][e] - pv[k][e] : qv[k][e];
                dst[e] = x > 0.0f ? x : 0.0f;  // the row is valid: max(d, 0)
            }
        }
    } else {
        for (int t0 = 0; t0 < VF_L; t0 += 8 * VF_THREADS) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + tid + VF_THREADS * e, i = a + t;
                x[e] = t < len ? (r.mode == 0 ? r.q[i] - r.p[i] : r.q[i]) : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sh_w[vf_slot(t0 + tid + VF_THREADS * e)] = x[e] > 0.0f ? x[e] : 0.0f;
        }
    }
    if (tid == 0) sh_int[1] = -1;
    __syncthreads();
    Dig lsum;
    dig_zero(lsum);
    {
        Band band;
        band_zero(band);
        const float* lw = sh_w + (TPL + 1) * tid;  // = vf_slot(TPL * tid)
#pragma unroll
        for (int e = 0; e < TPL; ++e) band_add_w(band, lw[e]);
        band_flush(band, lsum);
    }
    const Dig wsum = dig_wave_sum(lsum);
    if (lane == 0) sh_dig[wave] = wsum;
    __syncthreads();
    if (tid == 0) {
        Dig cum;
        dig_zero(cum);
        int ws = VF_THREADS / 64 - 1;
        Nat rem = thr;
        for (int q = 0; q < VF_THREADS / 64; ++q) {
            Dig next = cum;
            dig_add(next, sh_dig[q]);
            if (nat_gt(nat_of(next), thr)) {
                ws = q;
                rem = nat_sub(thr, nat_of(cum));
                break;
            }
            cum = next;
        }
        sh_int[0] = ws;
        sh_nat[0] = rem;
    }
    __syncthreads();
    const int ws = sh_int[0];
    if (wave == ws) {
        const Nat rem = sh_nat[0];
        // the lane: first whose inclusive prefix exceeds rem
        const Dig inc = dig_wave_scan(lsum);
        const uint64_t hit = __ballot(nat_gt(nat_of(inc), rem));
        const int L = hit ? (int)__builtin_ctzll(hit) : 63;
        Dig ex = inc;
#pragma unroll
        for (int k = 0; k < VF_ND; ++k) ex.d[k] -= lsum.d[k];
        // rem2 = rem - (exclusive prefix of lane L), broadcast from lane L
        Nat r2 = nat_sub(rem, nat_of(ex));
#pragma unroll
        for (int k = 0; k <= VF_NN; ++k) r2.n[k] = __shfl(r2.n[k], L, 64);
        // the token: lanes 0..31 take lane L's tokens
        const int t0 = TPL * (64 * ws + L);
        const float w = lane < TPL ? sh_w[vf_slot(t0 + lane)] : 0.0f;
        Dig mine;
        dig_zero(mine);
        dig_add_w(mine, w);
        const Dig tinc = dig_wave_scan(mine);
        const uint64_t thit = __ballot(lane < TPL && nat_gt(nat_of(tinc), r2));
        if (lane == 0) sh_int[1] = a + t0 + (thit ? (int)__builtin_ctzll(thit) : TPL - 1);
    }
    __syncthreads();
    return sh_int[1];
}

// Smallest t in [a, a + len) whose prefix (from a) exceeds thr; the range's
// weights are valid and their sum exceeds thr.  Every thread gets t.
__device__ int wg_search(const WRow& r, int a, int len, const Nat& thr, Dig* sh_dig, int* sh_int, Nat* sh_nat) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = VF_THREADS / 64;
    // quarters of 256-token multiples
    const int q4 = ((len + NW - 1) / NW + 255) / 256 * 256;
    const int qa = a + wave * q4, qe = min(a + len, qa + q4);
    // each wave's quarter sum
    Dig acc;
    dig_zero(acc);
    Band band;
    band_zero(band);
    uint32_t dummy = 0, dpos = 0;
    int it = 0;
    for (int i = qa + 4 * lane; i < qe; i += 256, ++it) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (i + e < qe) band_add_w(band, wval(r, i + e, dummy, dpos));
        if ((it & 63) == 63) band_flush(band, acc);
    }
    band_flush(band, acc);
    acc = dig_wave_sum(acc);
    if (lane == 0) sh_dig[wave] = acc;
    if (tid == 0) sh_int[1] = -1;
    __syncthreads();
    if (tid == 0) {
        Dig cum;
        dig_zero(cum);
        int ws = NW - 1;
        Nat rem = thr;
        for (int w = 0; w < NW; ++w) {
            Dig next = cum;
            dig_add(next, sh_dig[w]);
            if (nat_gt(nat_of(next), thr)) {
                ws = w;
                rem = nat_sub(thr, nat_of(cum));
                break;
            }
            cum = next;
        }
        sh_int[0] = ws;
        sh_nat[0] = rem;
    }
    __syncthreads();
    const int ws = sh_int[0];
    if (wave == ws) {
        const Nat rem = sh_nat[0];
        const int wa = a + ws * q4, we = min(a + len, wa + q4);
        Dig base;
        dig_zero(base);
        int found = -1;
        for (int i0 = wa; i0 < we && found < 0; i0 += 256) {
            const int i = i0 + 4 * lane;
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = i + e < we ? wval(r, i + e, dummy, dpos) : 0.0f;
            Dig mine;
            dig_zero(mine);
#pragma unroll
            for (int e = 0; e < 4; ++e) dig_add_w(mine, w[e]);
            // inclusive scan over the lanes
            Dig inc = mine;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const Dig up = dig_shfl_up(inc, o);
                if (lane >= o) dig_add(inc, up);
            }
            Dig tot = inc;
            dig_add(tot, base);
            const uint64_t hit = __ballot(nat_gt(nat_of(tot), rem));
            if (hit) {
                const int L = __builtin_ctzll(hit);
                if (lane == L) {
                    Dig run = tot;  // base + inclusive prefix; step back to the exclusive one
#pragma unroll
                    for (int k = 0; k < VF_ND; ++k) run.d[k] -= mine.d[k];
                    int t = i + 3;
                    for (int e = 0; e < 4; ++e) {
                        dig_add_w(run, w[e]);
                        if (nat_gt(nat_of(run), rem)) {
                            t = i + e;
                            break;
                        }
                    }
                    sh_int[1] = t;
                }
                found = 1;
            } else {
                // the wave total is lane 63's inclusive prefix
#pragma unroll
                for (int k = 0; k < VF_ND; ++k) {
                    const uint32_t lo = __shfl((uint32_t)inc.d[k], 63, 64), hi = __shfl((uint32_t)(inc.d[k] >> 32), 63, 64);
                    base.d[k] += ((uint64_t)hi << 32) | lo;
                }
            }
        }
    }
    __syncthreads();
    return sh_int[1];
}

template <bool VEC>
__global__ __launch_bounds__(VF_THREADS) void verify_kernel(VerifyArgs a) {
    __shared__ Dig sh_dig[VF_THREADS / 64];
    __shared__ uint32_t sh_flag[VF_THREADS / 64];
    __shared__ int sh_int[4];
    __shared__ Nat sh_nat[1];
    __shared__ float sh_w[VF_SLOTS];  // the searched chunk's weights (last arriver)
    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.C, c = blockIdx.x - b * a.C;
    const int N = a.N, V = a.V;

    // ---- j: the first rejected position (N if all kept)
    if (tid < 64) {
        bool reject = false;
        if (tid < N) {
            const int t = a.draft[(size_t)b * N + tid];
            const bool inside = t >= 0 && t < V;
            const float pd = inside ? a.p[((size_t)b * N + tid) * V + t] : 0.0f;
            const float qd = inside ? a.q[((size_t)b * (N + 1) + tid) * V + t] : 0.0f;
            const float u = a.u_acc[(size_t)b * N + tid];
            reject = !(__fmul_rn(u, pd) < qd);
        }
        const uint64_t rj = __ballot(reject);
        if (tid == 0) sh_int[2] = rj ? __builtin_ctzll(rj) : N;
    }
    __syncthreads();
    const int j = sh_int[2];
    WRow row;
    row.q = a.q + ((size_t)b * (N + 1) + j) * V;
    row.p = j < N ? a.p + ((size_t)b * N + j) * V : nullptr;
    row.mode = j < N ? 0 : 1;

    // ---- this chunk's exact sum and flags, published
    const int ca = c * a.L, clen = min(a.L, V - ca);
    Dig sum;
    uint32_t bad = 0, pos = 0;
    if (VEC && a.L == VF_L && clen == VF_L) wg_chunk_sum(row, ca, sum, bad, pos, sh_dig, sh_flag);
    else wg_range_sum<VEC>(row, ca, clen, sum, bad, pos, sh_dig, sh_flag);
    uint64_t* rec = a.rec + ((size_t)b * a.C + c) * 8;
    if (tid < VF_ND) {
        uint64_t v = 0;  // sum.d[tid] without indexing registers dynamically
#pragma unroll
        for (int k = 0; k < VF_ND; ++k) v = tid == k ? sum.d[k] : v;
        __hip_atomic_store(rec + tid, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == VF_ND) __hip_atomic_store(rec + VF_ND, (uint64_t)(bad | (pos << 1)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_int[3] = old == a.C - 1;
    }
    __syncthreads();
    if (!sh_int[3]) return;

    // ================= last arriver of sequence b =================
    if (tid == 0) __hip_atomic_store(a.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float u = a.u_res[b];
    int result = -1;
    // every chunk's record, one per thread (the plan keeps C <= 256): totals,
    // flags, and the inclusive prefix over the chunks in order
    const int lane = tid & 63, wave = tid >> 6;
    Dig mine;
    dig_zero(mine);
    uint32_t myfl = 0;
    if (tid < a.C) {
        const uint64_t* rc = a.rec + ((size_t)b * a.C + tid) * 8;
#pragma unroll
        for (int k = 0; k < VF_ND; ++k) mine.d[k] = __hip_atomic_load(rc + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        myfl = (uint32_t)__hip_atomic_load(rc + VF_ND, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    Dig inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const Dig up = dig_shfl_up(inc, o);
        if (lane >= o) dig_add(inc, up);
    }
    const uint32_t wfl = (__any(myfl & 1u) ? 1u : 0u) | (__any(myfl & 2u) ? 2u : 0u);
    if (lane == 63) {
        sh_dig[wave] = inc;
        sh_flag[wave] = wfl;
    }
    __syncthreads();
    Dig tot;
    dig_zero(tot);
    uint32_t fl = 0;
#pragma unroll
    for (int w = 0; w < VF_THREADS / 64; ++w) {
        if (w < wave) dig_add(inc, sh_dig[w]);
        dig_add(tot, sh_dig[w]);
        fl |= sh_flag[w];
    }
    __syncthreads();  // sh_dig / sh_flag are reused below
    const bool u_ok = u >= 0.0f && u < 1.0f;
    if (!u_ok || (fl & 1u)) {
        // invalid weights or u_res: no token
    } else if (fl & 2u) {
        // the chunk that holds the crossing: the first whose inclusive prefix exceeds the threshold
        const Nat thr = nat_mul_u(nat_of(tot), u);
        const bool over = tid < a.C && nat_gt(nat_of(inc), thr);
        if (tid == 0) sh_int[0] = a.C - 1;
        __syncthreads();
        const uint64_t bal = __ballot(over);
        if (lane == 0 && bal) atomicMin(&sh_int[0], wave * 64 + (int)__builtin_ctzll(bal));
        __syncthreads();
        const int cs = sh_int[0];
        if (tid == cs) {
            Dig ex = inc;
#pragma unroll
            for (int k = 0; k < VF_ND; ++k) ex.d[k] -= mine.d[k];
            sh_nat[0] = nat_sub(thr, nat_of(ex));
        }
        __syncthreads();
        const Nat rem = sh_nat[0];
        __syncthreads();
        const int sa = cs * a.L, slen = min(a.L, V - sa);
        result = a.L == VF_L ? wg_search_chunk<VEC>(row, sa, slen, rem, sh_dig, sh_int, sh_nat, sh_w)
                             : wg_search(row, sa, slen, rem, sh_dig, sh_int, sh_nat);
    } else if (row.mode == 0) {
        // the residual is all zero: draw from q_j over the whole row
        WRow qr = row;
        qr.mode = 1;
        Dig qt;
        uint32_t qbad = 0, qpos = 0;
        wg_range_sum<VEC>(qr, 0, V, qt, qbad, qpos, sh_dig, sh_flag);
        if (!qbad && qpos) {
            const Nat thr = nat_mul_u(nat_of(qt), u);
            result = wg_search(qr, 0, V, thr, sh_dig, sh_int, sh_nat);
        }
    }
    if (tid == 0) {
        a.n_acc[b] = j;
        a.next[b] = result;
    }
}

VerifyPlan plan_verify(int B, int N, int V) {
    VerifyPlan p;
    if (B < 1 || N < 1 || N > VERIFY_MAX_N || V < 1) return p;
    // chunks of VF_L tokens (the last arriver searches one chunk), at most
    // one per thread of the last arriver
    long long L = VF_L;
    while ((V + L - 1) / L > VF_THREADS) L *= 2;
    const long long C = (V + L - 1) / L;
    p.C = (int)C;
    p.L = (int)L;
    p.rec_bytes = (size_t)B * C * 8 * sizeof(uint64_t);
    p.ok = (long long)B * C <= 0x7fffffffLL;
    return p;
}

hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, bool vec, hipStream_t st) {
    if (!p.ok || a.C != p.C || a.L != p.L || a.C > VF_THREADS || a.N < 1 || a.N > VERIFY_MAX_N ||
        (long long)a.C * a.L < a.V)
        return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((long long)a.B * a.C);
    if (vec) verify_kernel<true><<<grid, VF_THREADS, 0, st>>>(a);
    else verify_kernel<false><<<grid, VF_THREADS, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace e31
