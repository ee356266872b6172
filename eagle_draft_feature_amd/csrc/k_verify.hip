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
// sequence's row is cut into C chunks of L tokens (2048, 4096 or 8192: small
// batches take small chunks so that more CUs share a row; at most 256 chunks
// per row), one workgroup each, and each chunk into four quarters, one per
// wave.  Every workgroup finds j itself (N loads); each wave sums its
// quarter's weights exactly (a lane issues all its loads of a 2048-token
// block before using any; per lane into four exponent bands of 64-bit sums,
// one add per token, turned into digits at the end), flags invalid values
// (NaN, above 1) and positive ones, and publishes its quarter record; the
// last workgroup of the sequence to arrive (device-scope counter) loads
// every chunk's record at once (one chunk per thread), scans the chunk totals
// to get the total and each chunk's prefix, forms the threshold, picks the
// first chunk whose prefix exceeds it and, from that chunk's quarter sums, the
// quarter.  Only that quarter is read again: 8 tokens per thread, one load
// round, a workgroup scan of the thread sums, then the chosen thread walks
// its tokens.  A residual that is all zero (only when q_j <= p_j everywhere)
// makes the last arriver sum and search q_j over the whole row itself.
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
// One DPP move of both halves of a 64-bit value (CTRL a DPP control code;
// lanes whose source lies outside their row, or whose row ROWS masks off,
// read 0): cross-lane traffic in registers, no LDS round trip.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, true);
    return ((uint64_t)hi << 32) | lo;
}
// v plus the value of the lane 16 (32) apart: a gfx950 permlane swap of each
// half with itself hands every lane the pair (its own value, its partner's)
__device__ __forceinline__ uint64_t xor16_sum64(uint64_t v) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    return (((uint64_t)hi[0] << 32) | lo[0]) + (((uint64_t)hi[1] << 32) | lo[1]);
}
__device__ __forceinline__ uint64_t xor32_sum64(uint64_t v) {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    return (((uint64_t)hi[0] << 32) | lo[0]) + (((uint64_t)hi[1] << 32) | lo[1]);
}
// the digits summed over the 64 lanes, in every lane (integer adds: any order
// gives the same bits): row rotations by 8, 4, 2, 1, then the two cross-row
// swaps.  The whole wave must be active.
__device__ __forceinline__ Dig dig_wave_sum(Dig a) {
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) {
        uint64_t v = a.d[i];
        v += dpp64<0x128>(v);
        v += dpp64<0x124>(v);
        v += dpp64<0x122>(v);
        v += dpp64<0x121>(v);
        a.d[i] = xor32_sum64(xor16_sum64(v));
    }
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

constexpr int VF_QMAX = 2048;  // tokens in a block of the quarter sum (32 per lane); longest fast-searched quarter
constexpr int VF_REC = 24;     // u64 words of a chunk record: four quarter digit sums, four flag words

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

// Exact sum of the weights [qa, qa + qlen) by one wave (every lane gets it);
// bad / pos OR-ed per lane, not across the wave.  Blocks of 2048 tokens: a
// lane issues all its loads of a block (8 vectors of q and of p, or 32
// scalars each when rows are not 16-byte aligned) before using any.  With VEC
// the range ends on a multiple of 4 tokens.
template <bool VEC>
__device__ void wave_range_sum(const WRow& r, int qa, int qlen, Dig& acc, uint32_t& bad, uint32_t& pos) {
    const int lane = threadIdx.x & 63;
    const int qe = qa + qlen;
    dig_zero(acc);
    for (int i0 = qa; i0 < qe; i0 += VF_QMAX) {
        Band band;
        band_zero(band);
        if (VEC) {
            f32x4 qv[8], pv[8];
            const f32x4* qb = reinterpret_cast<const f32x4*>(r.q + i0) + lane;
            const f32x4* pb = reinterpret_cast<const f32x4*>(r.p + i0) + lane;
            if (i0 + VF_QMAX <= qe) {  // a whole block
#pragma unroll
                for (int k = 0; k < 8; ++k) qv[k] = __builtin_nontemporal_load(qb + 64 * k);
                if (r.mode == 0) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) pv[k] = __builtin_nontemporal_load(pb + 64 * k);
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) pv[k] = qv[k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const bool in = i0 + 4 * lane + 256 * k < qe;
                    qv[k] = in ? __builtin_nontemporal_load(qb + 64 * k) : f32x4{0, 0, 0, 0};
                    pv[k] = in && r.mode == 0 ? __builtin_nontemporal_load(pb + 64 * k) : qv[k];
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float w[4];
                w4(r, qv[k], pv[k], w, bad, pos);
#pragma unroll
                for (int e = 0; e < 4; ++e) band_add_w(band, w[e]);
            }
        } else {
            float qs[32], ps[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                const int i = i0 + lane + 64 * k;
                const bool in = i < qe;
                qs[k] = in ? r.q[i] : 0.0f;
                ps[k] = in && r.mode == 0 ? r.p[i] : qs[k];
            }
#pragma unroll
            for (int k = 0; k < 32; k += 4) {
                float w[4];
                w4(r, f32x4{qs[k], qs[k + 1], qs[k + 2], qs[k + 3]}, f32x4{ps[k], ps[k + 1], ps[k + 2], ps[k + 3]}, w,
                   bad, pos);
#pragma unroll
                for (int e = 0; e < 4; ++e) band_add_w(band, w[e]);
            }
        }
        band_flush(band, acc);  // 32 tokens per lane and block: far below a band's limit
    }
    acc = dig_wave_sum(acc);
}

// inclusive scan of Dig over the 64 lanes: within each 16-lane row by DPP
// row shifts of 1, 2, 4, 8, then row r's total (its lane 15) added to row
// r + 1 (rows 1 and 3), then lane 31's (rows 0-1) to rows 2 and 3.  The
// whole wave must be active.
__device__ __forceinline__ Dig dig_wave_scan(Dig x) {
#pragma unroll
    for (int i = 0; i < VF_ND; ++i) {
        uint64_t v = x.d[i];
        v += dpp64<0x111>(v);
        v += dpp64<0x112>(v);
        v += dpp64<0x114>(v);
        v += dpp64<0x118>(v);
        v += dpp64<0x142, 0xa>(v);
        v += dpp64<0x143, 0xc>(v);
        x.d[i] = v;
    }
    return x;
}

// Smallest t in [a, a + len), len <= VF_QMAX, whose prefix (from a) exceeds
// thr; the range's weights are valid and their sum exceeds thr.  Thread i
// takes tokens [a + 8 i, +8) (one load round for the whole range); a
// workgroup scan of the thread sums finds the thread, which then walks its 8
// tokens.  Every thread gets t.
template <bool VEC>
__device__ int wg_search_quarter(const WRow& r, int a, int len, const Nat& thr, Dig* sh_dig, int* sh_int) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ta = a + 8 * tid, e_end = a + len;
    float w[8];
    if (VEC && ta + 8 <= e_end) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.q + ta + 4 * h));
            const f32x4 pv =
                r.mode == 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r.p + ta + 4 * h)) : qv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = r.mode == 0 ? qv[e] - pv[e] : qv[e];
                w[4 * h + e] = x > 0.0f ? x : 0.0f;  // the row is valid: max(d, 0)
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = ta + e;
            const float x = i < e_end ? (r.mode == 0 ? r.q[i] - r.p[i] : r.q[i]) : 0.0f;
            w[e] = x > 0.0f ? x : 0.0f;
        }
    }
    Dig mine;
    dig_zero(mine);
    {
        Band band;
        band_zero(band);
#pragma unroll
        for (int e = 0; e < 8; ++e) band_add_w(band, w[e]);
        band_flush(band, mine);
    }
    Dig inc = dig_wave_scan(mine);
    if (lane == 63) sh_dig[wave] = inc;
    if (tid == 0) sh_int[4] = VF_THREADS - 1;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < VF_THREADS / 64 - 1; ++v)
        if (v < wave) dig_add(inc, sh_dig[v]);
    const uint64_t hit = __ballot(nat_gt(nat_of(inc), thr));
    if (lane == 0 && hit) atomicMin(&sh_int[4], wave * 64 + (int)__builtin_ctzll(hit));
    __syncthreads();
    if (tid == sh_int[4]) {
        Dig run = inc;  // step back to the exclusive prefix, then add token by token
#pragma unroll
        for (int k = 0; k < VF_ND; ++k) run.d[k] -= mine.d[k];
        int t = ta + 7;
#pragma unroll 1
        for (int e = 0; e < 8; ++e) {
            float we = w[0];  // w[e] without indexing registers dynamically
#pragma unroll
            for (int k = 1; k < 8; ++k) we = e == k ? w[k] : we;
            dig_add_w(run, we);
            if (nat_gt(nat_of(run), thr)) {
                t = ta + e;
                break;
            }
        }
        sh_int[5] = t;
    }
    __syncthreads();
    return sh_int[5];
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
            Dig inc = dig_wave_scan(mine);
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
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)inc.d[k], 63);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(inc.d[k] >> 32), 63);
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
    __shared__ int sh_int[8];
    __shared__ Nat sh_nat[1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    // ---- wave w: exact sum and flags of quarter w of this chunk, published
    const int Q = a.L / 4;
    {
        const int qa = c * a.L + wave * Q;
        const int qlen = max(0, min(Q, V - qa));
        Dig qs;
        uint32_t bad = 0, pos = 0;
        wave_range_sum<VEC>(row, qa, qlen, qs, bad, pos);
        const uint64_t fl = (__any(bad) ? 1u : 0u) | (__any(pos) ? 2u : 0u);
        uint64_t* rec = a.rec + ((size_t)b * a.C + c) * VF_REC;
        if (lane < VF_ND) {
            uint64_t v = 0;  // qs.d[lane] without indexing registers dynamically
#pragma unroll
            for (int k = 0; k < VF_ND; ++k) v = lane == k ? qs.d[k] : v;
            __hip_atomic_store(rec + VF_ND * wave + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == VF_ND) __hip_atomic_store(rec + 4 * VF_ND + wave, fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
    // thread c < C: chunk c's record (the plan keeps C <= 256): its four
    // quarter sums (kept for the quarter pick), their total and the flags;
    // then the inclusive prefix over the chunks in order
    Dig qsum[4];
    uint32_t myfl = 0;
    Dig mine;
    dig_zero(mine);
#pragma unroll
    for (int w = 0; w < 4; ++w) dig_zero(qsum[w]);
    if (tid < a.C) {
        const uint64_t* rc = a.rec + ((size_t)b * a.C + tid) * VF_REC;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int k = 0; k < VF_ND; ++k)
                qsum[w].d[k] = __hip_atomic_load(rc + VF_ND * w + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            myfl |= (uint32_t)__hip_atomic_load(rc + 4 * VF_ND + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) dig_add(mine, qsum[w]);
    }
    Dig inc = dig_wave_scan(mine);
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
        // the chunk that holds the crossing: the first whose inclusive prefix
        // exceeds the threshold; its thread picks the quarter the same way
        const Nat thr = nat_mul_u(nat_of(tot), u);
        const bool over = tid < a.C && nat_gt(nat_of(inc), thr);
        if (tid == 0) sh_int[0] = a.C - 1;
        __syncthreads();
        const uint64_t bal = __ballot(over);
        if (lane == 0 && bal) atomicMin(&sh_int[0], wave * 64 + (int)__builtin_ctzll(bal));
        __syncthreads();
        const int cs = sh_int[0];
        if (tid == cs) {
            Dig run = inc;
#pragma unroll
            for (int k = 0; k < VF_ND; ++k) run.d[k] -= mine.d[k];
            int qsel = 3;
            bool found = false;
            Nat rem = nat_sub(thr, nat_of(run));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (!found) {
                    Dig nx = run;
                    dig_add(nx, qsum[w]);
                    if (nat_gt(nat_of(nx), thr) || w == 3) {
                        found = true;
                        qsel = w;
                        rem = nat_sub(thr, nat_of(run));
                    }
                    run = nx;
                }
            }
            sh_int[1] = qsel;
            sh_nat[0] = rem;
        }
        __syncthreads();
        const int qsel = sh_int[1];
        const Nat rem = sh_nat[0];
        __syncthreads();
        const int sa = cs * a.L + qsel * Q, slen = min(Q, V - sa);
        result = Q <= VF_QMAX ? wg_search_quarter<VEC>(row, sa, slen, rem, sh_dig, sh_int)
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
    // chunks of 2048 to 8192 tokens (a quarter per wave), larger only when a
    // row would need more than one chunk per thread of the last arriver;
    // small batches take small chunks so that more CUs share each row
    long long L = 2048;
    auto chunks = [&](long long l) { return (V + l - 1) / l; };
    while (chunks(L) > VF_THREADS || (L < 8192 && (long long)B * chunks(L) > VERIFY_TARGET_WGS)) L *= 2;
    const long long C = chunks(L);
    p.C = (int)C;
    p.L = (int)L;
    p.rec_bytes = (size_t)B * C * VF_REC * sizeof(uint64_t);
    p.ok = (long long)B * C <= 0x7fffffffLL;
    return p;
}
hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, bool vec, hipStream_t st) {
    if (!p.ok || a.C != p.C || a.L != p.L || a.C > VF_THREADS || a.N < 1 || a.N > VERIFY_MAX_N || a.L % 2048 ||
        (long long)a.C * a.L < a.V)
        return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((long long)a.B * a.C);
    if (vec) verify_kernel<true><<<grid, VF_THREADS, 0, st>>>(a);
    else verify_kernel<false><<<grid, VF_THREADS, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace e31
