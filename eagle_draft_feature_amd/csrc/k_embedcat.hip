// Drafter-input concatenation: dst[m] = [embed[tokens[m]] | fused[m]], the
// embedding of the token sampled just before joined to the fused feature
// (EAGLE-3 paper summary, honbul.tistory.com/173, section "EAGLE-3가 바꾼 것 2":
// the fused low / middle / high feature and the previous token's embedding
// form the draft model's input).  Byte work: nothing is rounded.
//
// One wave64 per row, rows at a grid stride.  A lane moves its P 16-byte
// pieces of each half (pieces lane, lane+64, ...; indices clamped into the
// row, so a lane past the end re-reads and re-writes the last piece with
// the same bytes as its owner, and nothing is under a branch).  A token id
// outside [0, vocab) reads row 0 as a stand-in, writes zeros instead and is
// counted once (vector atomic) when a counter is given.  The fused feature
// and the output are touched once (non-temporal hint); embedding rows may
// repeat and stay ordinary loads.  Without a fused feature (F false) only the
// embedding half is written: the fused kernels write the other half
// themselves, through their output row stride.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int EC_WAVES = 8;

template <int P, bool F>
__global__ __launch_bounds__(64 * EC_WAVES) void embed_concat_kernel(const int32_t* __restrict__ tokens, int M, int d,
                                                                     int vocab, const uint16_t* __restrict__ embed,
                                                                     const uint16_t* __restrict__ fused,
                                                                     uint16_t* __restrict__ dst,
                                                                     int32_t* __restrict__ bad_count) {
    const int lane = threadIdx.x & 63;
    const int nvec = d >> 3;
    const int nwaves = gridDim.x * EC_WAVES;
    for (int row = blockIdx.x * EC_WAVES + (threadIdx.x >> 6); row < M; row += nwaves) {
        const int t = tokens[row];
        const bool ok = t >= 0 && t < vocab;
        const u32x4* e = reinterpret_cast<const u32x4*>(embed + (size_t)(ok ? t : 0) * d);
        const u32x4* f = reinterpret_cast<const u32x4*>(fused + (size_t)row * d);
        u32x4* o = reinterpret_cast<u32x4*>(dst + (size_t)row * 2 * d);
        u32x4 ev[P], fv[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int vi = min(lane + 64 * i, nvec - 1);
            ev[i] = e[vi];
            if (F) fv[i] = __builtin_nontemporal_load(&f[vi]);
        }
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int vi = min(lane + 64 * i, nvec - 1);
            __builtin_nontemporal_store(ok ? ev[i] : zero, &o[vi]);
            if (F) __builtin_nontemporal_store(fv[i], &o[nvec + vi]);
        }
        if (!ok && lane == 0 && bad_count != nullptr) atomicAdd(bad_count, 1);
    }
}

hipError_t launch_embed_concat(const int32_t* tokens, int M, int d, int vocab, const uint16_t* embed,
                               const uint16_t* fused, uint16_t* dst, int32_t* bad_count, hipStream_t st) {
    if (d > EMBED_CONCAT_MAX_D || d % 64 != 0 || M <= 0 || vocab <= 0) return hipErrorInvalidValue;
    const int nvec = d / 8;
    const int need = (nvec + 63) / 64;
    const int grid = (int)std::min<int64_t>(((int64_t)M + EC_WAVES - 1) / EC_WAVES, 512);
#define E31_EC(PP)                                                                                                  \
    do {                                                                                                           \
        if (fused != nullptr)                                                                                      \
            embed_concat_kernel<PP, true><<<grid, 64 * EC_WAVES, 0, st>>>(tokens, M, d, vocab, embed, fused, dst,   \
                                                                          bad_count);                              \
        else                                                                                                       \
            embed_concat_kernel<PP, false><<<grid, 64 * EC_WAVES, 0, st>>>(tokens, M, d, vocab, embed, fused, dst,  \
                                                                           bad_count);                             \
    } while (0)
    if (need <= 1) E31_EC(1);
    else if (need <= 2) E31_EC(2);
    else if (need <= 4) E31_EC(4);
    else if (need <= 8) E31_EC(8);
    else if (need <= 12) E31_EC(12);
    else if (need <= 14) E31_EC(14);
    else E31_EC(16);
#undef E31_EC
    return hipGetLastError();
}

}  // namespace e31
