// Fold of the norm parameters into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the LayerNorm parameters are absorbed
// into the FC layer).  With W'_s = diag(gamma_s) W_s,
//     n(h_s) . W_s = rstd_s * (h_s . W'_s - mu_s * 1^T W'_s) + beta_s^T W_s,
// so the GEMMs run on the raw hidden states.
//
// Workgroup (strip, s) of 64 columns walks the d rows of state s in 64 x 64
// blocks: coalesced 16-byte loads of W (eight blocks in flight per thread),
// W' = bf16_rne(gamma * W) (the product of two bfloat16 values is exact in
// float32, so the rounding has one answer), a transpose through LDS, and
// 16-byte stores of the 1 KiB MFMA B-fragment tiles of W'.  In the same pass
// it sums each column of the stored W' into u_s and, for LayerNorm with a
// beta, of beta_s-weighted W into a partial of c.  The last of the strip's
// three workgroups to finish (a device-scope counter in the workspace, left
// at zero) forms c = bias + the three partials, in state order.  Every sum
// runs in a fixed order: the results are deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int FTH = 512;   // threads per workgroup: 64 rows x 8 chunks of 8 columns
constexpr int FPF = 8;     // 64-row blocks in flight per thread

__global__ __launch_bounds__(FTH) void fold_prepare_kernel(int d, int norm, const uint16_t* g0, const uint16_t* g1,
                                                           const uint16_t* g2, const uint16_t* b0,
                                                           const uint16_t* b1, const uint16_t* b2,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ wt, float* __restrict__ u,
                                                           float* __restrict__ c, int* __restrict__ counters,
                                                           float* __restrict__ cpart) {
    const int strip = blockIdx.x / 3, q = blockIdx.x - 3 * strip;
    const int n0 = strip * 64;
    const int tid = threadIdx.x;
    const int lr = tid >> 3;  // row inside a 64-row block
    const int ch = tid & 7;   // 8-column chunk
    const int T = 3 * d / 32; // tiles per 16-column block
    __shared__ __attribute__((aligned(16))) uint16_t tileT[64][72];  // [column][k], padded rows
    __shared__ float red[64][65];
    __shared__ int sh_last;

    const bool has_beta = norm == NORM_LN && (b0 != nullptr || b1 != nullptr || b2 != nullptr);
    const uint16_t* gam = norm == NORM_NONE ? nullptr : (q == 0 ? g0 : (q == 1 ? g1 : g2));
    const uint16_t* bet = has_beta ? (q == 0 ? b0 : (q == 1 ? b1 : b2)) : nullptr;
    float usum[8], csum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) usum[i] = csum[i] = 0.f;

    const int nblk = d / 64;
    const uint16_t* src = W + ((size_t)q * d + lr) * d + n0 + 8 * ch;
    // W rows and their gamma / beta values, FPF blocks ahead
    u32x4 ring[FPF];
    uint16_t gring[FPF], bring[FPF];
    auto fetch = [&](int p, int blk) __attribute__((always_inline)) {
        const int bb = min(blk, nblk - 1);
        ring[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)bb * 64 * d));
        gring[p] = gam ? gam[bb * 64 + lr] : (uint16_t)0x3F80;  // 1.0
        bring[p] = bet ? bet[bb * 64 + lr] : (uint16_t)0;
    };
#pragma unroll
    for (int p = 0; p < FPF; ++p) fetch(p, p);
    for (int kb = 0; kb < nblk; kb += FPF) {
#pragma unroll
        for (int p = 0; p < FPF; ++p) {
            const int blk = kb + p;
            if (blk >= nblk) break;
            const u32x4 w = ring[p];
            const float gk = bf_one(gring[p]), bk = bf_one(bring[p]);
            fetch(p, blk + FPF);
            const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t pk = pack_bf2(gk * bf_lo(ww[i]), gk * bf_hi(ww[i]));
                usum[2 * i] += bf_lo(pk);
                usum[2 * i + 1] += bf_hi(pk);
                csum[2 * i] = fmaf(bk, bf_lo(ww[i]), csum[2 * i]);
                csum[2 * i + 1] = fmaf(bk, bf_hi(ww[i]), csum[2 * i + 1]);
                tileT[8 * ch + 2 * i][lr] = (uint16_t)(pk & 0xffffu);
                tileT[8 * ch + 2 * i + 1][lr] = (uint16_t)(pk >> 16);
            }
            __syncthreads();
            // 8 KiB of tiles: 4 column blocks x 2 k-steps, each column
            // block's two tiles contiguous (2 KiB)
            {
                const int j = tid >> 7, within = tid & 127;
                const int kstep = within >> 6, l = within & 63;
                const int n = 16 * j + (l & 15);
                const int kk = 32 * kstep + 8 * (l >> 4);
                const u32x4 v = *reinterpret_cast<const u32x4*>(&tileT[n][kk]);
                const size_t k32 = ((size_t)q * d + (size_t)blk * 64) / 32;
                u32x4* dst = reinterpret_cast<u32x4*>(wt) + ((size_t)(n0 / 16 + j) * T + k32) * 64 + within;
                __builtin_nontemporal_store(v, dst);
            }
            __syncthreads();
        }
    }
    // column sums over the 64 row groups, in order: u_s, then this state's part of c
#pragma unroll
    for (int i = 0; i < 8; ++i) red[lr][8 * ch + i] = usum[i];
    __syncthreads();
    if (tid < 64) {
        float v = 0.f;
        for (int r = 0; r < 64; ++r) v += red[r][tid];
        u[(size_t)q * d + n0 + tid] = v;
    }
    __syncthreads();
    if (has_beta) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[lr][8 * ch + i] = csum[i];
        __syncthreads();
        if (tid < 64) {
            float v = 0.f;
            for (int r = 0; r < 64; ++r) v += red[r][tid];
            store_coherent(cpart + (size_t)q * d + n0 + tid, v);
        }
    }
    // the strip's last workgroup forms c (its stores completed before the count)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(counters + strip, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = old == 2;
    }
    __syncthreads();
    if (!sh_last) return;
    if (tid < 64) {
        const int n = n0 + tid;
        float v = bias ? bf_one(bias[n]) : 0.f;
        if (has_beta) {
            float part = load_coherent(cpart + n);
            part += load_coherent(cpart + (size_t)d + n);
            part += load_coherent(cpart + (size_t)2 * d + n);
            v += part;
        }
        c[n] = v;
    }
    if (tid == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_fold_prepare(int d, int norm, const uint16_t* const gamma[3], const uint16_t* const beta[3],
                               const uint16_t* W, const uint16_t* bias, uint16_t* wt, float* u, float* c,
                               int* counters, float* cpart, hipStream_t st) {
    if (d % 64 != 0 || counters == nullptr || cpart == nullptr) return hipErrorInvalidValue;
    fold_prepare_kernel<<<(d / 64) * 3, FTH, 0, st>>>(d, norm, gamma[0], gamma[1], gamma[2], beta[0], beta[1],
                                                       beta[2], W, bias, wt, u, c, counters, cpart);
    return hipGetLastError();
}

// Fills a buffer with zeros (used where hipMemsetAsync must be avoided, e.g.
// work a caller may capture into a graph).
__global__ void zero_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<uint4*>(p), n16);
    return hipGetLastError();
}

}  // namespace e31
