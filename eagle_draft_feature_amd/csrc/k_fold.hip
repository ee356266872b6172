// Fold of the norm parameters into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the LayerNorm parameters are absorbed
// into the FC layer).  With W'_s = diag(gamma_s) W_s,
//     n(h_s) . W_s = rstd_s * (h_s . W'_s - mu_s * 1^T W'_s) + beta_s^T W_s,
// so the GEMMs run on the raw hidden states.
//
// Workgroup (strip, q) of 64 columns: for q = 0, 1, 2 it walks the d rows of
// state q in 64 x 64 blocks: coalesced 16-byte loads of W (prefetched three
// blocks ahead), W' = bf16_rne(gamma * W) (the product of two bfloat16
// values is exact in float32, so the rounding has one answer), a transpose
// through LDS, and 16-byte stores of the 1 KiB MFMA B-fragment tiles of
// W'; it also sums the stored W' of each column into u_q.  Workgroup q = 3
// computes c = bias + sum_s beta_s^T W_s over all 3d rows of the strip (only
// LayerNorm with some beta; otherwise c = bias).  Every sum runs in a fixed
// order: the results are deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

constexpr int FTH = 512;   // threads per workgroup: 64 rows x 8 chunks of 8 columns
constexpr int FPF = 3;     // 64-row blocks in flight per thread

__global__ __launch_bounds__(FTH) void fold_prepare_kernel(int d, int norm, const uint16_t* g0, const uint16_t* g1,
                                                           const uint16_t* g2, const uint16_t* b0,
                                                           const uint16_t* b1, const uint16_t* b2,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ wt, float* __restrict__ u,
                                                           float* __restrict__ c) {
    const int strip = blockIdx.x >> 2, q = blockIdx.x & 3;
    const int n0 = strip * 64;
    const int tid = threadIdx.x;
    const int lr = tid >> 3;  // row inside a 64-row block
    const int ch = tid & 7;   // 8-column chunk
    const int T = 3 * d / 32; // tiles per 16-column block
    __shared__ __attribute__((aligned(16))) uint16_t tileT[64][72];  // [column][k], padded rows
    __shared__ float red[64][65];

    const bool has_beta = norm == NORM_LN && (b0 != nullptr || b1 != nullptr || b2 != nullptr);
    float sum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum[i] = 0.f;

    if (q < 3) {
        const uint16_t* gam = norm == NORM_NONE ? nullptr : (q == 0 ? g0 : (q == 1 ? g1 : g2));
        const int nblk = d / 64;
        const uint16_t* src = W + ((size_t)q * d + lr) * d + n0 + 8 * ch;
        uint4 ring[FPF];
#pragma unroll
        for (int p = 0; p < FPF; ++p)
            ring[p] = *reinterpret_cast<const uint4*>(src + (size_t)min(p, nblk - 1) * 64 * d);
        for (int kb = 0; kb < nblk; kb += FPF) {
#pragma unroll
            for (int p = 0; p < FPF; ++p) {
                const int blk = kb + p;
                if (blk >= nblk) break;
                const uint4 w = ring[p];
                ring[p] = *reinterpret_cast<const uint4*>(src + (size_t)min(blk + FPF, nblk - 1) * 64 * d);
                const int kl = blk * 64 + lr;  // row inside the state
                const float gk = gam ? bf_one(gam[kl]) : 1.f;
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t pk = pack_bf2(gk * bf_lo(ww[i]), gk * bf_hi(ww[i]));
                    sum[2 * i] += bf_lo(pk);
                    sum[2 * i + 1] += bf_hi(pk);
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
                    const uint4 v = *reinterpret_cast<const uint4*>(&tileT[n][kk]);
                    const size_t k32 = ((size_t)q * d + (size_t)blk * 64) / 32;
                    uint4* dst = reinterpret_cast<uint4*>(wt) + ((size_t)(n0 / 16 + j) * T + k32) * 64 + within;
                    *dst = v;
                }
                __syncthreads();
            }
        }
    } else if (has_beta) {
        // c: every row of the strip, in the order of the states
        const int nblk = 3 * d / 64;
        const uint16_t* src = W + (size_t)lr * d + n0 + 8 * ch;
        uint4 ring[FPF];
#pragma unroll
        for (int p = 0; p < FPF; ++p)
            ring[p] = *reinterpret_cast<const uint4*>(src + (size_t)min(p, nblk - 1) * 64 * d);
        for (int kb = 0; kb < nblk; kb += FPF) {
#pragma unroll
            for (int p = 0; p < FPF; ++p) {
                const int blk = kb + p;
                if (blk >= nblk) break;
                const uint4 w = ring[p];
                ring[p] = *reinterpret_cast<const uint4*>(src + (size_t)min(blk + FPF, nblk - 1) * 64 * d);
                const int k = blk * 64 + lr;
                const int s = k / d;
                const uint16_t* bet = s == 0 ? b0 : (s == 1 ? b1 : b2);
                const float bk = bet ? bf_one(bet[k - s * d]) : 0.f;
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sum[2 * i] = fmaf(bk, bf_lo(ww[i]), sum[2 * i]);
                    sum[2 * i + 1] = fmaf(bk, bf_hi(ww[i]), sum[2 * i + 1]);
                }
            }
        }
    }
    // column sums over the 64 row groups, in order
#pragma unroll
    for (int i = 0; i < 8; ++i) red[lr][8 * ch + i] = sum[i];
    __syncthreads();
    if (tid < 64) {
        float v = 0.f;
        for (int r = 0; r < 64; ++r) v += red[r][tid];
        if (q < 3) {
            u[(size_t)q * d + n0 + tid] = v;
        } else {
            c[n0 + tid] = (bias ? bf_one(bias[n0 + tid]) : 0.f) + v;
        }
    }
}

hipError_t launch_fold_prepare(int d, int norm, const uint16_t* const gamma[3], const uint16_t* const beta[3],
                               const uint16_t* W, const uint16_t* bias, uint16_t* wt, float* u, float* c,
                               hipStream_t st) {
    fold_prepare_kernel<<<(d / 64) * 4, FTH, 0, st>>>(d, norm, gamma[0], gamma[1], gamma[2], beta[0], beta[1],
                                                       beta[2], W, bias, wt, u, c);
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
