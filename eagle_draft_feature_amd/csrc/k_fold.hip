// Fold of the norm parameters into the FC (EAGLE 3.1 explainer,
// llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section
// "FC 정규화: EAGLE 3.1의 핵심 수정": the LayerNorm parameters are absorbed
// into the FC layer).  With W'_s = diag(gamma_s) W_s,
//     n(h_s) . W_s = rstd_s * (h_s . W'_s - mu_s * 1^T W'_s) + beta_s^T W_s,
// so the large-M path can run a plain GEMM on the raw hidden states.
//
// One workgroup per 64-column strip of W walks all 3d rows in 64 x 64 tiles:
// coalesced 16-byte loads of W, W' = bf16_rne(gamma * W) (the product of two
// bfloat16 values is exact in float32, so the rounding has one answer),
// a transpose through LDS, and coalesced 16-byte stores of W'^T [d, 3d]
// (k contiguous, the layout the GEMM streams).  Column sums u_s of the stored
// W' and c = bias + sum_s beta_s^T W_s are accumulated in float32 and reduced
// across the workgroup in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace e31 {

__global__ __launch_bounds__(256) void fold_prepare_kernel(int d, int norm, const uint16_t* g0, const uint16_t* g1,
                                                           const uint16_t* g2, const uint16_t* b0,
                                                           const uint16_t* b1, const uint16_t* b2,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ wt, float* __restrict__ u,
                                                           float* __restrict__ c) {
    const int n0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
    const int lr = tid >> 3;  // row of a 32-row half tile
    const int ch = tid & 7;   // 8-column chunk
    const size_t K3 = (size_t)3 * d;
    __shared__ __attribute__((aligned(16))) uint16_t tileT[64][72];  // [column][k], padded rows
    __shared__ float red[32][64];

    float csum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) csum[i] = 0.f;

    for (int s = 0; s < 3; ++s) {
        const uint16_t* gam = norm == NORM_NONE ? nullptr : (s == 0 ? g0 : (s == 1 ? g1 : g2));
        const uint16_t* bet = norm == NORM_LN ? (s == 0 ? b0 : (s == 1 ? b1 : b2)) : nullptr;
        float usum[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) usum[i] = 0.f;
        for (int k0 = s * d; k0 < (s + 1) * d; k0 += 64) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int kr = half * 32 + lr;
                const int k = k0 + kr;
                const uint4 w = *reinterpret_cast<const uint4*>(W + (size_t)k * d + n0 + 8 * ch);
                const float gk = gam ? bf_one(gam[k - s * d]) : 1.f;
                const float bk = bet ? bf_one(bet[k - s * d]) : 0.f;
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float x0 = bf_lo(ww[p]), x1 = bf_hi(ww[p]);
                    const uint32_t pk = pack_bf2(gk * x0, gk * x1);
                    usum[2 * p] += bf_lo(pk);
                    usum[2 * p + 1] += bf_hi(pk);
                    csum[2 * p] += bk * x0;
                    csum[2 * p + 1] += bk * x1;
                    tileT[8 * ch + 2 * p][kr] = (uint16_t)(pk & 0xffffu);
                    tileT[8 * ch + 2 * p + 1][kr] = (uint16_t)(pk >> 16);
                }
            }
            __syncthreads();
            {
                const int n = tid >> 2, kq = tid & 3;
                const uint4* src = reinterpret_cast<const uint4*>(&tileT[n][16 * kq]);
                uint4* dst = reinterpret_cast<uint4*>(wt + (size_t)(n0 + n) * K3 + k0 + 16 * kq);
                dst[0] = src[0];
                dst[1] = src[1];
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) red[lr][8 * ch + i] = usum[i];
        __syncthreads();
        if (tid < 64) {
            float v = 0.f;
            for (int r = 0; r < 32; ++r) v += red[r][tid];
            u[(size_t)s * d + n0 + tid] = v;
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[lr][8 * ch + i] = csum[i];
    __syncthreads();
    if (tid < 64) {
        float v = bias ? bf_one(bias[n0 + tid]) : 0.f;
        for (int r = 0; r < 32; ++r) v += red[r][tid];
        c[n0 + tid] = v;
    }
}

hipError_t launch_fold_prepare(int d, int norm, const uint16_t* const gamma[3], const uint16_t* const beta[3],
                               const uint16_t* W, const uint16_t* bias, uint16_t* wt, float* u, float* c,
                               hipStream_t st) {
    fold_prepare_kernel<<<d / 64, 256, 0, st>>>(d, norm, gamma[0], gamma[1], gamma[2], beta[0], beta[1], beta[2],
                                                  W, bias, wt, u, c);
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
