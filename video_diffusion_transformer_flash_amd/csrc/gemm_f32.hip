// fp32 projection GEMMs (VALU, LDS-tiled) for the fp32 form of the block,
// with the same fused epilogues as the MFMA path (see epilogue.h).
//
// Tile 64 tokens x 64 features, K step 16, 256 threads; thread (ty, tx) owns
// tokens 4ty..4ty+3 and features 4tx..4tx+3, so each epilogue call gets four
// consecutive features of one token. SWIGLU: the tile holds 64 ffn features
// and each thread keeps gate and up accumulators.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dit {

namespace detail {

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W0,
                                                       const float* __restrict__ W1, int M, int N, int K,
                                                       EpiParams ep) {
    constexpr int BT = 64, BF = 64, BK = 16;
    constexpr bool DUAL = MODE == EPI_SWIGLU;
    __shared__ float sA[BK][BT + 4];
    __shared__ float sW[BK][BF + 4];
    __shared__ float sU[DUAL ? BK : 1][BF + 4];

    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int nft = DUAL ? (N / 2) / BF : N / BF;
    const int tt = blockIdx.x / nft, tf = blockIdx.x - (blockIdx.x / nft) * nft;
    const int t0 = tt * BT, f0 = tf * BF;

    float acc[4][4] = {};
    float acu[DUAL ? 4 : 1][4] = {};

    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int am = min(t0 + lr, M - 1);
    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 a = *(const float4*)(A + (size_t)am * K + k0 + lk);
        float4 w = *(const float4*)(W0 + (size_t)(f0 + lr) * K + k0 + lk);
        sA[lk + 0][lr] = a.x; sA[lk + 1][lr] = a.y; sA[lk + 2][lr] = a.z; sA[lk + 3][lr] = a.w;
        sW[lk + 0][lr] = w.x; sW[lk + 1][lr] = w.y; sW[lk + 2][lr] = w.z; sW[lk + 3][lr] = w.w;
        if constexpr (DUAL) {
            float4 u = *(const float4*)(W1 + (size_t)(f0 + lr) * K + k0 + lk);
            sU[lk + 0][lr] = u.x; sU[lk + 1][lr] = u.y; sU[lk + 2][lr] = u.z; sU[lk + 3][lr] = u.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a4[4], w4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a4[i] = sA[kk][ty * 4 + i];
                w4[i] = sW[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], w4[j], acc[i][j]);
            if constexpr (DUAL) {
                float u4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) u4[i] = sU[kk][tx * 4 + i];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acu[i][j] = fmaf(a4[i], u4[j], acu[i][j]);
            }
        }
        __syncthreads();
    }

    const int n0 = f0 + tx * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = t0 + ty * 4 + i;
        float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        if constexpr (MODE == EPI_QKV) epi_qkv<float>(ep, m, n0, v, 1.f);
        else if constexpr (MODE == EPI_RESID) epi_resid<float>(ep, m, n0, v, 1.f);
        else if constexpr (MODE == EPI_DOWN) epi_down<float>(ep, m, n0, v, 1.f);
        else {
            float u[4] = {acu[DUAL ? i : 0][0], acu[DUAL ? i : 0][1], acu[DUAL ? i : 0][2], acu[DUAL ? i : 0][3]};
            epi_swiglu<float>(ep, m, n0, v, u, 1.f, 1.f);
        }
    }
}

}  // namespace detail
using namespace detail;

// N: output features (SWIGLU: 2 * F; each tile reads 64 rows of W0 and of W1)
hipError_t gemm_f32(int mode, const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    const int ntt = (M + 63) / 64;
    const int nft = mode == EPI_SWIGLU ? (N / 2) / 64 : N / 64;
    const dim3 grid(ntt * nft), block(256);
    const float *a = (const float*)A, *w0 = (const float*)W0, *w1 = (const float*)W1;
    switch (mode) {
        case EPI_QKV: hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, grid, block, 0, st, a, w0, w1, M, N, K, ep); break;
        case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, block, 0, st, a, w0, w1, M, N, K, ep); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, block, 0, st, a, w0, w1, M, N, K, ep); break;
        default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_DOWN>, grid, block, 0, st, a, w0, w1, M, N, K, ep); break;
    }
    return hipGetLastError();
}

}  // namespace dit
