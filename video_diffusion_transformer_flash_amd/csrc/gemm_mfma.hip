// MFMA projection GEMMs for gfx950: bf16 (v_mfma_f32_32x32x16_bf16) and
// fp8 e4m3 (v_mfma_f32_32x32x64_f8f6f4), fp32 accumulation, fused epilogues.
//
// out[m][n] = sum_k A[m][k] * W[n][k]: A = token activations [M][K], W =
// weights [N][K], both K-contiguous. The MFMA "rows" are weight features and
// its "columns" are tokens, so a lane owns one token and runs of four
// consecutive features: rotary pairs and the SwiGLU gate/up pair are then in
// the lane's own registers (see epilogue.h).
//
// Tiling: 256 threads = 4 waves (2 token halves x 2 feature halves); a tile
// of BT tokens x BF features; a K step of 128 bytes per row (64 bf16 or 128
// fp8); operands staged through LDS in two buffers (one barrier per K step)
// with a 16-byte-chunk XOR swizzle so that 16 lanes reading one chunk column
// of 16 consecutive rows hit 16 distinct bank groups of the 64-bank LDS.
// Workgroup ids are remapped so that neighbouring tiles share an XCD (L2).
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dit {

namespace detail {

constexpr int ROWB = 128;  // bytes of one LDS row per K step
typedef __attribute__((address_space(3))) uint8_t* LDSPTR;

DIT_DEV int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <bool FP8>
struct Elem;
template <>
struct Elem<false> {
    static constexpr int BK = 64;       // elements per K step
    static constexpr int SUB = 4;       // MFMA K sub-steps per K step (16 each)
};
template <>
struct Elem<true> {
    static constexpr int BK = 128;
    static constexpr int SUB = 2;       // 64 each
};

template <int BT, int BF, bool FP8, int MODE, typename TOUT>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W0,
                                                        const uint8_t* __restrict__ W1, int M, int N, int K,
                                                        EpiParams ep) {
#if defined(__HIP_DEVICE_COMPILE__)
    using E = Elem<FP8>;
    constexpr int WT = BT / 2, WF = BF / 2;  // per-wave tile
    constexpr int NBT = WT / 32, NBF = WF / 32;
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int LDS_T = BT * ROWB, LDS_F = BF * ROWB;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // buffer b: features at smem + b * (LDS_F + LDS_T), tokens right after
    auto sF = [&](int b) { return smem + b * (LDS_F + LDS_T); };
    auto sT = [&](int b) { return smem + b * (LDS_F + LDS_T) + LDS_F; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wt = wave & 1, wf = wave >> 1;

    // tile coordinates: XCD-aware, grouped along tokens (GM token tiles share W)
    const int ntt = (M + BT - 1) / BT;
    const int ntf = N / BF;
    const int ntiles = ntt * ntf;
    int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int group = tile / (GM * ntf);
    const int first_t = group * GM;
    const int gsz = min(ntt - first_t, GM);
    const int in_g = tile - group * GM * ntf;
    const int tt = first_t + in_g % gsz;
    const int tf = in_g / gsz;
    const int t0 = tt * BT;
    const int f0 = tf * BF;

    const int rowbytes = K * ESZ;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // Operand tiles go straight from memory to LDS (buffer_load ... lds, 16
    // bytes per lane): one instruction fills 8 rows of 128 bytes, the wave's
    // 64 lanes writing consecutive 16-byte slots; the swizzle is applied on
    // the memory side by fetching, for LDS slot (row, L % 8), the logical
    // chunk (L % 8) ^ swz(row). Instruction i of wave w covers rows
    // 32 i + 8 w .. +7 of the tile.
    const int r8 = 8 * wave + (lane >> 3);                 // row within a 32-row group
    const int cswz = ((lane & 7) ^ swz(r8, 0)) * 16;       // swz(r8 + 32 i) == swz(r8)
    // token rows past M read as zero: the bound check sees only the lane offset
    const int tvalid = min(M - t0, BT);
    const __amdgpu_buffer_rsrc_t rsT =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + (size_t)t0 * rowbytes), 0, tvalid * rowbytes, 0x00020000);
    int voT[BT / 32];
#pragma unroll
    for (int i = 0; i < BT / 32; ++i) voT[i] = (32 * i + r8) * rowbytes + cswz;
    __amdgpu_buffer_rsrc_t rsF0, rsF1;
    if constexpr (MODE == EPI_SWIGLU) {
        rsF0 = __builtin_amdgcn_make_buffer_rsrc((void*)(W0 + (size_t)(f0 / 2) * rowbytes), 0, (BF / 2) * rowbytes,
                                                 0x00020000);
        rsF1 = __builtin_amdgcn_make_buffer_rsrc((void*)(W1 + (size_t)(f0 / 2) * rowbytes), 0, (BF / 2) * rowbytes,
                                                 0x00020000);
    } else {
        rsF0 = __builtin_amdgcn_make_buffer_rsrc((void*)(W0 + (size_t)f0 * rowbytes), 0, BF * rowbytes, 0x00020000);
        rsF1 = rsF0;
    }
    const int voF = r8 * rowbytes + cswz;

    f32x16 acc[NBT][NBF];
#pragma unroll
    for (int a = 0; a < NBT; ++a)
#pragma unroll
        for (int b = 0; b < NBF; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nk = K / E::BK;

    auto issue = [&](int kt, int buf) {
        const int koff = kt * ROWB;
        LDSPTR lt = (LDSPTR)(sT(buf) + wave * 1024);
        LDSPTR lf = (LDSPTR)(sF(buf) + wave * 1024);
#pragma unroll
        for (int i = 0; i < BT / 32; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, lt + i * 4096, 16, voT[i] + koff, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BF / 32; ++i) {
            if constexpr (MODE == EPI_SWIGLU) {
                // 32-row blocks alternate gate / up rows of the same ffn features
                __builtin_amdgcn_raw_ptr_buffer_load_lds((i & 1) ? rsF1 : rsF0, lf + i * 4096, 16, voF + koff,
                                                         (i >> 1) * 32 * rowbytes, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsF0, lf + i * 4096, 16, voF + koff, i * 32 * rowbytes, 0, 0);
            }
        }
    };

    // LDS read offsets of this lane's operand rows
    int rowT[NBT], rowF[NBF];
#pragma unroll
    for (int a = 0; a < NBT; ++a) rowT[a] = wt * WT + a * 32 + lrow;
#pragma unroll
    for (int b = 0; b < NBF; ++b) rowF[b] = wf * WF + b * 32 + lrow;

    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
        const uint8_t* bT = sT(buf);
        const uint8_t* bF = sF(buf);
#pragma unroll
        for (int s = 0; s < E::SUB; ++s) {
            if constexpr (!FP8) {
                bf16x8_v fa[NBF], fb[NBT];
                const int c = 2 * s + lhalf;
#pragma unroll
                for (int b = 0; b < NBF; ++b)
                    fa[b] = *(const bf16x8_v*)(bF + rowF[b] * ROWB + swz(rowF[b], c) * 16);
#pragma unroll
                for (int a = 0; a < NBT; ++a)
                    fb[a] = *(const bf16x8_v*)(bT + rowT[a] * ROWB + swz(rowT[a], c) * 16);
#pragma unroll
                for (int a = 0; a < NBT; ++a)
#pragma unroll
                    for (int b = 0; b < NBF; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b], fb[a], acc[a][b], 0, 0, 0);
            } else {
                i32x8 fa[NBF], fb[NBT];
                const int c = 4 * s + 2 * lhalf;
#pragma unroll
                for (int b = 0; b < NBF; ++b) {
                    uint4 x0 = *(const uint4*)(bF + rowF[b] * ROWB + swz(rowF[b], c) * 16);
                    uint4 x1 = *(const uint4*)(bF + rowF[b] * ROWB + swz(rowF[b], c + 1) * 16);
                    fa[b] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                }
#pragma unroll
                for (int a = 0; a < NBT; ++a) {
                    uint4 x0 = *(const uint4*)(bT + rowT[a] * ROWB + swz(rowT[a], c) * 16);
                    uint4 x1 = *(const uint4*)(bT + rowT[a] * ROWB + swz(rowT[a], c + 1) * 16);
                    fb[a] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                }
#pragma unroll
                for (int a = 0; a < NBT; ++a)
#pragma unroll
                    for (int b = 0; b < NBF; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[b], fb[a], acc[a][b], 0, 0, 0,
                                                                                     0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS fills for the next step have landed
        __syncthreads();                 // ... and everyone's; the current buffer is free
    }

    // ---------------------------------------------------------------- epilogue
    if constexpr (MODE == EPI_SWIGLU) {
        const float sg = epi_scale(ep.amax_a, ep.s_w);
        const float su = epi_scale(ep.amax_a, ep.s_w2);
        float mx = 0.f;
        static_for<NBT>([&](auto a) {
            const int m = t0 + wt * WT + a * 32 + lrow;
            static_for<NBF / 2>([&](auto bp) {
                const int fbase = f0 / 2 + wf * (WF / 2) + bp * 32;
                // fp8: u stays fp32 so that its e4m3 codes come from full-precision values
                using UT = std::conditional_t<FP8, float, TOUT>;
                mx = fmaxf(mx, epi_block_swiglu<UT>(ep, m, fbase, lhalf, acc[a][2 * bp], acc[a][2 * bp + 1], sg, su));
            });
        });
        if (ep.u_amax) {
            mx = wave_max(mx);
            if (lane == 0) atomic_max_nonneg(ep.u_amax, mx);
        }
    } else {
        const float sc = epi_scale(ep.amax_a, ep.s_w);
        static_for<NBT>([&](auto a) {
            const int m = t0 + wt * WT + a * 32 + lrow;
            static_for<NBF>([&](auto b) {
                epi_block<MODE, TOUT>(ep, m, f0 + wf * WF + b * 32, lhalf, acc[a][b], sc);
            });
        });
    }
#endif  // device pass only: the host pass keeps just the launch stub
}

template <int BT, int BF, bool FP8, int MODE>
hipError_t launch_t(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    constexpr int smem = 2 * (BT + BF) * ROWB;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)&gemm_mfma_kernel<BT, BF, FP8, MODE, bf16_t>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int tiles = ((M + BT - 1) / BT) * (N / BF);
    hipLaunchKernelGGL((gemm_mfma_kernel<BT, BF, FP8, MODE, bf16_t>), dim3(tiles), dim3(256), smem, st, (const uint8_t*)A, (const uint8_t*)W0,
                       (const uint8_t*)W1, M, N, K, ep);
    return hipGetLastError();
}

template <bool FP8, int MODE>
hipError_t dispatch(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    // big tiles when there are enough of them to fill 256 CUs several times
    const long t256 = (long)((M + 255) / 256) * (N / 256);
    if (N % 256 == 0 && t256 >= 512) return launch_t<256, 256, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
    if (N % 256 == 0 && (long)((M + 127) / 128) * (N / 256) >= 256)
        return launch_t<128, 256, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
    return launch_t<128, 128, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
}

}  // namespace detail
using namespace detail;

// N: output features (for SWIGLU: 2 * F, gate and up interleaved per tile)
hipError_t gemm_mfma(bool fp8, int mode, const void* A, const void* W0, const void* W1, int M, int N, int K,
                     const EpiParams& ep, hipStream_t st) {
    if (!fp8) {
        switch (mode) {
            case EPI_QKV: return dispatch<false, EPI_QKV>(A, W0, W1, M, N, K, ep, st);
            case EPI_RESID: return dispatch<false, EPI_RESID>(A, W0, W1, M, N, K, ep, st);
            case EPI_SWIGLU: return dispatch<false, EPI_SWIGLU>(A, W0, W1, M, N, K, ep, st);
            default: return dispatch<false, EPI_DOWN>(A, W0, W1, M, N, K, ep, st);
        }
    }
    switch (mode) {
        case EPI_QKV: return dispatch<true, EPI_QKV>(A, W0, W1, M, N, K, ep, st);
        case EPI_RESID: return dispatch<true, EPI_RESID>(A, W0, W1, M, N, K, ep, st);
        case EPI_SWIGLU: return dispatch<true, EPI_SWIGLU>(A, W0, W1, M, N, K, ep, st);
        default: return dispatch<true, EPI_DOWN>(A, W0, W1, M, N, K, ep, st);
    }
}

}  // namespace dit
