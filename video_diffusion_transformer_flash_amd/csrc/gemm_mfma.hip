// MFMA projection GEMMs for gfx950: bf16 (v_mfma_f32_32x32x16_bf16) and
// fp8 e4m3 (v_mfma_f32_32x32x64_f8f6f4), fp32 accumulation, fused epilogues.
//
// out[m][n] = sum_k A[m][k] * W[n][k]: A = token activations [M][K], W =
// weights [N][K], both K-contiguous. The MFMA "rows" are weight features and
// its "columns" are tokens, so a lane owns one token and runs of four
// consecutive features: rotary pairs and the SwiGLU gate/up pair are then in
// the lane's own registers (see epilogue.h).
//
// Tiling: WGT x WGF waves (token groups x feature groups); a tile of BT
// tokens x BF features, each wave BT/WGT x BF/WGF; a K step of 128 bytes per
// row (64 bf16 or 128 fp8); operands staged through LDS in two buffers (one
// barrier per K step)
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

template <int BT, int BF, int WGT, int WGF, int NS, bool FP8, int MODE, typename TOUT>
__global__ __launch_bounds__(64 * WGT * WGF) void gemm_mfma_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W0,
                                                        const uint8_t* __restrict__ W1, int M, int N, int K,
                                                        EpiParams ep) {
#if defined(__HIP_DEVICE_COMPILE__)
    using E = Elem<FP8>;
    constexpr int NW = WGT * WGF;            // waves
    constexpr int WT = BT / WGT, WF = BF / WGF;  // per-wave tile
    static_assert(NW >= 2 && WT % 32 == 0 && WF % 64 == 0 && BT % (8 * NW) == 0 && BF % (8 * NW) == 0, "tile");
    constexpr int NBT = WT / 32, NBF = WF / 32;
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int LDS_T = BT * ROWB, LDS_F = BF * ROWB;

    // LDS: one array per pipeline stage (feature tile, then token tile). With
    // separate arrays the compiler can tell that the memory -> LDS loads into
    // one stage do not alias the LDS reads of another, and does not make those
    // reads wait for the loads. Stage addresses are constants.
    constexpr int SB = LDS_F + LDS_T;
    __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? SB : 16];
    auto stage = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return st0;
        else if constexpr (B == 1) return st1;
        else return st2;
    };
    constexpr int NR = FP8 ? 2 : 1;              // 16-byte LDS reads per operand fragment

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep it scalar
    const int wt = wave % WGT, wf = wave / WGT;

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
    // 8 NW i + 8 w .. +7 of the tile.
    constexpr int RPI = 8 * NW;                            // rows per round of instructions
    const int r8 = 8 * wave + (lane >> 3);                 // row within a round
    const int cswz = ((lane & 7) ^ swz(r8, 0)) * 16;       // swz(r8 + RPI i) == swz(r8): RPI % 16 == 0
    // token rows past M read as zero: the bound check sees only the lane offset
    const int tvalid = min(M - t0, BT);
    const __amdgpu_buffer_rsrc_t rsT = make_rsrc(A + (size_t)t0 * rowbytes, tvalid * rowbytes);
    int voT[BT / RPI];
#pragma unroll
    for (int i = 0; i < BT / RPI; ++i) voT[i] = (RPI * i + r8) * rowbytes + cswz;
    __amdgpu_buffer_rsrc_t rsF0, rsF1;
    if constexpr (MODE == EPI_SWIGLU) {
        rsF0 = make_rsrc(W0 + (size_t)(f0 / 2) * rowbytes, (BF / 2) * rowbytes);
        rsF1 = make_rsrc(W1 + (size_t)(f0 / 2) * rowbytes, (BF / 2) * rowbytes);
    } else {
        rsF0 = make_rsrc(W0 + (size_t)f0 * rowbytes, BF * rowbytes);
        rsF1 = rsF0;
    }
    const int voF = (lane >> 3) * rowbytes + cswz;         // lane part; the wave's row goes in soffset

    const int nk = K / E::BK;

    auto issue = [&](int kt, auto bufc) {
        const int koff = kt * ROWB;
        LDSPTR lt = (LDSPTR)(stage(bufc) + LDS_F + wave * 1024);   // 8 rows of 128 B per wave
        LDSPTR lf = (LDSPTR)(stage(bufc) + wave * 1024);
#pragma unroll
        for (int i = 0; i < BT / RPI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, lt + i * RPI * ROWB, 16, voT[i] + koff, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BF / RPI; ++i) {
            const int rowr = RPI * i + 8 * wave;               // first of this wave's 8 rows (uniform)
            if constexpr (MODE == EPI_SWIGLU) {
                // 32-row blocks of the tile alternate gate / up rows of the same
                // ffn features: block b holds gate (b even) or up rows b/2*32 ..
                const int blk = rowr / 32;
                __builtin_amdgcn_raw_ptr_buffer_load_lds((blk & 1) ? rsF1 : rsF0, lf + i * RPI * ROWB, 16, voF + koff,
                                                         ((blk >> 1) * 32 + rowr % 32) * rowbytes, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsF0, lf + i * RPI * ROWB, 16, voF + koff, rowr * rowbytes, 0,
                                                         0);
            }
        }
    };

    // Per-lane LDS byte offsets (buffer 0) of the operand fragments: fragment
    // (s, block) read r is the 16-byte chunk c = NR * (2 s + h) + r of the
    // lane's row. A lane's rows differ by multiples of 32 between blocks, so
    // the swizzle term (row >> 1) & 7 is the same for all of them and a block
    // is a constant 32 * ROWB further: one VGPR per (s, r), blocks and buffers
    // as immediate offsets.
    const int xs = (lrow >> 1) & 7;
    const int rowF0 = (wf * WF + lrow) * ROWB, rowT0 = LDS_F + (wt * WT + lrow) * ROWB;
    uint32_t aC[E::SUB][NR];
#pragma unroll
    for (int s = 0; s < E::SUB; ++s)
#pragma unroll
        for (int r = 0; r < NR; ++r) aC[s][r] = ((NR * (2 * s + lhalf) + r) ^ xs) * 16;

    f32x16 acc[NBT][NBF];
#pragma unroll
    for (int a = 0; a < NBT; ++a)
#pragma unroll
        for (int b = 0; b < NBF; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // two fragment register sets: substep s computes from one while s+1 loads into the other
    uint4 fF[2][NBF][NR], fT[2][NBT][NR];

    auto load_frags = [&](auto setc, auto sc, auto bufc) {
        constexpr int SET = decltype(setc)::value, S = decltype(sc)::value, BUF = decltype(bufc)::value;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint8_t* pF = stage(bufc) + rowF0 + aC[S][r];
            const uint8_t* pT = stage(bufc) + rowT0 + aC[S][r];
#pragma unroll
            for (int b = 0; b < NBF; ++b) fF[SET][b][r] = *(const uint4*)(pF + b * 32 * ROWB);
#pragma unroll
            for (int a = 0; a < NBT; ++a) fT[SET][a][r] = *(const uint4*)(pT + a * 32 * ROWB);
        }
    };
    auto mfmas = [&](auto setc) {
        constexpr int SET = decltype(setc)::value;
#pragma unroll
        for (int a = 0; a < NBT; ++a)
#pragma unroll
            for (int b = 0; b < NBF; ++b) {
                if constexpr (!FP8) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_v, fF[SET][b][0]),
                                                                         __builtin_bit_cast(bf16x8_v, fT[SET][a][0]),
                                                                         acc[a][b], 0, 0, 0);
                } else {
                    const uint4 x0 = fF[SET][b][0], x1 = fF[SET][b][1], y0 = fT[SET][a][0], y1 = fT[SET][a][1];
                    const i32x8 fa = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z,
                                      (int)x1.w};
                    const i32x8 fb = {(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z,
                                      (int)y1.w};
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[a][b], 0, 0, 0, 0, 0, 0);
                }
            }
    };

    // vmcnt immediate (gfx9 encoding, expcnt / lgkmcnt left at their maxima)
    constexpr int LPS = BT / RPI + BF / RPI;                       // memory -> LDS loads per step per wave
    constexpr int VM_KEEP = LPS * (NS - 2);                         // loads of later steps left in flight
    static_assert(VM_KEEP < 64, "vmcnt range");
    constexpr int WAIT_KEEP = (VM_KEEP & 15) | (7 << 4) | (15 << 8) | ((VM_KEEP >> 4) << 14);

    // One K step on LDS stage BUF: the fragments of substep 0 are already in
    // set 0, the loads for the next NS - 2 steps are in flight. Issue the loads
    // of step kt + NS - 1 into the stage freed by the previous step; substeps
    // 0..SUB-2 load the next substep's fragments while their MFMAs run; the
    // last substep's fragments are in registers before the barrier, so after
    // it the next step's first fragments load while the last MFMAs run.
    auto kstep = [&](auto bufc, int kt) {
        constexpr int BUF = decltype(bufc)::value;
        if (kt + NS - 1 < nk) issue(kt + NS - 1, std::integral_constant<int, (BUF + NS - 1) % NS>{});
        static_for<E::SUB - 1>([&](auto s) {
            load_frags(std::integral_constant<int, (s + 1) & 1>{}, std::integral_constant<int, s + 1>{}, bufc);
            mfmas(std::integral_constant<int, s & 1>{});
            __builtin_amdgcn_sched_barrier(0);   // keep later fragment loads out of this substep
        });
        // step kt + 1's LDS fills (this wave's) have landed; then everyone's
        if (kt + NS - 1 < nk) __builtin_amdgcn_s_waitcnt(WAIT_KEEP);
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                 // nobody reads stage BUF any more
        if (kt + 1 < nk) load_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
                                    std::integral_constant<int, (BUF + 1) % NS>{});
        mfmas(std::integral_constant<int, (E::SUB - 1) & 1>{});
        __builtin_amdgcn_sched_barrier(0);
    };

    static_for<NS - 1>([&](auto b) {
        if (b < nk) issue(b, b);
    });
    if (NS - 1 <= nk) __builtin_amdgcn_s_waitcnt(WAIT_KEEP);
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    load_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    for (int kt = 0; kt < nk; kt += NS) {
        static_for<NS>([&](auto b) {
            if (kt + b < nk) kstep(b, kt + b);
        });
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
                __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounded register pressure
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
                __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounded register pressure
            });
        });
    }
#endif  // device pass only: the host pass keeps just the launch stub
}

// Ping-pong variant for the large projections: 256 x 256 tile, 8 waves in two
// groups of four (one wave of each group per SIMD), wave tile 128 tokens x 64
// features. The groups run half a step apart: while one group issues its
// MFMAs for K step k, the other reads all of its fragments of a step from LDS
// (and group A also starts the memory -> LDS loads of step k + 1), so each
// SIMD always has a wave feeding the matrix core. Every phase ends in a
// workgroup barrier; group B takes one extra barrier at the start and group A
// one at the end. Two LDS stages: step k + 1 is loaded while step k is read,
// and its loads have two phases to land.
template <bool FP8, int MODE, typename TOUT>
__global__ __launch_bounds__(512) void gemm_pingpong_kernel(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ W0,
                                                            const uint8_t* __restrict__ W1, int M, int N, int K,
                                                            EpiParams ep) {
#if defined(__HIP_DEVICE_COMPILE__)
    using E = Elem<FP8>;
    constexpr int BT = 256, BF = 256, WT = 128, WF = 64;
    constexpr int NBT = WT / 32, NBF = WF / 32;
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int LDS_T = BT * ROWB, LDS_F = BF * ROWB;
    constexpr int NR = FP8 ? 2 : 1;

    // one LDS array per stage (feature tile, then token tile): see gemm_mfma_kernel
    __shared__ __attribute__((aligned(16))) uint8_t st0[LDS_F + LDS_T];
    __shared__ __attribute__((aligned(16))) uint8_t st1[LDS_F + LDS_T];
    auto stage = [&](auto bc) -> uint8_t* {
        if constexpr (decltype(bc)::value == 0) return st0;
        else return st1;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;                 // 0: group A (loads + compute), 1: group B
    const int wt = wave & 1, wf = (wave >> 1) & 3;

    const int ntt = (M + BT - 1) / BT;
    const int ntf = N / BF;
    const int ntiles = ntt * ntf;
    int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int group = tile / (GM * ntf);
    const int first_t = group * GM;
    const int gsz = min(ntt - first_t, GM);
    const int in_g = tile - group * GM * ntf;
    const int t0 = (first_t + in_g % gsz) * BT;
    const int f0 = (in_g / gsz) * BF;

    const int rowbytes = K * ESZ;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // memory -> LDS, by group A only: wave a (0..3) fills rows 32 i + 8 a .. +7
    // of each tile (i = 0..7), lanes fetching swizzled chunks
    const int a4 = wave & 3;
    const int r8 = 8 * a4 + (lane >> 3);
    const int cswz = ((lane & 7) ^ swz(r8, 0)) * 16;
    const int tvalid = min(M - t0, BT);
    const __amdgpu_buffer_rsrc_t rsT = make_rsrc(A + (size_t)t0 * rowbytes, tvalid * rowbytes);
    int voT[BT / 32];
#pragma unroll
    for (int i = 0; i < BT / 32; ++i) voT[i] = (32 * i + r8) * rowbytes + cswz;
    __amdgpu_buffer_rsrc_t rsF0, rsF1;
    if constexpr (MODE == EPI_SWIGLU) {
        rsF0 = make_rsrc(W0 + (size_t)(f0 / 2) * rowbytes, (BF / 2) * rowbytes);
        rsF1 = make_rsrc(W1 + (size_t)(f0 / 2) * rowbytes, (BF / 2) * rowbytes);
    } else {
        rsF0 = make_rsrc(W0 + (size_t)f0 * rowbytes, BF * rowbytes);
        rsF1 = rsF0;
    }
    const int voF = r8 * rowbytes + cswz;
    const int nk = K / E::BK;

    auto issue = [&](int kt, auto bufc) {
        const int koff = kt * ROWB;
        LDSPTR lt = (LDSPTR)(stage(bufc) + LDS_F + a4 * 1024);
        LDSPTR lf = (LDSPTR)(stage(bufc) + a4 * 1024);
#pragma unroll
        for (int i = 0; i < BT / 32; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, lt + i * 4096, 16, voT[i] + koff, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BF / 32; ++i) {
            if constexpr (MODE == EPI_SWIGLU)
                __builtin_amdgcn_raw_ptr_buffer_load_lds((i & 1) ? rsF1 : rsF0, lf + i * 4096, 16, voF + koff,
                                                         (i >> 1) * 32 * rowbytes, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsF0, lf + i * 4096, 16, voF + koff, i * 32 * rowbytes, 0, 0);
        }
    };

    const int xs = (lrow >> 1) & 7;
    const int rowF0 = (wf * WF + lrow) * ROWB, rowT0 = LDS_F + (wt * WT + lrow) * ROWB;
    uint32_t aC[E::SUB][NR];
#pragma unroll
    for (int s = 0; s < E::SUB; ++s)
#pragma unroll
        for (int r = 0; r < NR; ++r) aC[s][r] = ((NR * (2 * s + lhalf) + r) ^ xs) * 16;

    f32x16 acc[NBT][NBF];
#pragma unroll
    for (int a = 0; a < NBT; ++a)
#pragma unroll
        for (int b = 0; b < NBF; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    uint4 fF[E::SUB][NBF][NR], fT[E::SUB][NBT][NR];   // one whole step of fragments
    auto read_step = [&](auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
#pragma unroll
        for (int s = 0; s < E::SUB; ++s)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint8_t* pF = stage(bufc) + rowF0 + aC[s][r];
                const uint8_t* pT = stage(bufc) + rowT0 + aC[s][r];
#pragma unroll
                for (int b = 0; b < NBF; ++b) fF[s][b][r] = *(const uint4*)(pF + b * 32 * ROWB);
#pragma unroll
                for (int a = 0; a < NBT; ++a) fT[s][a][r] = *(const uint4*)(pT + a * 32 * ROWB);
            }
    };
    auto compute_step = [&]() {
#pragma unroll
        for (int s = 0; s < E::SUB; ++s)
#pragma unroll
            for (int a = 0; a < NBT; ++a)
#pragma unroll
                for (int b = 0; b < NBF; ++b) {
                    if constexpr (!FP8) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_v, fF[s][b][0]), __builtin_bit_cast(bf16x8_v, fT[s][a][0]),
                            acc[a][b], 0, 0, 0);
                    } else {
                        const uint4 x0 = fF[s][b][0], x1 = fF[s][b][1], y0 = fT[s][a][0], y1 = fT[s][a][1];
                        const i32x8 fa = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        const i32x8 fb = {(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                                          (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
                        acc[a][b] =
                            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[a][b], 0, 0, 0, 0, 0, 0);
                    }
                }
    };
    // one step: memory phase (reads of stage BUF; group A also issues step
    // kt + 1), barrier, compute phase, (A: wait for step kt + 1), barrier
    auto step = [&](auto bufc, int kt) {
        constexpr int BUF = decltype(bufc)::value;
        if (grp == 0 && kt + 1 < nk) issue(kt + 1, std::integral_constant<int, BUF ^ 1>{});
        read_step(bufc);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's fragments are in registers
        __syncthreads();
        __builtin_amdgcn_s_setprio(1);
        compute_step();
        __builtin_amdgcn_s_setprio(0);
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0);   // its LDS fills for step kt + 1 have landed
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };

    if (grp == 0) issue(0, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (grp == 1) __syncthreads();          // group B runs one phase behind
    for (int kt = 0; kt < nk; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
    }
    if (grp == 0) __syncthreads();          // match group B's barrier count

    // ---------------------------------------------------------------- epilogue
    if constexpr (MODE == EPI_SWIGLU) {
        const float sg = epi_scale(ep.amax_a, ep.s_w);
        const float su = epi_scale(ep.amax_a, ep.s_w2);
        float mx = 0.f;
        static_for<NBT>([&](auto a) {
            const int m = t0 + wt * WT + a * 32 + lrow;
            static_for<NBF / 2>([&](auto bp) {
                const int fbase = f0 / 2 + wf * (WF / 2) + bp * 32;
                using UT = std::conditional_t<FP8, float, TOUT>;
                mx = fmaxf(mx, epi_block_swiglu<UT>(ep, m, fbase, lhalf, acc[a][2 * bp], acc[a][2 * bp + 1], sg, su));
                __builtin_amdgcn_sched_barrier(0);
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
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    }
#endif
}

template <bool FP8, int MODE>
hipError_t launch_pingpong(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                           hipStream_t st) {
    const int tiles = ((M + 255) / 256) * (N / 256);
    hipLaunchKernelGGL((gemm_pingpong_kernel<FP8, MODE, bf16_t>), dim3(tiles), dim3(512), 0, st,
                       (const uint8_t*)A, (const uint8_t*)W0, (const uint8_t*)W1, M, N, K, ep);
    return hipGetLastError();
}

template <int BT, int BF, int WGT, int WGF, int NS, bool FP8, int MODE>
hipError_t launch_t(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    static_assert(NS * (BT + BF) * ROWB <= 160 * 1024, "LDS");   // NS stages of each operand tile
    const int tiles = ((M + BT - 1) / BT) * (N / BF);
    hipLaunchKernelGGL((gemm_mfma_kernel<BT, BF, WGT, WGF, NS, FP8, MODE, bf16_t>), dim3(tiles), dim3(64 * WGT * WGF), 0,
                       st, (const uint8_t*)A, (const uint8_t*)W0, (const uint8_t*)W1, M, N, K, ep);
    return hipGetLastError();
}

template <bool FP8, int MODE>
hipError_t dispatch(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    // big tiles when there are enough of them to fill 256 CUs several times
    const long t256 = (long)((M + 255) / 256) * (N / 256);
    if (N % 256 == 0 && t256 >= 512) return launch_pingpong<FP8, MODE>(A, W0, W1, M, N, K, ep, st);
    return launch_t<128, 128, 2, 2, 2, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
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
