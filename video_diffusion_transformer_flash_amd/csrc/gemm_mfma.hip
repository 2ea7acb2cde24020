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
// tokens x BF features, each wave BT/WGT x BF/WGF; a K step of RB bytes per
// row (RB = 128: 64 bf16 / 128 fp8; RB = 64: half that). Operands go from
// memory straight to LDS (buffer_load ... lds) through NS token stages and
// NSF weight stages (the weight rows, which miss the XCD's L2 more often, may
// get a third stage), one LDS array per operand and stage, one barrier per K
// step, with a 16-byte-chunk XOR swizzle so that 16 lanes reading one chunk
// column of 16 consecutive rows hit 16 distinct bank groups of the 64-bank
// LDS. Fragment reads of the next MFMA substep are issued under the current
// substep's MFMAs, and the 256 x 256 kernels spread a K step's fills over its
// substeps, one after each MFMA (or issue them a step early, right after the
// barrier), instead of a burst that stalls the wave's MFMA issue. Workgroup
// ids are remapped so that neighbouring tiles share an XCD (L2).
//
// K-split tail: when the tiles fill the compute units a whole number of
// times plus a small remainder, the remainder tiles are cut along K into
// `splits` slices that run as separate workgroups beside the whole tiles; each
// writes its fp32 slice sum to a partial buffer, and a second kernel adds the
// slices in a fixed order and runs the epilogue. The last round then takes a
// fraction of a tile's time instead of a whole one.
#include <atomic>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dit {

namespace detail {

typedef __attribute__((address_space(3))) uint8_t* LDSPTR;


// Row r of a tile with RB-byte rows: a 256-byte bank window holds G = 256 / RB
// rows, so 16 consecutive rows at one logical chunk must spread over the
// CPR = RB / 16 chunk slots of each of the G row residues: physical chunk =
// chunk ^ ((row / G) mod CPR).
template <int RB>
DIT_DEV int swz(int row, int chunk) {
    constexpr int G = 256 / RB, CPR = RB / 16;
    return chunk ^ ((row / G) & (CPR - 1));
}

// Token tiles per weight-tile group (tile_origin). With 32 workgroups in
// flight per XCD, 16 token tiles per weight tile make the token rows the
// operand that misses the XCD's L2 (each token K slice fetched for every pair
// of weight tiles); the bf16 projections, held by the power limit, are
// fastest so (smaller groups were slower uncompressed). The fp8 projections
// run at a higher clock and wait on their fills; with 4 token tiles per weight
// tile the misses move towards the weight rows, which have the deeper
// pipeline (same box: fp8 stack 540.7 -> 533.3 ms; 1, 2 and 8: 548.5, 537.3,
// 534.8).
constexpr int tile_group(bool fp8) { return fp8 ? 4 : 16; }

// First token and first output feature of tile `tile`: GM consecutive token
// tiles share one weight tile, so neighbouring tiles on an XCD reuse it in L2.
template <int BT, int BF, int GM>
DIT_DEV void tile_origin(int tile, int M, int N, int& t0, int& f0) {
    const int ntt = (M + BT - 1) / BT;
    const int ntf = N / BF;
    const int group = tile / (GM * ntf);
    const int first_t = group * GM;
    const int gsz = min(ntt - first_t, GM);
    const int in_g = tile - group * GM * ntf;
    t0 = (first_t + in_g % gsz) * BT;
    f0 = (in_g / gsz) * BF;
}

template <int BT, int BF, int WGT, int WGF, int NS, int NSF, int RB, int PF, int OCC, int SCHED, bool FP8, int MODE,
          typename TOUT>
__global__ __launch_bounds__(64 * WGT * WGF, OCC) void gemm_mfma_kernel(const uint8_t* __restrict__ A,
                                                                   const uint8_t* __restrict__ W0,
                                                                   const uint8_t* __restrict__ W1, int M, int N, int K,
                                                                   int nfull, int splits, EpiParams ep) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NW = WGT * WGF;                 // waves
    constexpr int WT = BT / WGT, WF = BF / WGF;   // per-wave tile
    constexpr int NBT = WT / 32, NBF = WF / 32;
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int BK = RB / ESZ;                  // elements per K step
    constexpr int KSUB = FP8 ? 64 : 16;           // K per MFMA
    constexpr int SUB = BK / KSUB;                // MFMA substeps per K step
    constexpr int NR = FP8 ? 2 : 1;               // 16-byte LDS reads per operand fragment
    constexpr int CPR = RB / 16;                  // 16-byte chunks per row
    constexpr int RPW = 1024 / RB;                // rows filled by one wave instruction (64 lanes x 16 B)
    constexpr int RPI = RPW * NW;                 // rows per round of instructions
    constexpr int LDS_T = BT * RB, LDS_F = BF * RB;
    static_assert(WT % 32 == 0 && WF % 64 == 0 && BT % RPI == 0 && BF % RPI == 0 && RPI % 16 == 0, "tile");
    static_assert(SUB >= 1 && NS >= 2 && NS <= 4 && NSF <= 4, "pipeline");

    // LDS: one array per operand and pipeline stage (NS token stages, NSF
    // weight stages). With separate arrays the compiler can tell that the
    // memory -> LDS loads into one stage do not alias the LDS reads of
    // another, and does not make those reads wait for the loads; every stage
    // address is a constant.
    __shared__ __attribute__((aligned(16))) uint8_t sT0[LDS_T];
    __shared__ __attribute__((aligned(16))) uint8_t sT1[LDS_T];
    __shared__ __attribute__((aligned(16))) uint8_t sT2[NS > 2 ? LDS_T : 16];
    __shared__ __attribute__((aligned(16))) uint8_t sT3[NS > 3 ? LDS_T : 16];
    __shared__ __attribute__((aligned(16))) uint8_t sF0[LDS_F];
    __shared__ __attribute__((aligned(16))) uint8_t sF1[LDS_F];
    __shared__ __attribute__((aligned(16))) uint8_t sF2[NSF > 2 ? LDS_F : 16];
    __shared__ __attribute__((aligned(16))) uint8_t sF3[NSF > 3 ? LDS_F : 16];
    auto stT = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return sT0;
        else if constexpr (B == 1) return sT1;
        else if constexpr (B == 2) return sT2;
        else return sT3;
    };
    auto stF = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return sF0;
        else if constexpr (B == 1) return sF1;
        else if constexpr (B == 2) return sF2;
        else return sF3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep it scalar
    const int wt = wave % WGT, wf = wave / WGT;

    // Tile coordinates, XCD-aware. Workgroups [0, nfull) take whole tiles;
    // the rest are (tail tile, K slice) units, unit u = slice * ntail + tile,
    // writing their sums to partial slot tile * splits + slice.
    const int ntiles = ((M + BT - 1) / BT) * (N / BF);
    int tile, nk = K / BK, kb = 0;
    float* pslot = nullptr;
    if ((int)blockIdx.x < nfull) {
        tile = xcd_remap(blockIdx.x, nfull);
    } else {
        const int ntail = ntiles - nfull;
        const int u = xcd_remap(blockIdx.x - nfull, ntail * splits);
        const int r = u % ntail, slice = u / ntail;
        tile = nfull + r;
        nk /= splits;
        kb = slice * nk;
        pslot = ep.part + (size_t)(r * splits + slice) * BT * BF;
    }
    int t0, f0;
    tile_origin<BT, BF, tile_group(FP8)>(tile, M, N, t0, f0);

    const int rowbytes = K * ESZ;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // Memory -> LDS: one instruction fills RPW rows of RB bytes, the wave's 64
    // lanes writing consecutive 16-byte slots; the swizzle is applied on the
    // memory side by fetching, for LDS slot (row, L % CPR), the logical chunk
    // (L % CPR) ^ swz-term(row). Instruction i of wave w covers rows
    // RPI i + RPW w .. +RPW-1 of the tile (the swizzle term repeats every 16
    // rows, so it is the same for every i).
    const int rw = RPW * wave + lane / CPR;
    const int cswz = swz<RB>(rw, lane % CPR) * 16;
    // Token rows past M read as zero through the descriptor's bound. The
    // per-step K offset goes in the scalar soffset, so the lane offsets are
    // loop-invariant registers that no later instruction overwrites (a fresh
    // address register per load made the compiler wait for the load before
    // reusing it, which drained the deeper stages).
    // (a K slice starts kb steps into every row: the bases move by kb RB bytes)
    const int tvalid = min(M - t0, BT);
    const __amdgpu_buffer_rsrc_t rsT = make_rsrc(A + (size_t)t0 * rowbytes + kb * RB, tvalid * rowbytes);
    int voT[BT / RPI];
#pragma unroll
    for (int i = 0; i < BT / RPI; ++i) voT[i] = (RPI * i + rw) * rowbytes + cswz;
    __amdgpu_buffer_rsrc_t rsF0, rsF1;
    if constexpr (MODE == EPI_SWIGLU) {
        rsF0 = make_rsrc(W0 + (size_t)(f0 / 2) * rowbytes + kb * RB, (BF / 2) * rowbytes);
        rsF1 = make_rsrc(W1 + (size_t)(f0 / 2) * rowbytes + kb * RB, (BF / 2) * rowbytes);
    } else {
        rsF0 = make_rsrc(W0 + (size_t)f0 * rowbytes + kb * RB, BF * rowbytes);
        rsF1 = rsF0;
    }
    const int voF = (lane / CPR) * rowbytes + cswz;   // lane part; the wave's row goes in soffset

    // The LDS base of a fill goes through an empty register move, so the fill
    // carries no array provenance: the compiler then counts it with the LDS
    // writes it cannot place and does not make reads of the named stage arrays
    // wait for it (its pairing of reads with earlier fills made some steps wait
    // for fills of later stages). Every read of a stage follows this wave's
    // explicit vmcnt wait for its fills and the barrier after it; at the IR
    // level the fill still writes unknown LDS, so no LDS access moves across it.
    auto untracked = [](uint8_t* p) {
        uint32_t a = (uint32_t)(uintptr_t)(LDSPTR)p;
        asm volatile("" : "+s"(a));
        return (LDSPTR)(uintptr_t)a;
    };
    auto issueT_at = [&](int kt, LDSPTR lt) {
        const int koff = kt * RB;
#pragma unroll
        for (int i = 0; i < BT / RPI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, lt + i * RPI * RB, 16, voT[i], koff, 0, 0);
    };
    auto issueF_one = [&](int kt, LDSPTR lf, auto ic) {
        constexpr int i = decltype(ic)::value;
        const int koff = kt * RB;
        const int rowr = RPI * i + RPW * wave;         // first of this wave's rows (uniform)
        if constexpr (MODE == EPI_SWIGLU) {
            // 32-row blocks of the tile alternate gate / up rows of the same
            // ffn features: block b holds gate (b even) or up rows b/2*32 ..
            const int blk = rowr / 32;
            __builtin_amdgcn_raw_ptr_buffer_load_lds((blk & 1) ? rsF1 : rsF0, lf + i * RPI * RB, 16, voF,
                                                     ((blk >> 1) * 32 + rowr % 32) * rowbytes + koff, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsF0, lf + i * RPI * RB, 16, voF, rowr * rowbytes + koff, 0, 0);
        }
    };
    auto issueF_at = [&](int kt, LDSPTR lf) { static_for<BF / RPI>([&](auto i) { issueF_one(kt, lf, i); }); };
    auto issueT = [&](int kt, auto bufc) { issueT_at(kt, untracked(stT(bufc) + wave * 1024)); };
    auto issueF = [&](int kt, auto bufc) { issueF_at(kt, untracked(stF(bufc) + wave * 1024)); };

    // Register prefetch (PF = 2): the same fetches into registers, register
    // set j % 2 holding step j; they are written to the free LDS stage at the
    // end of the step before their use, so a fetch has two steps to land
    // (with the direct loads above and two stages it has one).
    constexpr int NPT = BT / RPI, NPF = BF / RPI;
    uint4 pre[PF == 2 ? 2 : 1][NPT + NPF];
    auto gload = [&](int kt, auto setc) {
        constexpr int SET = decltype(setc)::value;
        const int koff = kt * RB;
#pragma unroll
        for (int i = 0; i < NPT; ++i)
            pre[SET][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsT, voT[i], koff, 0));
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            const int rowr = RPI * i + RPW * wave;
            if constexpr (MODE == EPI_SWIGLU) {
                const int blk = rowr / 32;
                pre[SET][NPT + i] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128((blk & 1) ? rsF1 : rsF0, voF,
                                                                 ((blk >> 1) * 32 + rowr % 32) * rowbytes + koff, 0));
            } else {
                pre[SET][NPT + i] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rsF0, voF, rowr * rowbytes + koff, 0));
            }
        }
    };
    auto lwrite = [&](auto setc, auto bufc) {
        constexpr int SET = decltype(setc)::value;
        uint8_t* lt = stT(bufc) + wave * 1024 + lane * 16;
        uint8_t* lf = stF(bufc) + wave * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < NPT; ++i) *(uint4*)(lt + i * RPI * RB) = pre[SET][i];
#pragma unroll
        for (int i = 0; i < NPF; ++i) *(uint4*)(lf + i * RPI * RB) = pre[SET][NPT + i];
    };
    // vmcnt immediates (gfx9 encoding, expcnt / lgkmcnt left at their maxima)
    auto vmwait = [](auto nc) {
        constexpr int n = decltype(nc)::value;
        static_assert(n < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    };

    // Per-lane LDS byte offsets of the operand fragments: fragment (s, block)
    // read r is the 16-byte chunk c = NR * (2 s + h) + r of the lane's row.
    // A lane's rows differ by multiples of 32 between blocks, so its swizzle
    // term is the same for all of them and a block is a constant 32 * RB
    // further: one VGPR per (s, r), blocks and stages as immediate offsets.
    const int rowF0 = (wf * WF + lrow) * RB, rowT0 = (wt * WT + lrow) * RB;
    uint32_t aC[SUB][NR];
#pragma unroll
    for (int s = 0; s < SUB; ++s)
#pragma unroll
        for (int r = 0; r < NR; ++r) aC[s][r] = swz<RB>(lrow, NR * (2 * s + lhalf) + r) * 16;

    f32x16 acc[NBT][NBF];
#pragma unroll
    for (int a = 0; a < NBT; ++a)
#pragma unroll
        for (int b = 0; b < NBF; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // two fragment register sets: substep s computes from one while s+1 loads into the other
    uint4 fF[2][NBF][NR], fT[2][NBT][NR];

    auto load_frags = [&](auto setc, auto sc, auto tbc, auto fbc) {
        constexpr int SET = decltype(setc)::value, S = decltype(sc)::value;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint8_t* pF = stF(fbc) + rowF0 + aC[S][r];
            const uint8_t* pT = stT(tbc) + rowT0 + aC[S][r];
#pragma unroll
            for (int b = 0; b < NBF; ++b) fF[SET][b][r] = *(const uint4*)(pF + b * 32 * RB);
#pragma unroll
            for (int a = 0; a < NBT; ++a) fT[SET][a][r] = *(const uint4*)(pT + a * 32 * RB);
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

    // One fragment read (index: weight blocks, then token blocks, per 16-byte
    // read r) and one MFMA, for the explicitly ordered substeps of SCHED 3.
    auto read_one = [&](auto setc, auto sc, auto tbc, auto fbc, auto ic) {
        constexpr int SET = decltype(setc)::value, S = decltype(sc)::value, I = decltype(ic)::value;
        constexpr int r = I / (NBF + NBT), j = I % (NBF + NBT);
        if constexpr (j < NBF) fF[SET][j][r] = *(const uint4*)(stF(fbc) + rowF0 + aC[S][r] + j * 32 * RB);
        else fT[SET][j - NBF][r] = *(const uint4*)(stT(tbc) + rowT0 + aC[S][r] + (j - NBF) * 32 * RB);
    };
    auto mfma_one = [&](auto setc, auto ic) {
        constexpr int SET = decltype(setc)::value, a = decltype(ic)::value / NBF, b = decltype(ic)::value % NBF;
        if constexpr (!FP8) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_v, fF[SET][b][0]),
                                                                 __builtin_bit_cast(bf16x8_v, fT[SET][a][0]), acc[a][b],
                                                                 0, 0, 0);
        } else {
            const uint4 x0 = fF[SET][b][0], x1 = fF[SET][b][1], y0 = fT[SET][a][0], y1 = fT[SET][a][1];
            const i32x8 fa = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            const i32x8 fb = {(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[a][b], 0, 0, 0, 0, 0, 0);
        }
    };

    // Instruction order inside a substep (SCHED 1: the next substep's
    // fragment reads first, then the MFMAs; SCHED 2: reads interleaved one
    // per MFMA; SCHED 3: as 2, and the memory -> LDS fills of the step are
    // spread over its first substeps, one per MFMA, instead of being issued
    // in a burst at its start; 0: left to the compiler). With one wave per
    // SIMD nothing else issues MFMAs while a wave issues its fills.
    constexpr int NRD = NR * (NBF + NBT), NMF = NBT * NBF;
    auto order_substep = [&](auto nfc) {
        constexpr int NFI = decltype(nfc)::value;   // fills issued in this substep
        if constexpr (SCHED == 3) {
            static_for<NMF>([&](auto i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                if constexpr (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                if constexpr (i < NFI) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM (fill)
            });
            if constexpr (NRD > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NRD - NMF, 0);
            if constexpr (NFI > NMF) __builtin_amdgcn_sched_group_barrier(0x010, NFI - NMF, 0);
        } else if constexpr (SCHED == 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);   // MFMA
        } else if constexpr (SCHED == 2) {
            static_for<NMF>([&](auto i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            });
            if constexpr (NRD > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NRD - NMF, 0);
        }
    };

    // Pipelines. Direct loads (PF = 0): step j's token rows go to token stage
    // j % NS and its weight rows to weight stage j % NSF; at step kt the loads
    // of token step kt + NS - 1 and weight step kt + NSF - 1 are issued (token
    // first), into the stages freed by the previous step. With NS = NSF the
    // loads of the NS - 2 later steps may stay in flight at the end of a
    // step; with NS = 2, NSF = 3 the weight loads of step kt + 2 may.
    static_assert(PF == 0 || (PF == 2 && NS == 2 && NSF == 2), "register prefetch runs on two stages");
    static_assert(NSF == NS || (NS == 2 && NSF == 3 && PF == 0), "uneven stages: two token, three weight");
    // SCHED 3 spreads the fills of the uneven direct-load pipeline over the
    // substeps before the barrier; SCHED 4 issues them in the substep after
    // it, one step earlier (step kt fills token step kt + 2 and weight step
    // kt + 3 into the stages it has just finished reading), which gives every
    // fill one more substep to land before its wait.
    constexpr bool SPREAD = SCHED >= 3, LATE = SCHED == 4;
    static_assert(!SPREAD || (PF == 0 && NS == 2 && NSF == 3 && SUB >= 2), "spread fills: uneven stages");
    // explicit substeps: after MFMA i come reads [i RPG, (i + 1) RPG) and fills [i FPG, (i + 1) FPG)
    constexpr int RPG = (NRD + NMF - 1) / NMF, FPG = (NPT + NPF + NMF - 1) / NMF;
    auto reads_after = [&](auto setc, auto sc, auto tbc, auto fbc, auto ic) {
        static_for<RPG>([&](auto k) {
            constexpr int j = decltype(ic)::value * RPG + decltype(k)::value;
            if constexpr (j < NRD) read_one(setc, sc, tbc, fbc, std::integral_constant<int, j>{});
        });
    };
    // fill f of a step's set: token fills 0..NPT-1, then weight fills
    auto fill_one = [&](auto fc, LDSPTR lt, LDSPTR lf, int ktT, int ktF) {
        constexpr int f = decltype(fc)::value;
        if constexpr (f < NPT) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, lt + f * RPI * RB, 16, voT[f], ktT * RB, 0, 0);
        else if constexpr (f < NPT + NPF) issueF_one(ktF, lf, std::integral_constant<int, f - NPT>{});
    };
    constexpr int LOOP = (NS == NSF) ? NS : 6;    // steps per loop iteration (stage indices repeat)

    // One K step on token stage TB and weight stage FB: the fragments of
    // substep 0 are already in register set P. Substeps 0..SUB-2 load the
    // next substep's fragments while their MFMAs run; the last substep's
    // fragments are in registers before the barrier, so after it the next
    // step's first fragments load while the last MFMAs run. Substep s
    // computes from set (P + s) mod 2.
    auto kstep = [&](auto tbc, auto fbc, auto pc, int kt) {
        constexpr int TB = decltype(tbc)::value, FB = decltype(fbc)::value, P = decltype(pc)::value;
        if constexpr (PF == 0 && NS == NSF) {
            if (kt + NS - 1 < nk) issueT(kt + NS - 1, std::integral_constant<int, (TB + NS - 1) % NS>{});
            if (kt + NSF - 1 < nk) issueF(kt + NSF - 1, std::integral_constant<int, (FB + NSF - 1) % NSF>{});
        } else if constexpr (PF == 0 && !SPREAD) {
            // uneven stages, branch-free: past the last step the fills repeat
            // step nk - 1 into stages that are not read again
            issueT(min(kt + 1, nk - 1), std::integral_constant<int, (TB + 1) % 2>{});
            issueF(min(kt + 2, nk - 1), std::integral_constant<int, (FB + 2) % 3>{});
        }
        // (SPREAD: the fill bases are taken here, outside the substeps, so
        // that their register moves do not split the substeps' scheduling)
        LDSPTR ltS = nullptr, lfS = nullptr;
        if constexpr (SPREAD && !LATE) {
            ltS = untracked(stT(std::integral_constant<int, (TB + 1) % 2>{}) + wave * 1024);
            lfS = untracked(stF(std::integral_constant<int, (FB + 2) % 3>{}) + wave * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
        static_for<SUB - 1>([&](auto s) {
            if constexpr (SPREAD) {
                // in this order: MFMA i, fragment read i of the next substep,
                // fill i (token fills in substep 0, weight fills after them,
                // in substep 1 or, with two substeps, also in substep 0)
                constexpr int S = decltype(s)::value;
                // fills [F0, F1) of the step go in this substep
                constexpr int F0 = LATE || S > 1 || (S == 1 && SUB == 2) ? 0 : (S == 0 ? 0 : NPT);
                constexpr int F1 = LATE || S > 1 ? 0 : (SUB == 2 ? NPT + NPF : (S == 0 ? NPT : NPT + NPF));
                constexpr int FG = (F1 - F0 + NMF - 1) / NMF;
                const int ktT = min(kt + 1, nk - 1), ktF = min(kt + 2, nk - 1);
                static_for<NMF>([&](auto i) {
                    mfma_one(std::integral_constant<int, (P + S) & 1>{}, i);
                    reads_after(std::integral_constant<int, (P + S + 1) & 1>{}, std::integral_constant<int, S + 1>{},
                                tbc, fbc, i);
                    static_for<FG>([&](auto k) {
                        constexpr int f = F0 + decltype(i)::value * FG + decltype(k)::value;
                        if constexpr (f < F1) fill_one(std::integral_constant<int, f>{}, ltS, lfS, ktT, ktF);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else {
                load_frags(std::integral_constant<int, (P + s + 1) & 1>{}, std::integral_constant<int, s + 1>{},
                           tbc, fbc);
                mfmas(std::integral_constant<int, (P + s) & 1>{});
                order_substep(std::integral_constant<int, 0>{});
            }
            __builtin_amdgcn_sched_barrier(0);   // keep later fragment loads out of this substep
        });
        if constexpr (PF == 0) {
            // this wave's fills of step kt + 1 have landed (then, after the barrier, everyone's)
            if constexpr (NS == NSF) {
                if (kt + NS - 1 < nk) vmwait(std::integral_constant<int, (NPT + NPF) * (NS - 2)>{});
                else vmwait(std::integral_constant<int, 0>{});
            } else {
                vmwait(std::integral_constant<int, NPF>{});   // the weight fills of step kt + 2 may stay in flight
            }
        } else {
            // step kt + 1's registers (fetched two steps ago) go to the free
            // stage; that set then fetches step kt + 3
            if (kt + 1 < nk) {
                if (kt + 2 < nk) vmwait(std::integral_constant<int, NPT + NPF>{});
                else vmwait(std::integral_constant<int, 0>{});
                lwrite(std::integral_constant<int, (TB + 1) % 2>{}, std::integral_constant<int, (TB + 1) % 2>{});
                if (kt + 3 < nk) gload(kt + 3, std::integral_constant<int, (TB + 1) % 2>{});
            }
        }
        lds_barrier();                   // nobody reads stages TB / FB any more
        if constexpr (LATE) {
            // last substep: MFMA i, read i of the next step's first substep,
            // fill i: token step kt + 2 into stage TB, then weight step kt + 3
            // into stage FB (past the last step: repeats of step nk - 1 into
            // stages that are not read again)
            const LDSPTR ltL = untracked(stT(tbc) + wave * 1024), lfL = untracked(stF(fbc) + wave * 1024);
            __builtin_amdgcn_sched_barrier(0);
            const int ktT = min(kt + 2, nk - 1), ktF = min(kt + 3, nk - 1);
            static_for<NMF>([&](auto i) {
                mfma_one(std::integral_constant<int, (P + SUB - 1) & 1>{}, i);
                reads_after(std::integral_constant<int, (P + SUB) & 1>{}, std::integral_constant<int, 0>{},
                            std::integral_constant<int, (TB + 1) % NS>{}, std::integral_constant<int, (FB + 1) % NSF>{},
                            i);
                static_for<FPG>([&](auto k) {
                    fill_one(std::integral_constant<int, decltype(i)::value * FPG + decltype(k)::value>{}, ltL, lfL,
                             ktT, ktF);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            if (NS != NSF || kt + 1 < nk)    // (uneven stages: after the last step these reads are unused)
                load_frags(std::integral_constant<int, (P + SUB) & 1>{}, std::integral_constant<int, 0>{},
                           std::integral_constant<int, (TB + 1) % NS>{}, std::integral_constant<int, (FB + 1) % NSF>{});
            mfmas(std::integral_constant<int, (P + SUB - 1) & 1>{});
            order_substep(std::integral_constant<int, 0>{});
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    using I0 = std::integral_constant<int, 0>;
    if constexpr (PF == 0) {
        if constexpr (NS == NSF) {
            static_for<NS - 1>([&](auto b) {
                if (b < nk) {
                    issueT(b, b);
                    issueF(b, b);
                }
            });
            if (NS - 1 <= nk) vmwait(std::integral_constant<int, (NPT + NPF) * (NS - 2)>{});
            else vmwait(I0{});
        } else if constexpr (LATE) {
            // steps 0 and 1 of both operands and weight step 2; at the first
            // step's wait only weight step 2 may still be in flight
            issueT(0, I0{});
            issueF(0, I0{});
            issueF(min(1, nk - 1), std::integral_constant<int, 1>{});
            issueT(min(1, nk - 1), std::integral_constant<int, 1>{});
            issueF(min(2, nk - 1), std::integral_constant<int, 2>{});
            vmwait(std::integral_constant<int, NPF + NPT + NPF>{});
        } else {
            issueT(0, I0{});
            issueF(0, I0{});
            issueF(min(1, nk - 1), std::integral_constant<int, 1>{});
            vmwait(std::integral_constant<int, NPF>{});
        }
    } else {
        gload(0, I0{});
        if (1 < nk) {
            gload(1, std::integral_constant<int, 1>{});
            vmwait(std::integral_constant<int, NPT + NPF>{});
        } else {
            vmwait(I0{});
        }
        lwrite(I0{}, I0{});
        if (2 < nk) gload(2, I0{});
    }
    lds_barrier();
    load_frags(I0{}, I0{}, I0{}, I0{});
    // LOOP steps per iteration; LOOP * SUB even, so every iteration starts on set 0
    static_assert((LOOP * SUB) % 2 == 0, "register set parity");
    for (int kt = 0; kt < nk; kt += LOOP) {
        static_for<LOOP>([&](auto b) {
            if (kt + b < nk)
                kstep(std::integral_constant<int, b % NS>{}, std::integral_constant<int, b % NSF>{},
                      std::integral_constant<int, (b * SUB) & 1>{}, kt + b);
        });
    }
    if constexpr (NS != NSF) {
        // the repeated fills past the last step must land before the epilogue reuses the LDS
        vmwait(I0{});
        lds_barrier();
    }

    // ---------------------------------------------------------------- epilogue
    // Each wave stages 32 tokens x 64 of its outputs (fp32, scaled) per round
    // in a private LDS slice (a wave with 128 outputs takes two rounds per 32
    // tokens, one per half), rows padded to 272 bytes so that both the writes
    // from the accumulator layout and the row reads are free of bank
    // conflicts, then works in row layout: a lane takes eight consecutive
    // outputs of one token (for v^T: one output column and eight consecutive
    // tokens), so every global load and store is 16-32 contiguous bytes per
    // lane and 128-256 per token row. The pipeline's LDS is free here: every
    // wave has passed the last step's barrier, after which nobody reads it.
    static_assert(WF % 64 == 0, "a wave's rows hold whole halves of 64 outputs");
    constexpr int NH = WF / 64;
    constexpr int RS = 64 * 4 + 16;
    // wave slices packed into the stage arrays in order sT0.., sF0..
    constexpr int SL = 32 * RS, capT = LDS_T / SL, capF = LDS_F / SL;
    static_assert(NS * capT + NSF * capF >= NW, "epilogue slices");
    uint8_t* wl = nullptr;
    {
        int w = wave;
        auto take = [&](uint8_t* arr, int cap) {
            if (wl) return;
            if (w < cap) wl = arr + w * SL;
            else w -= cap;
        };
        take(sT0, capT);
        take(sT1, capT);
        if constexpr (NS > 2) take(sT2, capT);
        if constexpr (NS > 3) take(sT3, capT);
        take(sF0, capF);
        take(sF1, capF);
        if constexpr (NSF > 2) take(sF2, capF);
        if constexpr (NSF > 3) take(sF3, capF);
    }
    float scb[NBF];
    if constexpr (MODE == EPI_SWIGLU) {
        const float sg = epi_scale(ep.amax_a, ep.s_w), su = epi_scale(ep.amax_a, ep.s_w2);
#pragma unroll
        for (int b = 0; b < NBF; ++b) scb[b] = (b & 1) ? su : sg;   // 32-row blocks: gate, up
    } else {
        const float sc = epi_scale(ep.amax_a, ep.s_w);
#pragma unroll
        for (int b = 0; b < NBF; ++b) scb[b] = sc;
    }
    const int fwave = f0 + wf * WF;       // first output (for SwiGLU: interleaved gate/up row) of the wave
    float mx = 0.f;
    // RESID: every residual row the epilogue adds (16 bytes of bf16 per lane,
    // row and round) is loaded here, before the first store. Vector memory
    // loads and stores share one in-order counter, so a load issued after a
    // store cannot be waited for without waiting for that store too. The
    // loads are unconditional (rows past M read row M - 1) and the h stores
    // go through a buffer descriptor that drops rows past M, so the rounds
    // are straight-line code in which the compiler can count exactly which
    // loads have landed; with a branch per row it waited for every earlier
    // store before each row.
    constexpr int NROUND = NBT * NH;   // rounds
    uint4 xres[MODE == EPI_RESID ? NROUND : 1][4];
    __amdgpu_buffer_rsrc_t rsH;
    if constexpr (MODE == EPI_RESID) {
        static_assert(std::is_same<TOUT, bf16_t>::value, "bf16 residual rows");
        int mr[NROUND * 4];
        const TOUT* rp[NROUND * 4];
#pragma unroll
        for (int k = 0; k < NROUND; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mr[4 * k + i] = min(t0 + wt * WT + (k / NH) * 32 + (lane >> 3) + 8 * i, ep.M - 1);
        seq_rows<TOUT>(ep.xin, mr, ep.D, rp);
#pragma unroll
        for (int k = 0; k < NROUND; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xres[k][i] = *(const uint4*)(rp[4 * k + i] + fwave + 64 * (k % NH) + (lane & 7) * 8);
        rsH = make_rsrc(ep.h + (size_t)t0 * ep.D, (min(ep.M, t0 + BT) - t0) * ep.D * 4);
    }
    auto row8 = [&](int r, int c0, float v[8]) {
        const float4 x = *(const float4*)(wl + r * RS + c0 * 4), y = *(const float4*)(wl + r * RS + c0 * 4 + 16);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    };
    // accumulator layout -> LDS rows of round ah: lane (token lrow) holds
    // outputs b 32 + 8 g + 4 h .. + 3
    auto stage = [&](auto ah) {
        constexpr int a = decltype(ah)::value / NH, hb = 2 * (decltype(ah)::value % NH);
        static_for<2>([&](auto b) {
            static_for<4>([&](auto g) {
                *(float4*)(wl + lrow * RS + (b * 32 + 8 * g + 4 * lhalf) * 4) =
                    make_float4(acc[a][hb + b][4 * g] * scb[hb + b], acc[a][hb + b][4 * g + 1] * scb[hb + b],
                                acc[a][hb + b][4 * g + 2] * scb[hb + b], acc[a][hb + b][4 * g + 3] * scb[hb + b]);
            });
        });
    };
    if constexpr (MODE == EPI_QKV) {
        // A wave's 64 outputs lie in one of q, k, v and one head (I and dh are
        // multiples of 64), so the choice is made once per wave.
        static_assert(NH == 1, "one 64-output half per wave");
        static_assert(std::is_same<TOUT, bf16_t>::value, "bf16 q, k, v");
        const int which = fwave / ep.I;
        const int rem = fwave - which * ep.I;
        const int head = rem / ep.dh;
        const int dw = rem - head * ep.dh;   // head-local feature of output column 0
        if (which < 2) {
            // q, k: rotary embedding with the row's (cos, sin) pairs, head-major
            // rows; rows [M, Mpad) zero. The rotary rows of round k + 1 (32
            // bytes a lane and row; rows past M read row M - 1) are loaded
            // before round k's stores, and the stores go through a descriptor
            // bounded at Mpad rows: the rounds are straight-line code, so no
            // load waits for an earlier store (loads and stores share one
            // in-order counter).
            const __amdgpu_buffer_rsrc_t rsQK =
                make_rsrc((const TOUT*)(which ? ep.k : ep.q) + (size_t)head * ep.Sp * ep.dh, ep.Mpad * ep.dh * 2);
            const int c0 = (lane & 7) * 8;
            float4 rcs[2][4][2];
            auto rope_load = [&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NROUND) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = min(t0 + wt * WT + k * 32 + (lane >> 3) + 8 * i, ep.M - 1);
                        const float4* t = (const float4*)(ep.rope.rows + (size_t)m * (ep.dh >> 1) + ((dw + c0) >> 1));
                        rcs[k & 1][i][0] = t[0];
                        rcs[k & 1][i][1] = t[1];
                    }
                }
            };
            rope_load(I0{});
            static_for<NROUND>([&](auto ah) {
                constexpr int k = decltype(ah)::value;
                stage(ah);
                rope_load(std::integral_constant<int, k + 1>{});
                const int mb = t0 + wt * WT + k * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = (lane >> 3) + 8 * i, m = mb + r;
                    float v[8];
                    row8(r, c0, v);
                    const float4 c01 = rcs[k & 1][i][0], c23 = rcs[k & 1][i][1];
                    const float2 cs[4] = {make_float2(c01.x, c01.y), make_float2(c01.z, c01.w),
                                          make_float2(c23.x, c23.y), make_float2(c23.z, c23.w)};
                    const bool live = m < ep.M;
                    u32x4_t o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x = v[2 * j], y = v[2 * j + 1];
                        // (x + i y)(c + i s), each part one product rounded, then a fused multiply-add
                        const float re = __builtin_fmaf(x, cs[j].x, -(y * cs[j].y));
                        const float im = __builtin_fmaf(x, cs[j].y, y * cs[j].x);
                        o[j] = pack_bf2(live ? re : 0.f, live ? im : 0.f);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(o, rsQK, (m * ep.dh + dw + c0) * 2, 0, 0);
                }
            });
        } else {
            // v^T [head][dh][Sp]: lane = output column, eight consecutive tokens per store
            static_for<NROUND>([&](auto ah) {
                stage(ah);
                const int mb = t0 + wt * WT + decltype(ah)::value * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m0 = mb + 8 * i;
                    if (m0 < ep.Mpad) {
                        float v[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) v[j] = m0 + j < ep.M ? *(const float*)(wl + (8 * i + j) * RS + lane * 4) : 0.f;
                        store8<TOUT>((TOUT*)ep.vt + ((size_t)head * ep.dh + dw + lane) * ep.Sp + m0, v);
                    }
                }
            });
        }
    }
    // DOWN without update rows (every row y = h + acc into its segment's
    // output): the residual rows of round k + 1 (32 bytes of fp32 per lane
    // and row; rows past M read row M - 1) are loaded before round k's
    // stores, and the stores need no branch (rows past M write the sink), so
    // no load waits for an earlier store (one in-order counter for both). A
    // loop of its own, so that its registers and the update path's are not
    // live together.
    bool done = false;
    if constexpr (MODE == EPI_DOWN) {
        static_assert(NH == 1, "one 64-output half per wave");
        static_assert(std::is_same<TOUT, bf16_t>::value, "bf16 rows");
        if (!ep.out.delta && ep.sink && !pslot) {
            done = true;
            const int c0 = (lane & 7) * 8;
            float hpf[2][4][8];
            auto hload = [&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NROUND) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = min(t0 + wt * WT + k * 32 + (lane >> 3) + 8 * i, ep.M - 1);
                        load8<float>(ep.hres + (size_t)m * ep.D + fwave + c0, hpf[k & 1][i]);
                    }
                }
            };
            hload(I0{});
            const SeqOut& o = ep.out;
            const int nt = ep.xin.nt, nv = ep.xin.nv, nc = ep.xin.nc;
            static_for<NROUND>([&](auto ah) {
                constexpr int k = decltype(ah)::value;
                stage(ah);
                hload(std::integral_constant<int, k + 1>{});
                const int mb = t0 + wt * WT + k * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = (lane >> 3) + 8 * i, m = mb + r;
                    float v[8];
                    row8(r, c0, v);
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = hpf[k & 1][i][j] + v[j];
                    const int n0 = fwave + c0;
                    TOUT* dst = m >= ep.M          ? (TOUT*)ep.sink
                                : m < nt           ? (TOUT*)o.yt + (size_t)m * ep.D + n0
                                : m < nt + nv      ? (TOUT*)o.yv + (size_t)(m - nt) * ep.D + n0
                                : m < nt + nv + nc ? (TOUT*)o.yc + (size_t)(m - nt - nv) * ep.D + n0
                                                   : (TOUT*)o.ya + (size_t)(m - nt - nv - nc) * ep.D + n0;
                    store8<TOUT>(dst, v);
                }
            });
        }
    }
    if constexpr (MODE != EPI_QKV) if (!done) static_for<NBT * NH>([&](auto ah) {
        constexpr int a = decltype(ah)::value / NH, hb = 2 * (decltype(ah)::value % NH);   // token block, first feature block of the half
        stage(ah);
        const int fw = fwave + 32 * hb;         // first output of the half
        const int mb = t0 + wt * WT + a * 32;   // first token of the round
        if constexpr (MODE == EPI_SWIGLU) {
            // columns 0..31 gate, 32..63 up of ffn features fw / 2 .. + 31; four lanes per token
            using UT = TOUT;   // u in the activation dtype (bf16); fp8 quantises it from there
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = (lane >> 2) + 16 * i, j0 = (lane & 3) * 8;
                float g[8], u[8];
                row8(r, j0, g);
                row8(r, 32 + j0, u);
                mx = fmaxf(mx, epi8_swiglu<UT>(ep, mb + r, fw / 2 + j0, g, u));
            }
        } else if constexpr (MODE == EPI_DOWN) {
            // every load of the round's four rows before its first store; with
            // fp8 (fewer free registers here) the residual rows of all four,
            // then each row's reference and rectangle rows before its store
            static_assert(std::is_same<TOUT, bf16_t>::value, "bf16 rows");
            DownRow dr[4];
            if (!pslot) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    down_issue_h(ep, mb + (lane >> 3) + 8 * i, fw + (lane & 7) * 8, dr[i]);
                    if constexpr (!FP8) down_issue_rest(ep, mb + (lane >> 3) + 8 * i, fw + (lane & 7) * 8, dr[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (lane >> 3) + 8 * i, c0 = (lane & 7) * 8;
                float v[8];
                row8(r, c0, v);
                if (pslot) {
                    store8<float>(pslot + (size_t)(mb - t0 + r) * BF + (fw - f0 + c0), v);
                } else {
                    if constexpr (FP8) down_issue_rest(ep, mb + r, fw + c0, dr[i]);
                    down_finish(ep, mb + r, fw + c0, v, dr[i]);
                }
            }
        } else if (pslot) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (lane >> 3) + 8 * i, c0 = (lane & 7) * 8;
                float v[8];
                row8(r, c0, v);
                store8<float>(pslot + (size_t)(mb - t0 + r) * BF + (fw - f0 + c0), v);
            }
        } else {
            // h = X + acc (fp32), rows past M dropped by the descriptor's bound
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (lane >> 3) + 8 * i, c0 = (lane & 7) * 8;
                float v[8];
                row8(r, c0, v);
                const uint4 x = xres[decltype(ah)::value][i];
                const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
                u32x4_t o[2];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[j >> 1][2 * (j & 1)] = __float_as_uint(__uint_as_float(xw[j] << 16) + v[2 * j]);
                    o[j >> 1][2 * (j & 1) + 1] = __float_as_uint(__uint_as_float(xw[j] & 0xFFFF0000u) + v[2 * j + 1]);
                }
                const int off = ((mb - t0 + r) * ep.D + fw + c0) * 4;
                __builtin_amdgcn_raw_buffer_store_b128(o[0], rsH, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(o[1], rsH, off + 16, 0, 0);
            }
        }
    });
    if constexpr (MODE == EPI_SWIGLU) {
        if (ep.u_amax) {
            // one atomic per workgroup; the wave maxima go to the tail of sT0,
            // past the epilogue slices packed into it
            static_assert(LDS_T - capT * SL >= NW * 4, "room for the wave maxima");
            float* wmax = (float*)(sT0 + LDS_T - NW * 4);
            mx = wave_max(mx);
            if (lane == 0) wmax[wave] = mx;
            __syncthreads();
            if (tid == 0) {
                float m = wmax[0];
#pragma unroll
                for (int w = 1; w < NW; ++w) m = fmaxf(m, wmax[w]);
                atomic_max_nonneg(ep.u_amax, m);
            }
        }
    }
#endif  // device pass only: the host pass keeps just the launch stub
}

// K-split tail, second pass: one thread per 8 consecutive outputs of a tail
// tile row; the slices are added in slice order, then the RESID / DOWN
// epilogue runs on the sum.
template <int MODE, int BT, int BF, bool FP8>
__global__ __launch_bounds__(256) void split_reduce_kernel(int M, int N, int nfull, int splits, EpiParams ep) {
    constexpr int TPR = BF / 8, RPB = 256 / TPR;   // threads per row, rows per block
    static_assert(BT % RPB == 0, "rows");
    const int r = blockIdx.x / (BT / RPB);
    const int row = (blockIdx.x % (BT / RPB)) * RPB + threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * 8;
    int t0, f0;
    tile_origin<BT, BF, tile_group(FP8)>(nfull + r, M, N, t0, f0);
    if (t0 + row >= M) return;
    const float* p = ep.part + ((size_t)r * splits * BT + row) * BF + c0;
    float v[8], x[8];
    load8<float>(p, v);
    for (int k = 1; k < splits; ++k) {
        load8<float>(p + (size_t)k * BT * BF, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += x[i];
    }
    if constexpr (MODE == EPI_RESID) epi8_resid<bf16_t>(ep, t0 + row, f0 + c0, v);
    else epi8_down<bf16_t>(ep, t0 + row, f0 + c0, v);
}

// Split of the tail: whole tiles fill `cus` compute units `nfull / cus`
// times; the remaining tiles run as K slices, `splits` per tile, at most one
// unit per compute unit, each slice at least 4 K steps.
struct SplitPlan {
    int nfull = 0, splits = 1;
    size_t bytes = 0;
};
constexpr int SPLIT_BT = 256, SPLIT_BF = 256;

SplitPlan split_plan(bool fp8, int mode, int M, int N, int K, int cus) {
    SplitPlan p;
    if ((mode != EPI_RESID && mode != EPI_DOWN) || N % SPLIT_BF || cus <= 0 || M <= 0) return p;
    const long tiles = (long)((M + SPLIT_BT - 1) / SPLIT_BT) * (N / SPLIT_BF);
    if (tiles < 32) return p;
    const long nfull = tiles / cus * cus, tail = tiles - nfull;
    if (tail == 0) return p;
    const int nk = K / (fp8 ? 128 : 64);
    int s = (int)std::min<long>(8, cus / tail);
    while (s > 1 && (nk % s || nk / s < 4)) --s;
    if (s < 2) return p;
    p.nfull = (int)nfull;
    p.splits = s;
    p.bytes = (size_t)tail * s * SPLIT_BT * SPLIT_BF * sizeof(float);
    return p;
}

// compute units of the current device (cached per device; 256 when it cannot be read)
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
        (void)hipGetLastError();
        c = 256;
    }
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <int BT, int BF, int WGT, int WGF, int NS, int NSF, int RB, int PF, int OCC, int SCHED, bool FP8, int MODE>
hipError_t launch_t(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st, const SplitPlan& sp = SplitPlan{}) {
    static_assert((NS * BT + NSF * BF) * RB <= 160 * 1024, "LDS");   // NS token and NSF weight stages
    const int tiles = ((M + BT - 1) / BT) * (N / BF);
    const int nfull = sp.splits > 1 ? sp.nfull : tiles;
    const int grid = nfull + (tiles - nfull) * sp.splits;
    hipLaunchKernelGGL((gemm_mfma_kernel<BT, BF, WGT, WGF, NS, NSF, RB, PF, OCC, SCHED, FP8, MODE, bf16_t>),
                       dim3(grid), dim3(64 * WGT * WGF), 0, st, (const uint8_t*)A, (const uint8_t*)W0,
                       (const uint8_t*)W1, M, N, K, nfull, sp.splits, ep);
    if constexpr ((MODE == EPI_RESID || MODE == EPI_DOWN) && BT == SPLIT_BT && BF == SPLIT_BF) {
        if (sp.splits > 1) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((split_reduce_kernel<MODE, BT, BF, FP8>), dim3((tiles - nfull) * (BT / (256 / (BF / 8)))),
                               dim3(256), 0, st, M, N, nfull, sp.splits, ep);
        }
    }
    return hipGetLastError();
}

template <bool FP8, int MODE>
hipError_t dispatch(const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st) {
    // 256 x 256 tiles: fills spread over the substeps; for the long-K down
    // projection and every fp8 projection issued one step early (measured on
    // the 540p block and the fp8 stack: bf16 QKV, gate/up and O fastest with
    // the first, the others with the second)
    constexpr int SCH = (FP8 || MODE == EPI_DOWN) ? 4 : 3;
    if constexpr (MODE == EPI_RESID || MODE == EPI_DOWN) {
        // 256 x 256 tiles with a K-split tail when the partial buffer holds it
        const SplitPlan sp = split_plan(FP8, MODE, M, N, K, device_cus());
        if (sp.splits > 1 && ep.part && sp.bytes <= ep.part_bytes)
            return launch_t<256, 256, 2, 4, 2, 3, 128, 0, 2, SCH, FP8, MODE>(A, W0, W1, M, N, K, ep, st, sp);
    }
    // big tiles when there are enough of them to fill 256 CUs several times
    const long t256 = (long)((M + 255) / 256) * (N / 256);
    if (N % 256 == 0 && t256 >= 512) return launch_t<256, 256, 2, 4, 2, 3, 128, 0, 2, SCH, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
    return launch_t<128, 128, 2, 2, 2, 3, 128, 0, 2, 0, FP8, MODE>(A, W0, W1, M, N, K, ep, st);
}

}  // namespace detail
using namespace detail;

// A split never has more than min(cus, 8 x tiles) slice units (at most 8
// slices of at most cus / tail units each), and no split happens below 32 tiles.
size_t gemm_split_bytes_bound(int M, int N) {
    if (M <= 0 || N % SPLIT_BF) return 0;
    const long tiles = (long)((M + SPLIT_BT - 1) / SPLIT_BT) * (N / SPLIT_BF);
    if (tiles < 32) return 0;
    return (size_t)std::min<long>(device_cus(), 8 * tiles) * SPLIT_BT * SPLIT_BF * sizeof(float);
}

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
