// Joint-sequence attention for gfx950: o = softmax(q k^T / sqrt(dh)) v per
// head, unmasked, over [text | video | audio] (tokendh.com article, backbone
// section: one shared denoiser over all modalities; PaperDaily review,
// section 2: attention cost grows strongly with sequence length, which the
// compressed layers shorten).
//
// Inputs come from the QKV epilogue: q, k [head][Sp][dh] (rotated), v
// transposed [head][dh][Sp]; rows [S, Sp) are zero. Output o [S][heads * dh].
// The softmax runs in base 2: c = log2(e) * scale multiplies the raw scores
// inside the exp2 argument (one fma per score), so q keeps its own rounding.
//
// bf16 kernel: a workgroup of 4 waves takes 128 queries of one head, a wave
// 32 queries. The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (keys on the MFMA rows, queries on its columns): a lane then owns one
// query and 32 of its 64 scores per key tile, so the online-softmax row max
// and sum need a single exchange with the partner lane l^32. P^T goes straight
// from the accumulator to the B operand of O^T += V^T P^T; the key order
// inside each 16-key step is the accumulator's order, and V^T is read from
// LDS in that same order. K and V^T tiles of 64 keys are double-buffered in
// LDS with XOR swizzles for the 64-bank LDS.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace detail {

[[maybe_unused]] constexpr int KT = 64;   // keys per tile (device code only)
constexpr int QW = 32;   // queries per wave
typedef __attribute__((address_space(3))) uint8_t* LDSPTR;

DIT_DEV int swzK(int row, int c) { return c ^ (row & 15); }          // 16-byte chunks, 256-byte K rows
DIT_DEV int swzV(int row, int c) { return c ^ ((row >> 1) & 7); }    // 16-byte chunks, 128-byte V^T rows
// Key order of the S^T rows: lane row i reads key rho(i) (bits 2 and 3
// swapped) so that each lane's eight P values of a 16-key step are 8
// consecutive keys, matching one 16-byte read of a V^T row.
DIT_DEV int rho(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// lanes l and l ^ 32 exchange through v_permlane32_swap (no LDS round trip):
// the swap of x with itself leaves (low half, high half) of x in the two results
DIT_DEV void swap32(float x, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

// Software pipelining: iteration t issues the score MFMAs of key tile t next
// to the rescale of O, then the P V MFMAs of tile t - 1 next to the softmax of
// tile t, so that each wave's own instruction stream keeps its SIMD's matrix
// core and VALU busy together instead of alternating between them. K and V^T
// tiles sit one tile apart in LDS: iteration t reads K(t) and V^T(t - 1) while
// K(t + 1) and V^T(t) are in flight, two stages per operand; its second half
// fills K(t + 2) and V^T(t + 1) (details at the iteration below).
template <int NW>
__global__ __launch_bounds__(64 * NW, (NW == 4 ? 2 : 1)) void attn_bf16_pipe_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ Vt, bf16_t* __restrict__ O,
    int S, int Sp, int nh, float c, float* o_amax) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(NW == 4 || NW == 8, "waves");
    constexpr int DH = 128, QB = QW * NW;
    __shared__ __attribute__((aligned(16))) uint8_t sK0[KT * DH * 2];
    __shared__ __attribute__((aligned(16))) uint8_t sK1[KT * DH * 2];
    __shared__ __attribute__((aligned(16))) uint8_t sV0[DH * KT * 2];
    __shared__ __attribute__((aligned(16))) uint8_t sV1[DH * KT * 2];
    // stage bases; the stage index is a compile-time constant in the main
    // loop and a run-time value (t % 2) in the last iterations
    auto stK = [&](int bc) -> uint8_t* { return bc ? sK1 : sK0; };
    auto stV = [&](int bc) -> uint8_t* { return bc ? sV1 : sV0; };

    const int nq = (S + QB - 1) / QB;
    const int blk = xcd_remap(blockIdx.x, nq * nh);
    const int head = blk / nq;
    const int qt = blk - head * nq;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int q0 = qt * QB + wave * QW;

    const bf16_t* Qh = Q + (size_t)head * Sp * DH;
    const bf16_t* Kh = K + (size_t)head * Sp * DH;
    const bf16_t* Vh = Vt + (size_t)head * DH * Sp;

    const __amdgpu_buffer_rsrc_t rsQ = make_rsrc(Qh, Sp * DH * 2);
    bf16x8_v qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = __builtin_bit_cast(bf16x8_v, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rsQ, ((q0 + lrow) * DH + 16 * s + 8 * lhalf) * 2, 0, 0));
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]), "v"(qf[7]));

    const __amdgpu_buffer_rsrc_t rsK = make_rsrc(Kh, Sp * DH * 2);
    const __amdgpu_buffer_rsrc_t rsV = make_rsrc(Vh, Sp * DH * 2);
    const int krow = 4 * wave + (lane >> 4);
    const int voK = krow * 256 + swzK(krow, lane & 15) * 16;
    const int vrow = 8 * wave + (lane >> 3);
    const int voV = vrow * Sp * 2 + swzV(vrow, lane & 7) * 16;
    auto untracked = [](uint8_t* p) {
        uint32_t a = (uint32_t)(uintptr_t)(LDSPTR)p;
        asm volatile("" : "+s"(a));
        return (LDSPTR)(uintptr_t)a;
    };
    constexpr int NF = 16 / NW;   // fills per operand, wave and tile
    auto fillK_one = [&](int kt, LDSPTR lk, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, lk + i * NW * 1024, 16, voK, kt * KT * 256 + i * 4 * NW * 256, 0,
                                                 0);
    };
    auto fillV_one = [&](int kt, LDSPTR lv, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, lv + i * NW * 1024, 16, voV, kt * KT * 2 + i * 8 * NW * Sp * 2, 0,
                                                 0);
    };
    auto fillK = [&](int kt, auto bc) {
        LDSPTR lk = untracked(stK(bc) + wave * 1024);
#pragma unroll
        for (int i = 0; i < NF; ++i) fillK_one(kt, lk, i);
    };
    auto fillV = [&](int kt, auto bc) {
        LDSPTR lv = untracked(stV(bc) + wave * 1024);
#pragma unroll
        for (int i = 0; i < NF; ++i) fillV_one(kt, lv, i);
    };
    auto vmwait0 = []() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); };

    int kOff[8], vOff[4];
    {
        const int kr = rho(lrow);
#pragma unroll
        for (int s = 0; s < 8; ++s) kOff[s] = kr * 256 + swzK(kr, 2 * s + lhalf) * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vOff[ks] = lrow * 128 + swzV(lrow, 2 * ks + lhalf) * 16;
    }

    f32x16 o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float mrun = -INFINITY, lrun = 0.f;   // lrun: this lane's half of the row sum
    float alpha = 1.f;                     // O rescale owed before the next P V product
    uint32_t pk[2][8];                     // P of the previous tile, bf16 pairs
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) pk[b][j] = 0u;
    const bf16x2_v ones = {(__bf16)1.f, (__bf16)1.f};
    const int nkt = (S + KT - 1) / KT;

    // Iteration t on K stage KB = t % 2 (V^T(t - 1) is in stage KB ^ 1).
    // QK: tile t exists (t < nkt); PV: tile t - 1 exists (t >= 1); MASK: tile
    // t is the last one and keys >= S are masked.
    // Entering iteration t: K(t) and V^T(t - 1) are in LDS, the first half of
    // K(t)'s fragments in kpre; this wave's fills of K(t + 1) and V^T(t) are in
    // flight. The barrier sits in phase B right after its last V^T read: then
    // every wave is done with K(t) and V^T(t - 1), and the rest of phase B
    // fills K(t + 2) and V^T(t + 1) into their stages and reads K(t + 1)'s
    // first fragments, so phase A starts on fragments already in registers.
    bf16x8_v kpre[4][2];
    auto step = [&](int t, auto kbc, auto qkc, auto pvc, auto maskc) {
        const int KB = kbc;
        constexpr bool QK = decltype(qkc)::value, PV = decltype(pvc)::value, MASK = decltype(maskc)::value;
        // The two phases are written slot by slot, one MFMA per slot with the
        // VALU work and LDS reads that should issue beside it; the fences keep
        // the compiler from regrouping them (it otherwise issues all MFMAs of a
        // phase back to back and the VALU work after them).
        auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
        // ---- phase A: S(t) = K(t) Q^T on the matrix core, O *= alpha on the VALU
        f32x16 sc[2];
        bf16x8_v kf[4][2];   // second half of K(t)'s fragments
        const uint8_t* bK = stK(KB);
        // V^T(t - 1) landed before the barrier of the previous iteration, so
        // the fragments phase B starts on are read in phase A's second half
        const uint8_t* bV = stV(KB ^ 1);
        bf16x8_v vf[4][4];
        auto vread = [&](int ks, int d) { vf[ks][d] = *(const bf16x8_v*)(bV + vOff[ks] + d * 4096); };
        if constexpr (QK) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) sc[b][r] = 0.f;
        }
        fence();
        static_for<16>([&](auto ic) {
            constexpr int i = ic, s = i / 2, b = i % 2;
            if constexpr (QK) {
                if constexpr (s < 4) sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kpre[s][b], qf[s], sc[b], 0, 0, 0);
                else sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s - 4][b], qf[s], sc[b], 0, 0, 0);
            }
            if constexpr (PV) {
#pragma unroll
                for (int r = 0; r < 4; ++r) o[i / 4][(i % 4) * 4 + r] *= alpha;
            }
            if constexpr (QK && s < 4) kf[s][b] = *(const bf16x8_v*)(bK + kOff[s + 4] + b * 8192);
            if constexpr (PV && i >= 8) vread((i - 8) / 4, (i - 8) % 4);
            fence();
        });
        // ---- phase B: O^T += V^T(t - 1) P^T(t - 1) on the matrix core, softmax of S(t) on the VALU
        // fill bases of K(t + 2) (stage KB) and V^T(t + 1) (stage KB ^ 1), taken outside the slots
        LDSPTR lkN = nullptr, lvN = nullptr;
        if constexpr (QK) {
            lkN = untracked(stK(KB) + wave * 1024);
            lvN = untracked(stV(KB ^ 1) + wave * 1024);
        }
        const int ktK = min(t + 2, nkt - 1), ktV = min(t + 1, nkt - 1);   // past the end: repeats, not read again
        const uint8_t* bKn = stK(KB ^ 1);
        fence();
        float t0 = 0.f, t1 = 0.f, mc = 0.f, psum = 0.f;
        uint32_t pn[2][8];   // P of tile t
        auto pair = [&](int p) {
            const int b = p >> 3, j = p & 7;
            pn[b][j] = pack_bf2(__builtin_amdgcn_exp2f(fmaf(sc[b][2 * j], c, mc)),
                                __builtin_amdgcn_exp2f(fmaf(sc[b][2 * j + 1], c, mc)));
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, pn[b][j]), ones, psum, false);
        };
        static_for<16>([&](auto jc) {
            constexpr int j = jc, ks = j / 4, d = j % 4;
            if constexpr (PV) {
                const int b = ks >> 1, j0 = 4 * (ks & 1);
                const bf16x8_v pf = __builtin_bit_cast(
                    bf16x8_v, make_uint4(pk[b][j0], pk[b][j0 + 1], pk[b][j0 + 2], pk[b][j0 + 3]));
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][d], pf, o[d], 0, 0, 0);
                if constexpr (j == 0 || j == 1) { vread(2, 2 * j); vread(2, 2 * j + 1); }
                if constexpr (j == 6 || j == 7) { vread(3, 2 * (j - 6)); vread(3, 2 * (j - 6) + 1); }
            }
            if constexpr (QK) {
                if constexpr (j == 1 && MASK) {
                    // register r of block b holds key 32 b + rho(8 (r / 4) + 4 h + r % 4)
                    // = 32 b + 16 (r / 8) + 8 h + 4 ((r / 4) % 2) + r % 4 of the tile
                    const int lim = S - t * KT - 8 * lhalf;
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (32 * bb + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3) >= lim) sc[bb][r] = -INFINITY;
                }
                if constexpr (j == 2) {
                    t0 = fmaxf(sc[0][0], sc[0][1]);
                    t1 = fmaxf(sc[1][0], sc[1][1]);
#pragma unroll
                    for (int r = 2; r < 8; ++r) {
                        t0 = fmaxf(t0, sc[0][r]);
                        t1 = fmaxf(t1, sc[1][r]);
                    }
                }
                if constexpr (j == 3) {
#pragma unroll
                    for (int r = 8; r < 16; ++r) {
                        t0 = fmaxf(t0, sc[0][r]);
                        t1 = fmaxf(t1, sc[1][r]);
                    }
                }
                if constexpr (j == 4) {
                    float a, bb;
                    swap32(fmaxf(t0, t1), a, bb);
                    const float mnew = fmaxf(mrun, fmaxf(a, bb));
                    alpha = __builtin_amdgcn_exp2f((mrun - mnew) * c);
                    mrun = mnew;
                    mc = -mnew * c;
                }
                // the 16 exp pairs over slots 5..15: two in slots 5..9, one after
                if constexpr (j >= 5 && j <= 9) { pair(2 * (j - 5)); pair(2 * (j - 5) + 1); }
                if constexpr (j >= 10) pair(j);
                if constexpr (j == 7) {
                    // the last V^T reads were in this slot: own fills of K(t + 1)
                    // and V^T(t) landed, then everyone's; K(t), V^T(t - 1) are free
                    vmwait0();
                    lds_barrier();
                }
                if constexpr (j >= 8) {
                    constexpr int f = j - 8;   // fills K(t + 2) then V^T(t + 1), one per slot
                    if constexpr (f < NF) fillK_one(ktK, lkN, f);
                    else if constexpr (f < 2 * NF) fillV_one(ktV, lvN, f - NF);
                    kpre[f / 2][f % 2] = *(const bf16x8_v*)(bKn + kOff[f / 2] + (f % 2) * 8192);
                }
            }
            fence();
        });
        if constexpr (QK) {
            lrun = lrun * alpha + psum;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int j = 0; j < 8; ++j) pk[b][j] = pn[b][j];
        }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using T_ = std::true_type;
    using F_ = std::false_type;

    fillK(0, 0);
    vmwait0();
    lds_barrier();
#pragma unroll
    for (int f = 0; f < 8; ++f) kpre[f / 2][f % 2] = *(const bf16x8_v*)(sK0 + kOff[f / 2] + (f % 2) * 8192);
    fillK(min(1, nkt - 1), 1);
    fillV(0, 0);
    int t = 1;
    if (nkt == 1) {
        step(0, B0{}, T_{}, F_{}, T_{});
    } else {
        step(0, B0{}, T_{}, F_{}, F_{});
        for (; t + 2 < nkt; t += 2) {
            step(t, B1{}, T_{}, T_{}, F_{});
            step(t + 1, B0{}, T_{}, T_{}, F_{});
        }
        // t is odd; one or two tiles remain, the last one masked
        if (t + 2 == nkt) {
            step(t, B1{}, T_{}, T_{}, F_{});
            ++t;
        }
        step(t, t & 1, T_{}, T_{}, T_{});
        ++t;
    }
    step(t, t & 1, F_{}, T_{}, F_{});   // the last P V (t = nkt)
    vmwait0();   // the repeated K fill of the last iteration

    float l0, l1;
    swap32(lrun, l0, l1);
    const float inv = 1.f / (l0 + l1);
    const int q = q0 + lrow;
    float mx = 0.f;
    if (q < S) {
        bf16_t* orow = O + (size_t)q * nh * DH + head * DH;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v0 = o[d][4 * g] * inv, v1 = o[d][4 * g + 1] * inv;
                float v2 = o[d][4 * g + 2] * inv, v3 = o[d][4 * g + 3] * inv;
                uint2 w = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
                *(uint2*)(orow + d * 32 + 8 * g + 4 * lhalf) = w;
                if (o_amax) {
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(bf2f(f2bf(v0))), fabsf(bf2f(f2bf(v1)))),
                                         fmaxf(fabsf(bf2f(f2bf(v2))), fabsf(bf2f(f2bf(v3))))));
                }
            }
    }
    if (o_amax) {
        // one atomic per workgroup
        __shared__ float wmax[NW];
        mx = wave_max(mx);
        if (lane == 0) wmax[wave] = mx;
        __syncthreads();
        if (tid == 0) {
            float m = wmax[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) m = fmaxf(m, wmax[w]);
            atomic_max_nonneg(o_amax, m);
        }
    }
#endif  // device pass only: the host pass keeps just the launch stub
}

// fp32 attention: one thread per query, 64 queries of one head per block,
// key tiles of 32 in LDS; fp32 online softmax.
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ Vt, float* __restrict__ O, int S,
                                                      int Sp, int nh, float c) {
    constexpr int KB = 32;
    __shared__ float sk[KB][DH + 1];
    __shared__ float sv[KB][DH + 1];
    const int nq = (S + 63) / 64;
    const int head = blockIdx.x / nq;
    const int qt = blockIdx.x - head * nq;
    const int q = qt * 64 + threadIdx.x;
    const float* Qh = Q + (size_t)head * Sp * DH;
    const float* Kh = K + (size_t)head * Sp * DH;
    const float* Vh = Vt + (size_t)head * DH * Sp;
    float qr[DH], acc[DH];
    const int qq = min(q, Sp - 1);
#pragma unroll
    for (int d = 0; d < DH; ++d) {
        qr[d] = Qh[(size_t)qq * DH + d];
        acc[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int k0 = 0; k0 < S; k0 += KB) {
        __syncthreads();
        for (int i = threadIdx.x; i < KB * DH; i += 64) {
            int r = i / DH, d = i - r * DH;
            int key = k0 + r;
            sk[r][d] = key < Sp ? Kh[(size_t)key * DH + d] : 0.f;
            int vd = i / KB, vr = i - vd * KB;
            int vkey = k0 + vr;
            sv[vr][vd] = vkey < Sp ? Vh[(size_t)vd * Sp + vkey] : 0.f;
        }
        __syncthreads();
        float s[KB];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            float a = 0.f;
#pragma unroll
            for (int d = 0; d < DH; ++d) a = fmaf(qr[d], sk[j][d], a);
            s[j] = (k0 + j < S) ? a : -INFINITY;
            tmax = fmaxf(tmax, s[j]);
        }
        const float mn = fmaxf(m, tmax);
        const float alpha = exp2f((m - mn) * c);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[d] *= alpha;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const float p = exp2f(fmaf(s[j], c, -mn * c));
            l += p;
#pragma unroll
            for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, sv[j][d], acc[d]);
        }
    }
    if (q < S) {
        float* orow = O + (size_t)q * nh * DH + head * DH;
        const float inv = 1.f / l;
#pragma unroll
        for (int d = 0; d < DH; ++d) orow[d] = acc[d] * inv;
    }
}

// [S][nh*dh] -> head-major padded layouts (q scaled), zero rows [S, Sp)
template <typename T>
__global__ void attn_pack_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                                 T* __restrict__ Qp, T* __restrict__ Kp, T* __restrict__ Vtp, int S, int Sp, int nh,
                                 int dh, float qscale) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)Sp * nh * dh;
    if (i >= total) return;
    const int d = (int)(i % dh);
    const int hh = (int)((i / dh) % nh);
    const int s = (int)(i / ((size_t)dh * nh));
    float qv = 0.f, kv = 0.f, vv = 0.f;
    if (s < S) {
        const size_t src = (size_t)s * nh * dh + (size_t)hh * dh + d;
        if constexpr (sizeof(T) == 2) {
            qv = bf2f(q[src]); kv = bf2f(k[src]); vv = bf2f(v[src]);
        } else {
            qv = q[src]; kv = k[src]; vv = v[src];
        }
        qv *= qscale;
    }
    const size_t o = ((size_t)hh * Sp + s) * dh + d;
    const size_t ov = ((size_t)hh * dh + d) * Sp + s;
    if constexpr (sizeof(T) == 2) {
        Qp[o] = f2bf(qv); Kp[o] = f2bf(kv); Vtp[ov] = f2bf(vv);
    } else {
        Qp[o] = qv; Kp[o] = kv; Vtp[ov] = vv;
    }
}

}  // namespace detail
using namespace detail;

// Workgroup shape: 4 waves (128 queries, two workgroups per CU) or 8 waves
// (256 queries sharing each K / V^T tile, one per CU, half the fill traffic
// per query). Outputs are identical (each wave's arithmetic is the same). The
// 8-wave form is taken only for long sequences (at least 4 rounds of
// workgroups) whose last round it fills better; elsewhere it measured 2-8 %
// slower (at 12628 tokens, 56 heads, it is 3 % faster).
int attention_waves(int S, int nh) {
    const int cus = device_cus();
    auto rounds = [&](int nw, int per_cu) {
        return (double)((S + QW * nw - 1) / (QW * nw)) * nh / (double)(cus * per_cu);
    };
    auto fill = [&](double r) { return r / std::ceil(r); };
    const double r4 = rounds(4, 2), r8 = rounds(8, 1);
    return r8 >= 4.0 && fill(r8) > fill(r4) + 0.005 ? 8 : 4;
}

hipError_t attention_bf16(const void* Q, const void* K, const void* Vt, void* O, int S, int Sp, int nh, int dh,
                          float c, float* o_amax, hipStream_t st) {
    if (dh != 128) return hipErrorInvalidValue;
    if (attention_waves(S, nh) == 8) {
        const int nq = (S + QW * 8 - 1) / (QW * 8);
        hipLaunchKernelGGL((attn_bf16_pipe_kernel<8>), dim3(nq * nh), dim3(64 * 8), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)Vt, (bf16_t*)O, S, Sp, nh, c, o_amax);
    } else {
        const int nq = (S + QW * 4 - 1) / (QW * 4);
        hipLaunchKernelGGL((attn_bf16_pipe_kernel<4>), dim3(nq * nh), dim3(64 * 4), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)Vt, (bf16_t*)O, S, Sp, nh, c, o_amax);
    }
    return hipGetLastError();
}

hipError_t attention_f32(const void* Q, const void* K, const void* Vt, void* O, int S, int Sp, int nh, int dh,
                         float c, hipStream_t st) {
    const int nq = (S + 63) / 64;
    if (dh == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(nq * nh), dim3(64), 0, st, (const float*)Q, (const float*)K,
                           (const float*)Vt, (float*)O, S, Sp, nh, c);
    else if (dh == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(nq * nh), dim3(64), 0, st, (const float*)Q, (const float*)K,
                           (const float*)Vt, (float*)O, S, Sp, nh, c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t attention_pack(bool bf16, const void* q, const void* k, const void* v, void* Qp, void* Kp, void* Vtp,
                          int S, int Sp, int nh, int dh, float qscale, hipStream_t st) {
    const size_t total = (size_t)Sp * nh * dh;
    const int blocks = (int)((total + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL(attn_pack_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)q,
                           (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)Qp, (bf16_t*)Kp, (bf16_t*)Vtp, S, Sp, nh,
                           dh, qscale);
    else
        hipLaunchKernelGGL(attn_pack_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)q,
                           (const float*)k, (const float*)v, (float*)Qp, (float*)Kp, (float*)Vtp, S, Sp, nh, dh,
                           qscale);
    return hipGetLastError();
}

}  // namespace dit
