// Shared device/host helpers of the gfx950 Flash DiT library (internal).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdtflash.h"

#define DIT_DEV __device__ __forceinline__

typedef uint16_t bf16_t;                                    // raw bfloat16 bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;  // MFMA operand type
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

namespace dit {

// ----------------------------------------------------------------- bf16 / fp32
DIT_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair; the library's values are finite)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
DIT_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
DIT_DEV uint32_t pack_bf2(float a, float b) {
    const bf16x2_v v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// ----------------------------------------------------------------- fp8 e4m3
// fp32 -> OCP e4m3 code: nearest value, ties to even, saturating at +-448,
// sign kept. The code space is monotone in the magnitude: subnormal codes are
// rint(a * 2^9) (a < 2^-6) and a normal a in [2^e, 2^(e+1)) has code
// 8 (e + 6) + rint(a * 2^(3 - e)); both scalings are exact, so the only
// rounding is the round-half-even of v_rndne_f32, and a carry out of the
// mantissa moves to the next exponent by itself.
DIT_DEV uint32_t f32_to_e4m3(float x) {
    uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
    float a = fminf(fabsf(x), 448.f);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.f);
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
        float scaled = a * __uint_as_float((uint32_t)(127 + 3 - e) << 23);
        code = (uint32_t)(8 * (e + 6)) + (uint32_t)__builtin_rintf(scaled);
    }
    return s | code;
}

// ----------------------------------------------------------------- streaming loads
// 16 bytes read once (no reuse expected): the load carries the nontemporal
// hint, so the line does not displace reused data in the caches. On streaming
// kernels this raised the achieved HBM bandwidth by about 13 % (540p
// broadcast, 5.3 -> 6.1 TB/s).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
DIT_DEV uint4 ld_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ----------------------------------------------------------------- reductions
DIT_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
DIT_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Running max of non-negative floats (x >= 0: their bit patterns order as
// unsigned integers). The current value is read first and the atomic issued only when
// x exceeds it: the value only grows, so a stale read can only be smaller and
// costs a redundant atomic, never a lost maximum; thousands of workgroups
// updating one address otherwise queue on it.
DIT_DEV void atomic_max_nonneg(float* addr, float x) {
    const unsigned cur = __hip_atomic_load((unsigned int*)addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(x) > cur) atomicMax((unsigned int*)addr, __float_as_uint(x));
}

// ----------------------------------------------------------------- sequence layout
// The joint sequence is [text | video tokens | control | audio]. Video tokens
// are either every position of x_video (vidx == nullptr) or the rows listed in
// vidx; control tokens (nc of them, possibly none) likewise every position of
// the control frames or the rows listed in cidx.
struct SeqIn {
    const void* xt;
    const void* xv;
    const void* xc;
    const void* xa;
    const int32_t* vidx;   // video token j -> row of xv (nullptr: j)
    const int32_t* cidx;   // control token j -> row of xc (nullptr: j)
    int nt, nv, nc, na;
};

// Output rows of the block. With delta != nullptr the video rows are not
// written to yv: their update y_j - ref_j (fp32; ref_j the row of the
// reference sequence) either goes to delta[j], or, with bout set, straight to
// every video position p whose nearest kept slot is j: bout[p] = bx[p] +
// update (the nearest-kept broadcast with the full-resolution residual).
struct SeqOut {
    void* yt;
    void* yv;
    void* yc;
    void* ya;
    float* delta;
    const void* bx;        // full-resolution video input [T][H][W][D] of the broadcast
    void* bout;            // its output (may be bx itself)
};

// The compression's grid: kept slot j is (t, a, b) in raster order over
// [T][Hk][Wk]; along an axis of n the a-th kept index is min(a s, n - 1).
struct KeepGeom {
    int H, W, Hk, Wk, s;
};

// Positions r of an axis of length n (kept indices min(a s, n - 1), nk of
// them) whose nearest kept index (ties to the lower) is the a-th one: the
// interval [lo, hi]. Between kept k and k' the midpoint floor((k + k') / 2)
// still goes to k.
DIT_DEV void kept_preimage(int a, int n, int s, int nk, int& lo, int& hi) {
    const int k = min(a * s, n - 1);
    lo = a == 0 ? 0 : (min((a - 1) * s, n - 1) + k) / 2 + 1;
    hi = a == nk - 1 ? n - 1 : (k + min((a + 1) * s, n - 1)) / 2;
}

// Rotary geometry: per-token coordinates and fp32 (cos, sin) tables per band.
struct Rope {
    const float2* tab_t;   // [npos_t][rt/2]
    const float2* tab_h;   // [H][rh/2]
    const float2* tab_w;   // [W][rw/2]
    const int32_t* vpos;   // video token j -> flat position (nullptr: j)
    const int32_t* cpos;   // control token j -> flat position in the control grid (nullptr: j)
    const float2* rows;    // per sequence row: (cos, sin) of all head_dim / 2 pairs (MFMA epilogue)
    int rt, rh, rw;
    int H, W;
    int nt, nv, nc;        // text / video / control token counts in the sequence
    int toff;              // time offset of video and audio tokens (control frames before the target)
};

template <typename T>
DIT_DEV const T* seq_row(const SeqIn& s, int m, int D) {
    if (m < s.nt) return (const T*)s.xt + (size_t)m * D;
    m -= s.nt;
    if (m < s.nv) {
        int r = s.vidx ? s.vidx[m] : m;
        return (const T*)s.xv + (size_t)r * D;
    }
    m -= s.nv;
    if (m < s.nc) return (const T*)s.xc + (size_t)(s.cidx ? s.cidx[m] : m) * D;
    return (const T*)s.xa + (size_t)(m - s.nc) * D;
}

// coordinates (t, h, w) of sequence row m: text -> (0,0,0); video ->
// (t + toff, h, w); control frame k -> (k, h, w); audio j -> (j + toff, 0, 0)
DIT_DEV int3 rope_coords(const Rope& r, int m) {
    if (m < r.nt) return make_int3(0, 0, 0);
    m -= r.nt;
    const int hw = r.H * r.W;
    if (m < r.nv || m - r.nv < r.nc) {
        const bool video = m < r.nv;
        const int p = video ? (r.vpos ? r.vpos[m] : m) : (r.cpos ? r.cpos[m - r.nv] : m - r.nv);
        const int t = p / hw;
        const int rem = p - t * hw;
        const int h = rem / r.W;
        return make_int3(t + (video ? r.toff : 0), h, rem - h * r.W);
    }
    return make_int3(m - r.nv - r.nc + r.toff, 0, 0);
}

// (cos, sin) for head-local feature d (even member of its pair) at coords c
DIT_DEV float2 rope_cs(const Rope& r, int d, int3 c) {
    if (d < r.rt) return r.tab_t[c.x * (r.rt >> 1) + (d >> 1)];
    d -= r.rt;
    if (d < r.rh) return r.tab_h[c.y * (r.rh >> 1) + (d >> 1)];
    d -= r.rh;
    return r.tab_w[c.z * (r.rw >> 1) + (d >> 1)];
}

// Compile-time loop: f(integral_constant<int, i>) for i = 0 .. N-1, so that
// register arrays are only ever indexed by constants.
template <int N, int I = 0, class F>
DIT_DEV void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Workgroup barrier for LDS pipelines fed by memory -> LDS loads: waits for
// this wave's LDS instructions only (lgkmcnt 0). __syncthreads() would also
// wait for every load still in flight (vmcnt 0), draining the deeper stages of
// the pipeline; those loads are waited for explicitly, per stage, with
// s_waitcnt vmcnt(n) before the barrier. The empty asm statements keep the
// compiler from moving memory accesses across it.
DIT_DEV void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0), vmcnt / expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer resource over [p, p + bytes) (reads past the end return zero).
// The pieces go through readfirstlane so that the compiler keeps the
// descriptor in scalar registers (a vector-held descriptor would turn every
// buffer access into a waterfall loop).
DIT_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, n, 0x00020000);
}

// XCD-aware remap of a linear workgroup id: the hardware deals workgroups
// round-robin to the 8 XCDs; consecutive logical tiles should share an XCD
// (and its L2), so logical = (bid % 8) * (n / 8) + bid / 8 on the full part.
DIT_DEV int xcd_remap(int bid, int n) {
    int full = (n / 8) * 8;
    if (bid >= full) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

}  // namespace dit
