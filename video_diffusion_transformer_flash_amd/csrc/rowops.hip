// Bandwidth-bound row kernels of the Flash DiT block for gfx950: index maps of
// the spatial token compression, rotary tables, RMSNorm (+ e4m3 activation
// quantisation), kept-row gather, nearest-kept update broadcast with the
// full-resolution residual, Euler update, fp8 weight quantisation.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace detail {

// ----------------------------------------------------------------- compression index maps
// Kept indices along an axis of length n at stride s (PaperDaily review,
// section 2; tokendh.com article, training section): multiples of s plus the
// last index. Rank a -> index min(a*s, n-1). Nearest kept index to r (ties
// to the lower): the multiple L = floor(r/s)*s below r or the next kept index
// U = min(L + s, n - 1) above it.
DIT_DEV int kept_at(int a, int n, int s) { return min(a * s, n - 1); }
DIT_DEV int kept_rank(int k, int n, int s, int nk) { return k == n - 1 ? nk - 1 : k / s; }
DIT_DEV int nearest_kept(int r, int n, int s) {
    const int L = (r / s) * s;
    if (L == r) return r;
    const int U = min(L + s, n - 1);
    return (r - L <= U - r) ? L : U;
}

__global__ void keep_index_kernel(int T, int H, int W, int s, int Hk, int Wk, int32_t* keep) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= T * Hk * Wk) return;
    const int t = j / (Hk * Wk);
    const int r = j - t * Hk * Wk;
    const int a = r / Wk, b = r - (r / Wk) * Wk;
    keep[j] = t * H * W + kept_at(a, H, s) * W + kept_at(b, W, s);
}

__global__ void nearest_map_kernel(int T, int H, int W, int s, int Hk, int Wk, int32_t* nk) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= T * H * W) return;
    const int t = p / (H * W);
    const int r = p - t * H * W;
    const int h = r / W, w = r - (r / W) * W;
    const int rh = kept_rank(nearest_kept(h, H, s), H, s, Hk);
    const int rw = kept_rank(nearest_kept(w, W, s), W, s, Wk);
    nk[p] = t * Hk * Wk + rh * Wk + rw;
}

// Bounded long-video history (tokendh.com article, long-video section;
// PaperDaily review, section 3): token j of the history list -> flat position
// in the [n_hist, H, W] grid of the history latents; the kept frames, their
// strides and token ranges come from history_plan.
__global__ void history_index_kernel(HistPlan hp, int H, int W, int32_t* idx) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= hp.start[hp.n]) return;
    int e = 0;
    while (e + 1 < hp.n && j >= hp.start[e + 1]) ++e;
    const int r = j - hp.start[e];
    const int a = r / hp.wk[e], b = r - (r / hp.wk[e]) * hp.wk[e];
    idx[j] = hp.frame[e] * H * W + a * hp.stride[e] * W + b * hp.stride[e];
}

// ----------------------------------------------------------------- rotary tables
// (cos, sin) of pos * base^(-2i/width) in fp64, stored fp32; three bands back to back.
__global__ void rope_table_kernel(float2* tab, int n_t, int rt, int n_h, int rh, int n_w, int rw, double base) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int et = n_t * (rt / 2), eh = n_h * (rh / 2), ew = n_w * (rw / 2);
    if (e >= et + eh + ew) return;
    int pos, i, width;
    if (e < et) { pos = e / (rt / 2); i = e % (rt / 2); width = rt; }
    else if (e < et + eh) { int x = e - et; pos = x / (rh / 2); i = x % (rh / 2); width = rh; }
    else { int x = e - et - eh; pos = x / (rw / 2); i = x % (rw / 2); width = rw; }
    const double theta = pow(base, -2.0 * i / (double)width);
    const double ang = (double)pos * theta;
    tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

// Per sequence row m, the (cos, sin) of every pair of head-local features:
// rows[m][i] for pair i of band t, h or w at the row's coordinates (from the
// per-axis tables); text rows get position 0 on every axis (identity).
__global__ void rope_rows_kernel(Rope r, float2* rows, int S, int npair) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= S * npair) return;
    const int m = e / npair, i = e - m * npair;
    rows[e] = rope_cs(r, 2 * i, rope_coords(r, m));
}

// ----------------------------------------------------------------- RMSNorm
template <typename T> DIT_DEV void ld4(const T* p, float v[4]);
template <> DIT_DEV void ld4<float>(const float* p, float v[4]) {
    float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <> DIT_DEV void ld4<bf16_t>(const bf16_t* p, float v[4]) {
    uint2 x = *(const uint2*)p;
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
}
template <typename T> DIT_DEV void st4(T* p, const float v[4]);
template <> DIT_DEV void st4<float>(float* p, const float v[4]) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
template <> DIT_DEV void st4<bf16_t>(bf16_t* p, const float v[4]) {
    *(uint2*)p = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}

// One wave per row: n = x / sqrt(mean(x^2) + eps) * g. Input rows come from
// the joint-sequence segments (SEQ) or from a dense fp32 [M][D] tensor.
// MODE 0: write n (TO). MODE 1: only the row factor rinv[m] and the tensor's
// max |n| (atomic). MODE 2: write e4m3 codes of n * 448 / amax.
template <typename TI, typename TG, typename TO, bool SEQ, int MODE>
__global__ __launch_bounds__(256) void rmsnorm_kernel(SeqIn seq, const float* __restrict__ dense,
                                                      const TG* __restrict__ g, TO* __restrict__ out,
                                                      float* __restrict__ rinv, float* __restrict__ amax, int M,
                                                      int D, float eps) {
    // one wave per row; the stats pass (MODE 1) takes RPW rows per wave and
    // makes one atomic per workgroup (one per row serialised thousands of
    // atomics on the single amax word)
    constexpr int RPW = MODE == 1 ? 4 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float mx = 0.f;
    for (int i = 0; i < RPW; ++i) {
        const int m = (blockIdx.x * RPW + i) * 4 + wave;
        if (m >= M) break;
        const TI* x = SEQ ? seq_row<TI>(seq, m, D) : (const TI*)(dense + (size_t)m * D);
        float r;
        if (MODE == 2) {
            r = rinv[m];
        } else {
            float ss = 0.f;
            for (int c = lane * 4; c < D; c += 256) {
                float v[4];
                ld4<TI>(x + c, v);
                ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
            }
            ss = wave_sum(ss);
            r = 1.f / sqrtf(ss / (float)D + eps);
        }
        float qs = 1.f;
        if (MODE == 2) {
            const float a = *amax;
            qs = a > 0.f ? 448.f / a : 1.f;
        }
        for (int c = lane * 4; c < D; c += 256) {
            float v[4], gv[4];
            ld4<TI>(x + c, v);
            ld4<TG>(g + c, gv);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = v[k] * r * gv[k];
            if constexpr (MODE == 0) {
                st4<TO>(out + (size_t)m * D + c, v);
            } else if constexpr (MODE == 1) {
#pragma unroll
                for (int k = 0; k < 4; ++k) mx = fmaxf(mx, fabsf(v[k]));
            } else {
                uint32_t w = f32_to_e4m3(v[0] * qs) | (f32_to_e4m3(v[1] * qs) << 8) | (f32_to_e4m3(v[2] * qs) << 16) |
                             (f32_to_e4m3(v[3] * qs) << 24);
                *(uint32_t*)((uint8_t*)out + (size_t)m * D + c) = w;
            }
        }
        if (MODE == 1 && lane == 0) rinv[m] = r;
    }
    if constexpr (MODE == 1) {
        __shared__ float wmax[4];
        mx = wave_max(mx);
        if (lane == 0) wmax[wave] = mx;
        __syncthreads();
        if (threadIdx.x == 0) atomic_max_nonneg(amax, fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    }
}

// Single-pass form: one wave per row with the whole row in registers (up to
// NCM 16-byte chunks per lane: D <= 64 * NCM * 16 / sizeof(TI)); the row is
// read from memory once. MODE as above; MODE 2 still reads the row again,
// since the codes need the tensor's max, known only after every row.
template <int N, typename T> DIT_DEV void ldn(const T* p, float v[N]);
template <> DIT_DEV void ldn<4, float>(const float* p, float v[4]) { ld4<float>(p, v); }
template <> DIT_DEV void ldn<4, bf16_t>(const bf16_t* p, float v[4]) { ld4<bf16_t>(p, v); }
template <> DIT_DEV void ldn<8, bf16_t>(const bf16_t* p, float v[8]) {
    const uint4 x = *(const uint4*)p;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <> DIT_DEV void ldn<8, float>(const float* p, float v[8]) {
    ld4<float>(p, v);
    ld4<float>(p + 4, v + 4);
}
// 16 bytes of TI -> N = 16 / sizeof(TI) floats
template <typename TI> DIT_DEV void unpack16(const uint4& r, float* v);
template <> DIT_DEV void unpack16<bf16_t>(const uint4& r, float* v) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <> DIT_DEV void unpack16<float>(const uint4& r, float* v) {
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y); v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
}
template <int N, typename TO> DIT_DEV void stn(TO* p, const float* v);
template <> DIT_DEV void stn<4, float>(float* p, const float* v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
template <> DIT_DEV void stn<4, bf16_t>(bf16_t* p, const float* v) {
    *(uint2*)p = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}
template <> DIT_DEV void stn<8, bf16_t>(bf16_t* p, const float* v) {
    *(uint4*)p = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
}
DIT_DEV uint32_t e4m3x4(const float* v, float qs) {
    return f32_to_e4m3(v[0] * qs) | (f32_to_e4m3(v[1] * qs) << 8) | (f32_to_e4m3(v[2] * qs) << 16) |
           (f32_to_e4m3(v[3] * qs) << 24);
}
template <> DIT_DEV void stn<4, uint8_t>(uint8_t* p, const float* v) { *(uint32_t*)p = e4m3x4(v, 1.f); }
template <> DIT_DEV void stn<8, uint8_t>(uint8_t* p, const float* v) {
    *(uint2*)p = make_uint2(e4m3x4(v, 1.f), e4m3x4(v + 4, 1.f));
}

template <typename TI, typename TG, typename TO, bool SEQ, int MODE, int NCM>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(SeqIn seq, const float* __restrict__ dense,
                                                          const TG* __restrict__ g, TO* __restrict__ out,
                                                          float* __restrict__ rinv, float* __restrict__ amax, int M,
                                                          int D, float eps) {
    constexpr int EPC = 16 / sizeof(TI);   // elements per 16-byte chunk
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
    float mx = 0.f;
    if (m < M) {
        const TI* x = SEQ ? seq_row<TI>(seq, m, D) : (const TI*)(dense + (size_t)m * D);
        const int nch = D / EPC;
        uint4 r[NCM];
        // the statistics pass keeps its rows cacheable: the quantise pass reads them again
#pragma unroll
        for (int i = 0; i < NCM; ++i)
            if (lane + 64 * i < nch) r[i] = MODE == 1 ? ((const uint4*)x)[lane + 64 * i] : ld_stream((const uint4*)x + lane + 64 * i);
        float rr;
        if constexpr (MODE == 2) {
            rr = rinv[m];
        } else {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < NCM; ++i)
                if (lane + 64 * i < nch) {
                    float v[EPC];
                    unpack16<TI>(r[i], v);
#pragma unroll
                    for (int k = 0; k < EPC; ++k) ss = fmaf(v[k], v[k], ss);
                }
            ss = wave_sum(ss);
            rr = 1.f / sqrtf(ss / (float)D + eps);
        }
        float qs = 1.f;
        if constexpr (MODE == 2) {
            const float a = *amax;
            qs = a > 0.f ? 448.f / a : 1.f;
        }
#pragma unroll
        for (int i = 0; i < NCM; ++i) {
            const int c = lane + 64 * i;
            if (c < nch) {
                float v[EPC], gv[EPC];
                unpack16<TI>(r[i], v);
                ldn<EPC, TG>(g + c * EPC, gv);
#pragma unroll
                for (int k = 0; k < EPC; ++k) v[k] = v[k] * rr * gv[k];
                if constexpr (MODE == 0) {
                    stn<EPC, TO>(out + (size_t)m * D + c * EPC, v);
                } else if constexpr (MODE == 1) {
#pragma unroll
                    for (int k = 0; k < EPC; ++k) mx = fmaxf(mx, fabsf(v[k]));
                } else {
#pragma unroll
                    for (int k = 0; k < EPC; ++k) v[k] *= qs;
                    stn<EPC, uint8_t>((uint8_t*)out + (size_t)m * D + c * EPC, v);
                }
            }
        }
        if (MODE == 1 && lane == 0) rinv[m] = rr;
    }
    if constexpr (MODE == 1) {
        __shared__ float wmax[4];
        mx = wave_max(mx);
        if (lane == 0) wmax[wave] = mx;
        __syncthreads();
        if (threadIdx.x == 0) atomic_max_nonneg(amax, fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    }
}

// ----------------------------------------------------------------- quantisation
// e4m3 codes of src * 448 / amax for a bf16 / fp32 tensor (amax on the device)
template <typename T>
__global__ void quant_kernel(const T* __restrict__ src, uint8_t* __restrict__ dst, const float* __restrict__ amax,
                             size_t n4) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float a = *amax;
    const float qs = a > 0.f ? __fdiv_rn(448.f, a) : 1.f;
    float v[4];
    ld4<T>(src + 4 * i, v);
    uint32_t w = f32_to_e4m3(v[0] * qs) | (f32_to_e4m3(v[1] * qs) << 8) | (f32_to_e4m3(v[2] * qs) << 16) |
                 (f32_to_e4m3(v[3] * qs) << 24);
    ((uint32_t*)dst)[i] = w;
}

// the same codes for a bf16 tensor, 8 elements (one 16-byte streaming read, one
// 8-byte store) per thread
__global__ void quant8_bf16_kernel(const bf16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                   const float* __restrict__ amax, size_t n8) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const float a = *amax;
    const float qs = a > 0.f ? __fdiv_rn(448.f, a) : 1.f;
    float v[8];
    unpack16<bf16_t>(ld_stream((const uint4*)src + i), v);
    ((uint2*)dst)[i] = make_uint2(e4m3x4(v, qs), e4m3x4(v + 4, qs));
}

template <typename T>
__global__ void amax_kernel(const T* __restrict__ src, size_t n4, float* amax) {
    float mx = 0.f;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        float v[4];
        ld4<T>(src + 4 * i, v);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax, mx);
}

__global__ void fill_kernel(float* p, int n, float v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// scale = amax / 448 (amax 0 -> 1), in place
__global__ void amax_to_scale_kernel(float* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const float a = *p;
        *p = a > 0.f ? __fdiv_rn(a, 448.f) : 1.f;
    }
}

// ----------------------------------------------------------------- gather / broadcast
// out[j] = x[idx[j]], rows of `chunks` 16-byte chunks. A workgroup of 512
// threads copies two consecutive output rows, 256 threads each (the source
// row is then uniform per wave), up to four loads in flight per thread; the
// copy is written non-temporally (streaming loads were no faster here).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_v;
__global__ __launch_bounds__(512) void gather_rows_kernel(const uint8_t* __restrict__ x, const int32_t* __restrict__ idx,
                                                          uint8_t* __restrict__ out, int n, int chunks) {
    constexpr int U = 4;
    const int j = blockIdx.x * 2 + (threadIdx.x >> 8);
    if (j >= n) return;
    const int t = threadIdx.x & 255;
    const int src = __builtin_amdgcn_readfirstlane(idx[j]);
    const uint4* xr = (const uint4*)x + (size_t)src * chunks;
    u32x4_v* orow = (u32x4_v*)out + (size_t)j * chunks;
    for (int c0 = t; c0 < chunks; c0 += U * 256) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u * 256 < chunks) v[u] = xr[c0 + u * 256];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u * 256 < chunks) {
                const u32x4_v w = {v[u].x, v[u].y, v[u].z, v[u].w};
                __builtin_nontemporal_store(w, orow + c0 + u * 256);
            }
    }
}

// out[p] = x[p] + delta[nk[p]] (delta fp32 or bf16, the add in fp32). A
// workgroup of 512 threads takes two
// consecutive video positions, 256 threads each (the kept slot nk[p] is then
// uniform per wave), 8 elements per 16/32-byte access, up to four accesses in
// flight per thread; the output is written non-temporally (it is not read
// again by this block). Position pairs are dealt to XCDs in contiguous
// ranges: raster neighbours, which share their kept slot's delta row, then
// meet that row in the same L2.
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
template <typename T>
struct Chunk8;
template <>
struct Chunk8<bf16_t> {
    uint4 v;
    DIT_DEV void load(const bf16_t* p) { v = ld_stream(p); }
    DIT_DEV void add_store(bf16_t* p, float4 d0, float4 d1) const {
        uint4 o;
        o.x = pack_bf2(__uint_as_float(v.x << 16) + d0.x, __uint_as_float(v.x & 0xFFFF0000u) + d0.y);
        o.y = pack_bf2(__uint_as_float(v.y << 16) + d0.z, __uint_as_float(v.y & 0xFFFF0000u) + d0.w);
        o.z = pack_bf2(__uint_as_float(v.z << 16) + d1.x, __uint_as_float(v.z & 0xFFFF0000u) + d1.y);
        o.w = pack_bf2(__uint_as_float(v.w << 16) + d1.z, __uint_as_float(v.w & 0xFFFF0000u) + d1.w);
        const u32x4_v ov = {o.x, o.y, o.z, o.w};
        __builtin_nontemporal_store(ov, (u32x4_v*)p);
    }
};
template <>
struct Chunk8<float> {
    float4 a, b;
    DIT_DEV void load(const float* p) {
        const uint4 u = ld_stream(p), w = ld_stream(p + 4);
        a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
        b = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
    DIT_DEV void add_store(float* p, float4 d0, float4 d1) const {
        const f32x4_v u = {a.x + d0.x, a.y + d0.y, a.z + d0.z, a.w + d0.w};
        const f32x4_v v = {b.x + d1.x, b.y + d1.y, b.z + d1.z, b.w + d1.w};
        __builtin_nontemporal_store(u, (f32x4_v*)p);
        __builtin_nontemporal_store(v, (f32x4_v*)(p + 4));
    }
};

// eight update values from fp32 or bf16 rows
template <typename TD> DIT_DEV void load_d8(const TD* p, float4& d0, float4& d1);
template <> DIT_DEV void load_d8<float>(const float* p, float4& d0, float4& d1) {
    d0 = *(const float4*)p;
    d1 = *(const float4*)(p + 4);
}
template <> DIT_DEV void load_d8<bf16_t>(const bf16_t* p, float4& d0, float4& d1) {
    const uint4 v = *(const uint4*)p;
    d0 = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xFFFF0000u));
    d1 = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u), __uint_as_float(v.w << 16),
                     __uint_as_float(v.w & 0xFFFF0000u));
}

template <typename T, typename TD>
__global__ __launch_bounds__(512) void broadcast_residual_kernel(const T* x, const TD* __restrict__ delta,
                                                                 const int32_t* __restrict__ nk, T* out, int n_video,
                                                                 int D) {
    // x and out may be the same buffer: every element is read, then written, by one thread
    constexpr int U = 4;
    // p is wave-uniform, so the kept slot nk[p] comes through a scalar load,
    // and the x loads (which do not depend on it) go out before it arrives
    const int p = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, (n_video + 1) / 2) * 2 + (threadIdx.x >> 8));
    if (p >= n_video) return;
    const int per_row = D / 8;
    const T* xr = x + (size_t)p * D;
    T* orow = out + (size_t)p * D;
    Chunk8<T> xv[U];
    auto load_x = [&](int c0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u * 256 < per_row) xv[u].load(xr + 8 * (c0 + u * 256));
    };
    int c0 = threadIdx.x & 255;
    load_x(c0);
    const TD* dr = delta + (size_t)nk[p] * D;
    for (;;) {
        float4 d0[U], d1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 256;
            if (c < per_row) load_d8<TD>(dr + 8 * c, d0[u], d1[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 256;
            if (c < per_row) xv[u].add_store(orow + 8 * c, d0[u], d1[u]);
        }
        c0 += U * 256;
        if (c0 >= per_row) break;
        load_x(c0);
    }
}

// x += dt * v (4 elements per thread); v may be x itself (a stack without
// layers: the velocity is the state), so neither pointer is restrict
template <typename T>
__global__ void euler_kernel(T* x, const T* v, size_t n4, float dt) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float a[4], b[4];
    ld4<T>(x + 4 * i, a);
    ld4<T>(v + 4 * i, b);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += dt * b[k];
    st4<T>(x + 4 * i, a);
}

inline unsigned nblk(size_t n, unsigned b = 256) { return (unsigned)((n + b - 1) / b); }

}  // namespace detail
using namespace detail;

// The first frame at stride 1, the two most recent at stride 2, up to eight
// frames right before those at stride 4; older middle frames are dropped.
// A frame at stride s keeps rows and columns that are multiples of s.
HistPlan history_plan(int n_hist, int H, int W) {
    HistPlan hp{};
    auto add = [&](int f, int s) {
        hp.frame[hp.n] = f;
        hp.stride[hp.n] = s;
        hp.hk[hp.n] = (H + s - 1) / s;
        hp.wk[hp.n] = (W + s - 1) / s;
        hp.start[hp.n + 1] = hp.start[hp.n] + hp.hk[hp.n] * hp.wk[hp.n];
        ++hp.n;
    };
    if (n_hist <= 0) return hp;
    add(0, 1);
    const int recent0 = std::max(1, n_hist - 2);          // first of the (up to) two recent frames
    for (int f = std::max(1, recent0 - 8); f < recent0; ++f) add(f, 4);
    for (int f = recent0; f < n_hist; ++f) add(f, 2);
    return hp;
}

hipError_t history_index_launch(const HistPlan& hp, int H, int W, int32_t* idx, hipStream_t st) {
    const int n = hp.start[hp.n];
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(history_index_kernel, dim3(nblk(n)), dim3(256), 0, st, hp, H, W, idx);
    return hipGetLastError();
}

hipError_t keep_index_launch(int T, int H, int W, int s, int Hk, int Wk, int32_t* keep, hipStream_t st) {
    const int n = T * Hk * Wk;
    hipLaunchKernelGGL(keep_index_kernel, dim3(nblk(n)), dim3(256), 0, st, T, H, W, s, Hk, Wk, keep);
    return hipGetLastError();
}

hipError_t nearest_map_launch(int T, int H, int W, int s, int Hk, int Wk, int32_t* nk, hipStream_t st) {
    const int n = T * H * W;
    hipLaunchKernelGGL(nearest_map_kernel, dim3(nblk(n)), dim3(256), 0, st, T, H, W, s, Hk, Wk, nk);
    return hipGetLastError();
}

hipError_t rope_tables_launch(float2* tab, int n_t, int rt, int n_h, int rh, int n_w, int rw, double base,
                              hipStream_t st) {
    const int n = n_t * (rt / 2) + n_h * (rh / 2) + n_w * (rw / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(nblk(n)), dim3(256), 0, st, tab, n_t, rt, n_h, rh, n_w, rw, base);
    return hipGetLastError();
}

hipError_t rope_rows_launch(const Rope& r, float2* rows, int S, int npair, hipStream_t st) {
    hipLaunchKernelGGL(rope_rows_kernel, dim3(nblk((long)S * npair)), dim3(256), 0, st, r, rows, S, npair);
    return hipGetLastError();
}

// register-resident rows when they fit: D <= 6144 (12 chunks of 16 bytes per
// lane for bf16 rows, 24 for fp32 rows)
constexpr int DMAX_REG = 6144;

template <typename TI, typename TG, typename TO, bool SEQ, int MODE>
void rms_go(dim3 grid, dim3 gstat, hipStream_t st, const SeqIn& seq, const float* dense, const void* g, void* out,
            float* rinv, float* amax, int M, int D, float eps) {
    constexpr int NCM = DMAX_REG * (int)sizeof(TI) / 1024;
    if (D <= DMAX_REG)
        hipLaunchKernelGGL((rmsnorm_reg_kernel<TI, TG, TO, SEQ, MODE, NCM>), grid, dim3(256), 0, st, seq, dense,
                           (const TG*)g, (TO*)out, rinv, amax, M, D, eps);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<TI, TG, TO, SEQ, MODE>), MODE == 1 ? gstat : grid, dim3(256), 0, st, seq,
                           dense, (const TG*)g, (TO*)out, rinv, amax, M, D, eps);
}

hipError_t rmsnorm_launch(int act, bool seq_input, const SeqIn& seq, const float* dense, const void* g, void* out,
                          int M, int D, float eps, hipStream_t st) {
    const dim3 grid(nblk(M, 4)), gstat(nblk(M, 16));
    if (act == DIT_F32) {
        if (seq_input) rms_go<float, float, float, true, 0>(grid, gstat, st, seq, dense, g, out, nullptr, nullptr, M, D, eps);
        else rms_go<float, float, float, false, 0>(grid, gstat, st, seq, dense, g, out, nullptr, nullptr, M, D, eps);
    } else {
        if (seq_input) rms_go<bf16_t, bf16_t, bf16_t, true, 0>(grid, gstat, st, seq, dense, g, out, nullptr, nullptr, M, D, eps);
        else rms_go<float, bf16_t, bf16_t, false, 0>(grid, gstat, st, seq, dense, g, out, nullptr, nullptr, M, D, eps);
    }
    return hipGetLastError();
}

// bf16 activations, fp8 output: stats pass (rinv, amax) then quantise pass;
// *amax must hold 0 (or a lower bound of the result) on entry
hipError_t rmsnorm_fp8_launch(bool seq_input, const SeqIn& seq, const float* dense, const void* g, uint8_t* out,
                              float* rinv, float* amax, int M, int D, float eps, hipStream_t st) {
    const dim3 grid(nblk(M, 4)), gstat(nblk(M, 16));   // the two-pass fallback's stats pass: 4 rows per wave
    if (seq_input) {
        rms_go<bf16_t, bf16_t, uint8_t, true, 1>(grid, gstat, st, seq, dense, g, out, rinv, amax, M, D, eps);
        rms_go<bf16_t, bf16_t, uint8_t, true, 2>(grid, gstat, st, seq, dense, g, out, rinv, amax, M, D, eps);
    } else {
        rms_go<float, bf16_t, uint8_t, false, 1>(grid, gstat, st, seq, dense, g, out, rinv, amax, M, D, eps);
        rms_go<float, bf16_t, uint8_t, false, 2>(grid, gstat, st, seq, dense, g, out, rinv, amax, M, D, eps);
    }
    return hipGetLastError();
}

hipError_t fill_launch(float* p, int n, float v, hipStream_t st) {
    hipLaunchKernelGGL(fill_kernel, dim3(nblk(n)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t quant_launch(bool bf16, const void* src, uint8_t* dst, const float* amax, size_t n, hipStream_t st) {
    const size_t n4 = n / 4;
    if (bf16 && n % 8 == 0 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 7) == 0) {
        const size_t n8 = n / 8;
        hipLaunchKernelGGL(quant8_bf16_kernel, dim3(nblk(n8)), dim3(256), 0, st, (const bf16_t*)src, dst, amax, n8);
    } else if (bf16)
        hipLaunchKernelGGL(quant_kernel<bf16_t>, dim3(nblk(n4)), dim3(256), 0, st, (const bf16_t*)src, dst, amax, n4);
    else
        hipLaunchKernelGGL(quant_kernel<float>, dim3(nblk(n4)), dim3(256), 0, st, (const float*)src, dst, amax, n4);
    return hipGetLastError();
}

hipError_t amax_launch(bool bf16, const void* src, size_t n, float* amax, hipStream_t st) {
    const size_t n4 = n / 4;
    const unsigned blocks = (unsigned)std::min<size_t>(nblk(n4), 4096);
    if (bf16)
        hipLaunchKernelGGL(amax_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)src, n4, amax);
    else
        hipLaunchKernelGGL(amax_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)src, n4, amax);
    return hipGetLastError();
}

hipError_t amax_to_scale_launch(float* p, hipStream_t st) {
    hipLaunchKernelGGL(amax_to_scale_kernel, dim3(1), dim3(64), 0, st, p);
    return hipGetLastError();
}

hipError_t gather_rows_launch(const void* x, const int32_t* idx, void* out, int n, size_t rowbytes, hipStream_t st) {
    const int chunks = (int)(rowbytes / 16);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((n + 1) / 2), dim3(512), 0, st, (const uint8_t*)x, idx, (uint8_t*)out, n,
                       chunks);
    return hipGetLastError();
}

hipError_t broadcast_residual_launch(bool bf16, const void* x, const void* delta, bool delta_bf16, const int32_t* nk,
                                     void* out, int n_video, int D, hipStream_t st) {
    if (n_video == 0) return hipSuccess;
    const dim3 grid((n_video + 1) / 2), block(512);
    if (bf16 && delta_bf16)
        hipLaunchKernelGGL((broadcast_residual_kernel<bf16_t, bf16_t>), grid, block, 0, st, (const bf16_t*)x,
                           (const bf16_t*)delta, nk, (bf16_t*)out, n_video, D);
    else if (bf16)
        hipLaunchKernelGGL((broadcast_residual_kernel<bf16_t, float>), grid, block, 0, st, (const bf16_t*)x,
                           (const float*)delta, nk, (bf16_t*)out, n_video, D);
    else if (delta_bf16)
        hipLaunchKernelGGL((broadcast_residual_kernel<float, bf16_t>), grid, block, 0, st, (const float*)x,
                           (const bf16_t*)delta, nk, (float*)out, n_video, D);
    else
        hipLaunchKernelGGL((broadcast_residual_kernel<float, float>), grid, block, 0, st, (const float*)x,
                           (const float*)delta, nk, (float*)out, n_video, D);
    return hipGetLastError();
}

hipError_t euler_launch(bool bf16, void* x, const void* v, size_t n, float dt, hipStream_t st) {
    const size_t n4 = n / 4;
    if (bf16)
        hipLaunchKernelGGL(euler_kernel<bf16_t>, dim3(nblk(n4)), dim3(256), 0, st, (bf16_t*)x, (const bf16_t*)v, n4, dt);
    else
        hipLaunchKernelGGL(euler_kernel<float>, dim3(nblk(n4)), dim3(256), 0, st, (float*)x, (const float*)v, n4, dt);
    return hipGetLastError();
}

}  // namespace dit
