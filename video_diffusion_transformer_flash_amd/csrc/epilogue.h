// GEMM epilogues of the Flash DiT block (internal).
//
// Every projection GEMM computes acc[m][n] = sum_k A[m][k] W[n][k] with the
// token index m and the output feature n; the MFMA kernels hand the epilogue
// four consecutive features n0..n0+3 of one token (the lane-owned run of the
// 32x32 accumulator layout), the fp32 kernel does the same. The epilogues fuse
// what follows each projection in the block (PaperDaily review, section 2:
// norm, quantisation, rotary embedding and residual update are fused):
//   QKV   : rotary embedding on q and k (pairs (2i, 2i+1) of each band),
//           written head-major: q, k [head][Sp][dh], v transposed [head][dh][Sp];
//   RESID : h = X + acc in fp32 (attention output projection);
//   SWIGLU: u = silu(gate) * up in the activation dtype, with the running
//           max of the stored |u| for fp8 (quantised from there);
//   DOWN  : y = h + acc to the text / video / audio outputs, or for kept video
//           rows of a compressed block the update y - X_ref: in fp32 to a
//           buffer, or (MFMA kernels) added straight onto every video
//           position whose nearest kept slot is that row (the broadcast with
//           the full-resolution residual, fused).
#pragma once

#include <type_traits>

#include "common.h"

namespace dit {

enum EpiMode { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_DOWN = 3 };

struct EpiParams {
    int M;          // valid token rows
    int Mpad;       // QKV: token rows [M, Mpad) are written as zeros
    int D, I, F, dh;
    // fp8: acc *= (amax_a / 448) * (*s_w); both on the device. nullptr: no scaling
    const float* amax_a;
    const float* s_w;
    const float* s_w2;      // SWIGLU: scale of the up weights (gate uses s_w)
    // QKV
    void* q;
    void* k;
    void* vt;
    int Sp;
    Rope rope;
    // RESID
    SeqIn xin;
    float* h;
    // SWIGLU
    void* u;
    float* u_amax;          // nullptr: no max tracking
    // DOWN
    const float* hres;
    SeqOut out;
    SeqIn refin;            // reference rows for delta (video segment only)
    KeepGeom kg;            // the compression's grid (broadcast into out.bout)
    // DOWN: 16 writable bytes that nothing reads; the rows past M store
    // there, so the output stores need no branch (nullptr: they branch)
    void* sink;
    // RESID / DOWN: fp32 partial tiles of K-split tail tiles (nullptr or too
    // small: no split)
    float* part;
    size_t part_bytes;
};

template <typename T> DIT_DEV void store4(T* p, const float v[4]);
template <> DIT_DEV void store4<float>(float* p, const float v[4]) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
template <> DIT_DEV void store4<bf16_t>(bf16_t* p, const float v[4]) {
    *(uint2*)p = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}
template <typename T> DIT_DEV void load4(const T* p, float v[4]);
template <> DIT_DEV void load4<float>(const float* p, float v[4]) {
    float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <> DIT_DEV void load4<bf16_t>(const bf16_t* p, float v[4]) {
    uint2 x = *(const uint2*)p;
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
}
template <typename T> DIT_DEV T cvt_out(float v);
template <> DIT_DEV float cvt_out<float>(float v) { return v; }
template <> DIT_DEV bf16_t cvt_out<bf16_t>(float v) { return f2bf(v); }
// the value a store of type T keeps
template <typename T> DIT_DEV float stored(float v);
template <> DIT_DEV float stored<float>(float v) { return v; }
template <> DIT_DEV float stored<bf16_t>(float v) { return bf2f(f2bf(v)); }

DIT_DEV float epi_scale(const float* amax_a, const float* s_w) {
    if (!amax_a) return 1.f;
    float a = *amax_a;
    float sa = a > 0.f ? a / 448.f : 1.f;
    return sa * (*s_w);
}

// m: token row, n0: first of four consecutive output features (n0 % 4 == 0)
template <typename T>
DIT_DEV void epi_qkv(const EpiParams& p, int m, int n0, float v[4], float sc) {
    if (m >= p.Mpad) return;
    const int which = n0 / p.I;
    const int rem = n0 - which * p.I;
    const int head = rem / p.dh;
    const int d0 = rem - head * p.dh;
    if (m >= p.M) {
        v[0] = v[1] = v[2] = v[3] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sc;
        if (which < 2) {
            const int3 c = rope_coords(p.rope, m);
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                float2 cs = rope_cs(p.rope, d0 + j, c);
                float a = v[j], b = v[j + 1];
                v[j] = a * cs.x - b * cs.y;
                v[j + 1] = a * cs.y + b * cs.x;
            }
        }
    }
    if (which == 0) {
        store4<T>((T*)p.q + ((size_t)head * p.Sp + m) * p.dh + d0, v);
    } else if (which == 1) {
        store4<T>((T*)p.k + ((size_t)head * p.Sp + m) * p.dh + d0, v);
    } else {
        T* vt = (T*)p.vt + ((size_t)head * p.dh + d0) * p.Sp + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) vt[(size_t)i * p.Sp] = cvt_out<T>(v[i]);
    }
}

template <typename T>
DIT_DEV void epi_resid(const EpiParams& p, int m, int n0, float v[4], float sc) {
    if (m >= p.M) return;
    float x[4];
    load4<T>(seq_row<T>(p.xin, m, p.D) + n0, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] += v[i] * sc;
    store4<float>(p.h + (size_t)m * p.D + n0, x);
}

// gate / up for ffn features f0..f0+3
template <typename T>
DIT_DEV float epi_swiglu(const EpiParams& p, int m, int f0, const float g[4], const float up[4], float sg, float su) {
    if (m >= p.M) return 0.f;
    float o[4];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float z = g[i] * sg;
        o[i] = z / (1.f + __expf(-z)) * (up[i] * su);
    }
    store4<T>((T*)p.u + (size_t)m * p.F + f0, o);
    if (p.u_amax) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(stored<T>(o[i])));  // max of the stored values
    }
    return mx;
}

template <typename T>
DIT_DEV void epi_down(const EpiParams& p, int m, int n0, float v[4], float sc) {
    if (m >= p.M) return;
    float y[4];
    load4<float>(p.hres + (size_t)m * p.D + n0, y);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] += v[i] * sc;
    const SeqOut& o = p.out;
    const int nt = p.xin.nt, nv = p.xin.nv, nc = p.xin.nc;
    if (m < nt) {
        store4<T>((T*)o.yt + (size_t)m * p.D + n0, y);
    } else if (m < nt + nv) {
        const int j = m - nt;
        if (o.delta) {
            float x[4];
            load4<T>(seq_row<T>(p.refin, m, p.D) + n0, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] -= x[i];
            store4<float>(o.delta + (size_t)j * p.D + n0, y);
        } else {
            store4<T>((T*)o.yv + (size_t)j * p.D + n0, y);
        }
    } else if (m < nt + nv + nc) {
        store4<T>((T*)o.yc + (size_t)(m - nt - nv) * p.D + n0, y);
    } else {
        store4<T>((T*)o.ya + (size_t)(m - nt - nv - nc) * p.D + n0, y);
    }
}

// ---------------------------------------------------------------------------
// Row layout (MFMA kernels): the accumulators are staged through LDS and each
// lane then takes eight consecutive outputs n0 .. n0 + 7 (n0 % 8 == 0) of one
// token m, already scaled; every global access is 16 or 32 contiguous bytes.

template <typename T> DIT_DEV void store8(T* p, const float v[8]);
template <> DIT_DEV void store8<float>(float* p, const float v[8]) {
    ((float4*)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    ((float4*)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <> DIT_DEV void store8<bf16_t>(bf16_t* p, const float v[8]) {
    *(uint4*)p = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
}
template <typename T> DIT_DEV void load8(const T* p, float v[8]);
template <> DIT_DEV void load8<float>(const float* p, float v[8]) {
    const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> DIT_DEV void load8<bf16_t>(const bf16_t* p, float v[8]) {
    const uint4 x = *(const uint4*)p;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// load8 of rows read once (the full-resolution rows of the broadcast)
template <typename T> DIT_DEV void load8_stream(const T* p, float v[8]);
template <> DIT_DEV void load8_stream<float>(const float* p, float v[8]) {
    const uint4 a = ld_stream(p), b = ld_stream(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
}
template <> DIT_DEV void load8_stream<bf16_t>(const bf16_t* p, float v[8]) {
    const uint4 x = ld_stream(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <typename T>
DIT_DEV void epi8_resid(const EpiParams& p, int m, int n0, const float v[8]) {
    if (m >= p.M) return;
    float x[8];
    load8<T>(seq_row<T>(p.xin, m, p.D) + n0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += v[i];
    store8<float>(p.h + (size_t)m * p.D + n0, x);
}

// Source rows of N sequence rows m[i] (as seq_row) in two passes: every
// index lookup (vidx / cidx, clamped into range so that each load is valid
// whichever segment the row is in) is issued before any is used, so the
// lookups of all N rows cost one memory latency instead of one each.
template <typename T, int N>
DIT_DEV void seq_rows(const SeqIn& s, const int (&m)[N], int D, const T* (&out)[N]) {
    const int nt = s.nt, nv = s.nv, nc = s.nc;
    int vi[N], ci[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        vi[i] = (s.vidx && nv > 0) ? s.vidx[min(max(m[i] - nt, 0), nv - 1)] : m[i] - nt;
        ci[i] = (s.cidx && nc > 0) ? s.cidx[min(max(m[i] - nt - nv, 0), nc - 1)] : m[i] - nt - nv;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int r = m[i];
        out[i] = r < nt             ? (const T*)s.xt + (size_t)r * D
                 : r < nt + nv      ? (const T*)s.xv + (size_t)vi[i] * D
                 : r < nt + nv + nc ? (const T*)s.xc + (size_t)ci[i] * D
                                    : (const T*)s.xa + (size_t)(r - nt - nv - nc) * D;
    }
}

// u = silu(gate) * up for ffn features f0 .. f0 + 7; returns max |stored u|
template <typename T>
DIT_DEV float epi8_swiglu(const EpiParams& p, int m, int f0, const float g[8], const float up[8]) {
    if (m >= p.M) return 0.f;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = g[i] * __builtin_amdgcn_rcpf(1.f + __expf(-g[i])) * up[i];   // rcp: 1 ulp
    store8<T>((T*)p.u + (size_t)m * p.F + f0, o);
    float mx = 0.f;
    if (p.u_amax) {
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(stored<T>(o[i])));
    }
    return mx;
}

// the update d of kept slot j (eight outputs from n0) onto every video
// position whose nearest kept slot is j: bout[p] = bx[p] + d (a rectangle of
// at most 2 x 2 positions at stride 2; loads first, then stores)
template <typename T>
DIT_DEV void bcast8(const EpiParams& p, int j, int n0, const float d[8]) {
    const KeepGeom& g = p.kg;
    const int per = g.Hk * g.Wk;
    const int t = j / per, r = j - t * per, a = r / g.Wk, b = r - a * g.Wk;
    int h0, h1, w0, w1;
    kept_preimage(a, g.H, g.s, g.Hk, h0, h1);
    kept_preimage(b, g.W, g.s, g.Wk, w0, w1);
    const T* x = (const T*)p.out.bx;
    T* out = (T*)p.out.bout;
    const size_t base = (size_t)t * g.H * g.W;
    if (h1 - h0 <= 1 && w1 - w0 <= 1) {
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int h = h0 + (q >> 1), w = w0 + (q & 1);
            if (h <= h1 && w <= w1) load8_stream<T>(x + (base + (size_t)h * g.W + w) * p.D + n0, v[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int h = h0 + (q >> 1), w = w0 + (q & 1);
            if (h <= h1 && w <= w1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[q][i] += d[i];
                store8<T>(out + (base + (size_t)h * g.W + w) * p.D + n0, v[q]);
            }
        }
        return;
    }
    for (int h = h0; h <= h1; ++h)
        for (int w = w0; w <= w1; ++w) {
            const size_t off = (base + (size_t)h * g.W + w) * p.D + n0;
            float v[8];
            load8_stream<T>(x + off, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += d[i];
            store8<T>(out + off, v);
        }
}

template <typename T>
DIT_DEV void epi8_down(const EpiParams& p, int m, int n0, const float v[8]) {
    if (m >= p.M) return;
    float y[8];
    load8<float>(p.hres + (size_t)m * p.D + n0, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] += v[i];
    const SeqOut& o = p.out;
    const int nt = p.xin.nt, nv = p.xin.nv, nc = p.xin.nc;
    if (m < nt) {
        store8<T>((T*)o.yt + (size_t)m * p.D + n0, y);
    } else if (m < nt + nv) {
        const int j = m - nt;
        if (o.delta) {
            float x[8];
            load8<T>(seq_row<T>(p.refin, m, p.D) + n0, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] -= x[i];
            if (o.bout) bcast8<T>(p, j, n0, y);
            else store8<float>(o.delta + (size_t)j * p.D + n0, y);
        } else {
            store8<T>((T*)o.yv + (size_t)j * p.D + n0, y);
        }
    } else if (m < nt + nv + nc) {
        store8<T>((T*)o.yc + (size_t)(m - nt - nv) * p.D + n0, y);
    } else {
        store8<T>((T*)o.ya + (size_t)(m - nt - nv - nc) * p.D + n0, y);
    }
}

// The DOWN epilogue of one row in two parts, so that a round can issue the
// loads of all its rows before its first store (stores may alias the
// full-resolution rows, so the compiler keeps a later row's loads behind an
// earlier row's stores): down_issue loads the residual row and, for a kept
// video row with its update, the reference row and the full-resolution rows
// of the slot's rectangle when it is at most 2 x 2; down_finish adds and
// stores as epi8_down does (the same arithmetic, the same results). bf16 rows.
// down_issue_h loads the residual row only, down_issue_rest the others.
struct DownRow {
    float h[8];
    uint4 ref;
    uint4 bx[4];
};

DIT_DEV void down_issue_h(const EpiParams& p, int m, int n0, DownRow& d) {
    if (m < p.M) load8<float>(p.hres + (size_t)m * p.D + n0, d.h);
}

// the reference row and the rectangle's rows (after down_issue_h)
DIT_DEV void down_issue_rest(const EpiParams& p, int m, int n0, DownRow& d) {
    if (m >= p.M) return;
    const int nt = p.xin.nt;
    if (m < nt || m >= nt + p.xin.nv || !p.out.delta) return;
    d.ref = *(const uint4*)(seq_row<bf16_t>(p.refin, m, p.D) + n0);
    if (!p.out.bout) return;
    const KeepGeom& g = p.kg;
    const int j = m - nt, per = g.Hk * g.Wk;
    const int t = j / per, r = j - t * per, a = r / g.Wk, b = r - a * g.Wk;
    int h0, h1, w0, w1;
    kept_preimage(a, g.H, g.s, g.Hk, h0, h1);
    kept_preimage(b, g.W, g.s, g.Wk, w0, w1);
    if (h1 - h0 > 1 || w1 - w0 > 1) return;
    const bf16_t* x = (const bf16_t*)p.out.bx + n0;
    const size_t base = (size_t)t * g.H * g.W;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int h = h0 + (q >> 1), w = w0 + (q & 1);
        if (h <= h1 && w <= w1) d.bx[q] = ld_stream(x + (base + (size_t)h * g.W + w) * p.D);
    }
}

DIT_DEV void down_finish(const EpiParams& p, int m, int n0, const float v[8], const DownRow& d) {
    if (m >= p.M) return;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = d.h[i] + v[i];
    const SeqOut& o = p.out;
    const int nt = p.xin.nt, nv = p.xin.nv, nc = p.xin.nc;
    if (m < nt) {
        store8<bf16_t>((bf16_t*)o.yt + (size_t)m * p.D + n0, y);
    } else if (m < nt + nv) {
        const int j = m - nt;
        if (o.delta) {
            const uint32_t rw[4] = {d.ref.x, d.ref.y, d.ref.z, d.ref.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[2 * i] -= __uint_as_float(rw[i] << 16);
                y[2 * i + 1] -= __uint_as_float(rw[i] & 0xFFFF0000u);
            }
            if (!o.bout) {
                store8<float>(o.delta + (size_t)j * p.D + n0, y);
                return;
            }
            const KeepGeom& g = p.kg;
            const int per = g.Hk * g.Wk;
            const int t = j / per, r = j - t * per, a = r / g.Wk, b = r - a * g.Wk;
            int h0, h1, w0, w1;
            kept_preimage(a, g.H, g.s, g.Hk, h0, h1);
            kept_preimage(b, g.W, g.s, g.Wk, w0, w1);
            if (h1 - h0 > 1 || w1 - w0 > 1) {
                bcast8<bf16_t>(p, j, n0, y);
                return;
            }
            bf16_t* out = (bf16_t*)o.bout + n0;
            const size_t base = (size_t)t * g.H * g.W;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int h = h0 + (q >> 1), w = w0 + (q & 1);
                if (h <= h1 && w <= w1) {
                    const uint32_t xw[4] = {d.bx[q].x, d.bx[q].y, d.bx[q].z, d.bx[q].w};
                    float z[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        z[2 * i] = __uint_as_float(xw[i] << 16) + y[2 * i];
                        z[2 * i + 1] = __uint_as_float(xw[i] & 0xFFFF0000u) + y[2 * i + 1];
                    }
                    store8<bf16_t>(out + (base + (size_t)h * g.W + w) * p.D, z);
                }
            }
        } else {
            store8<bf16_t>((bf16_t*)o.yv + (size_t)j * p.D + n0, y);
        }
    } else if (m < nt + nv + nc) {
        store8<bf16_t>((bf16_t*)o.yc + (size_t)(m - nt - nv) * p.D + n0, y);
    } else {
        store8<bf16_t>((bf16_t*)o.ya + (size_t)(m - nt - nv - nc) * p.D + n0, y);
    }
}

// One 32x32 MFMA accumulator block of a lane: token m, features
// nb + 8 g + 4 h + {0..3} in registers 4 g .. 4 g + 3 (g = 0..3, h = lane / 32).
template <int MODE, typename T>
DIT_DEV void epi_block(const EpiParams& p, int m, int nb, int h, const f32x16& acc, float sc) {
    static_for<4>([&](auto g) {
        float v[4] = {acc[4 * g + 0], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        const int n0 = nb + 8 * g + 4 * h;
        if constexpr (MODE == EPI_QKV) epi_qkv<T>(p, m, n0, v, sc);
        else if constexpr (MODE == EPI_RESID) epi_resid<T>(p, m, n0, v, sc);
        else epi_down<T>(p, m, n0, v, sc);
    });
}

// SwiGLU: gate block and up block of the same ffn features fb + 8 g + 4 h + {0..3}
template <typename T>
DIT_DEV float epi_block_swiglu(const EpiParams& p, int m, int fb, int h, const f32x16& gacc, const f32x16& uacc,
                               float sg, float su) {
    float mx = 0.f;
    static_for<4>([&](auto g) {
        float gv[4] = {gacc[4 * g + 0], gacc[4 * g + 1], gacc[4 * g + 2], gacc[4 * g + 3]};
        float uv[4] = {uacc[4 * g + 0], uacc[4 * g + 1], uacc[4 * g + 2], uacc[4 * g + 3]};
        mx = fmaxf(mx, epi_swiglu<T>(p, m, fb + 8 * g + 4 * h, gv, uv, sg, su));
    });
    return mx;
}

}  // namespace dit
