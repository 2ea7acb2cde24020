// C ABI of the gfx950 Flash DiT block library: validation, workspace plans,
// launch sequencing of one block and of the flow-matching stack.
//
// Block (tokendh.com article, backbone and training sections; PaperDaily
// review, section 2), one stream, no host synchronisation:
//   rmsnorm1 (reads the joint sequence through its three segments; with
//             compression the video rows are gathered through keep on read)
//   -> QKV GEMM (+ rotary embedding, head-major q/k, transposed v)
//   -> attention -> O GEMM (+ residual, fp32 h) -> rmsnorm2
//   -> gate/up GEMM (+ SwiGLU) -> down GEMM (+ residual; text/audio/video
//      rows to the outputs, or delta = y - X for kept video rows)
//   -> compressed only: broadcast of delta[nk[p]] onto every x_video[p].
// With fp8 weights every GEMM input is e4m3 with a per-tensor dynamic scale:
// the norm kernels quantise in a second pass after an amax pass, the
// attention and SwiGLU outputs are quantised by a separate pass.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

using namespace dit;

namespace {

thread_local int g_last_hip = 0;

// ------------------------------------------------------------------ tracing
// Process-global event trace for profiling: when enabled, a hipEvent is
// recorded on the call's stream before each kernel group and after the last
// one ("end"); durations are read back after the fact. Not thread-safe.
struct TraceState {
    int cap = 0;
    int n = 0;
    std::vector<hipEvent_t> ev;
    std::vector<const char*> name;
};
TraceState g_tr;

inline void trace(const char* name, hipStream_t st) {
    if (g_tr.n < g_tr.cap) {
        (void)hipEventRecord(g_tr.ev[g_tr.n], st);
        g_tr.name[g_tr.n] = name;
        ++g_tr.n;
    }
}
#define TR(name) trace(name, st)

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int keep_count(int n, int s) { return (n + s - 1) / s + (((n - 1) % s) != 0 ? 1 : 0); }

#define HIPCHK(expr)                           \
    do {                                       \
        hipError_t e_ = (expr);                \
        if (e_ != hipSuccess) {                \
            g_last_hip = (int)e_;              \
            return DIT_EHIP;                   \
        }                                      \
    } while (0)

int esize(int dt) { return dt == DIT_F32 ? 4 : (dt == DIT_BF16 ? 2 : 1); }



int validate_dims(const dit_dims* d) {
    if (!d) return DIT_EINVAL;
    if (d->T < 1 || d->H < 1 || d->W < 1 || d->n_text < 0 || d->n_audio < 0 || d->stride < 1) return DIT_EINVAL;
    if (d->d_model < 64 || d->d_model % 64 || d->d_ffn < 64 || d->d_ffn % 64 || d->n_heads < 1) return DIT_EINVAL;
    if (d->head_dim != 64 && d->head_dim != 128) return DIT_EUNSUPPORTED;
    if (d->rope_t < 0 || d->rope_h < 0 || d->rope_w < 0 || (d->rope_t | d->rope_h | d->rope_w) & 1) return DIT_EINVAL;
    if (d->rope_t + d->rope_h + d->rope_w != d->head_dim) return DIT_EINVAL;
    if (!(d->rope_base > 0.f) || !(d->eps >= 0.f)) return DIT_EINVAL;
    if (d->n_ctrl < 0 || d->ctrl_offset < 0 || (d->n_ctrl > 0 && d->ctrl_offset < 1)) return DIT_EINVAL;
    if (d->n_ctrl > (1 << 20) || d->ctrl_offset > (1 << 20)) return DIT_EINVAL;
    if (d->n_fixed < 0 || d->n_fixed > d->T) return DIT_EINVAL;
    const long long nv = (long long)d->T * d->H * d->W;
    const long long S = nv + (long long)d->n_ctrl * d->H * d->W + d->n_text + d->n_audio;
    if (S > (1LL << 30) || nv * d->d_model > (1LL << 40)) return DIT_EINVAL;
    const int a = d->act_dtype, w = d->w_dtype;
    const bool f32 = a == DIT_F32 && w == DIT_F32;
    const bool bf = a == DIT_BF16 && w == DIT_BF16;
    const bool f8 = a == DIT_BF16 && w == DIT_FP8_E4M3;
    if (!(f32 || bf || f8)) return DIT_EUNSUPPORTED;
    if (!f32) {
        const int I = d->n_heads * d->head_dim;
        if (d->head_dim != 128) return DIT_EUNSUPPORTED;
        if (d->d_model % 128 || I % 128 || d->d_ffn % 128) return DIT_EUNSUPPORTED;
        if (d->rope_t % 8 || d->rope_h % 8 || d->rope_w % 8) return DIT_EUNSUPPORTED;
        // the MFMA epilogues address a head's q / k rows and a tile's rows
        // through buffer descriptors with 32-bit byte offsets (a head holds
        // S x 256 bytes); 2^23 tokens is far past what one GPU's memory holds
        if (S > (1LL << 23)) return DIT_EUNSUPPORTED;
    }
    return DIT_OK;
}

// ------------------------------------------------------------------ workspace plan
struct Plan {
    int S, Sp, nv_seq;
    size_t tab, rrows, n, rinv, q, k, vt, o, o8, h, u, u8, delta, part, part_bytes, sc, total;
    int ntab_t;
};

Plan make_plan(const dit_dims& d, int nv_seq, bool delta, int nc) {
    Plan p{};
    const bool fp8 = d.w_dtype == DIT_FP8_E4M3;
    const size_t es = esize(d.act_dtype);
    const size_t D = d.d_model, I = (size_t)d.n_heads * d.head_dim, F = d.d_ffn;
    p.nv_seq = nv_seq;
    p.S = d.n_text + nv_seq + nc + d.n_audio;
    p.Sp = (p.S + 127) / 128 * 128;
    // time positions: video t + off, control k, audio j + off
    p.ntab_t = std::max(std::max(d.T + d.ctrl_offset, d.n_audio + d.ctrl_offset), std::max(d.n_ctrl, 1));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t ntab = (size_t)p.ntab_t * (d.rope_t / 2) + (size_t)d.H * (d.rope_h / 2) + (size_t)d.W * (d.rope_w / 2);
    p.tab = take(std::max<size_t>(ntab, 1) * sizeof(float2));
    p.rrows = d.act_dtype == DIT_F32 ? 0 : take((size_t)p.S * (d.head_dim / 2) * sizeof(float2));
    p.n = take((size_t)p.S * D * (fp8 ? 1 : es));
    p.rinv = take((size_t)p.S * 4);
    p.q = take((size_t)d.n_heads * p.Sp * d.head_dim * es);
    p.k = take((size_t)d.n_heads * p.Sp * d.head_dim * es);
    p.vt = take((size_t)d.n_heads * p.Sp * d.head_dim * es);
    p.o = take((size_t)p.S * I * es);
    p.o8 = fp8 ? take((size_t)p.S * I) : 0;
    p.h = take((size_t)p.S * D * 4);
    p.u = take((size_t)p.S * F * es);
    p.u8 = fp8 ? take((size_t)p.S * F) : 0;
    p.delta = delta ? take((size_t)nv_seq * D * 4) : 0;
    // fp32 partial tiles of the O and down projections' K-split tails (a bound
    // that grows with S, so a workspace sized for more tokens always suffices)
    p.part_bytes = d.act_dtype == DIT_F32 ? 0 : gemm_split_bytes_bound(p.S, (int)D);
    p.part = p.part_bytes ? take(p.part_bytes) : 0;
    p.sc = take(32 * sizeof(float));   // amax values [0..3], the down projection's sink [16..19]
    p.total = off;
    return p;
}

// ------------------------------------------------------------------ one block
// `in`: the joint sequence; `vpos`: flat positions of its video tokens
// (nullptr: raster); `out`: output segments (or delta); `refin`: rows the
// delta is taken against.
// rope_ready: the rotary tables and rows of this plan are already in the
// workspace (the previous block of a stack ran on the same plan)
int run_block(const dit_dims& d, const dit_block_weights& w, const SeqIn& in, const int32_t* vpos, const int32_t* cpos,
              const SeqOut& out,
              const SeqIn& refin, uint8_t* ws, const Plan& P, hipStream_t st, bool rope_ready = false) {
    const bool f32 = d.act_dtype == DIT_F32;
    const bool fp8 = d.w_dtype == DIT_FP8_E4M3;
    const int D = d.d_model, nh = d.n_heads, dh = d.head_dim, I = nh * dh, F = d.d_ffn;
    const int S = P.S, Sp = P.Sp;

    float2* tab = (float2*)(ws + P.tab);
    const int nt_pos = P.ntab_t;
    if (!rope_ready) {
        TR("rope_tables");
        HIPCHK(rope_tables_launch(tab, nt_pos, d.rope_t, d.H, d.rope_h, d.W, d.rope_w, (double)d.rope_base, st));
    }
    Rope rope{};
    rope.tab_t = tab;
    rope.tab_h = tab + (size_t)nt_pos * (d.rope_t / 2);
    rope.tab_w = rope.tab_h + (size_t)d.H * (d.rope_h / 2);
    rope.vpos = vpos;
    rope.cpos = cpos;
    rope.rt = d.rope_t; rope.rh = d.rope_h; rope.rw = d.rope_w;
    rope.H = d.H; rope.W = d.W;
    rope.nt = in.nt; rope.nv = in.nv; rope.nc = in.nc;
    rope.toff = d.ctrl_offset;
    if (d.act_dtype != DIT_F32) {
        if (!rope_ready) {
            TR("rope_rows");
            HIPCHK(rope_rows_launch(rope, (float2*)(ws + P.rrows), P.S, d.head_dim / 2, st));
        }
        rope.rows = (const float2*)(ws + P.rrows);
    }

    void* n = ws + P.n;
    float* rinv = (float*)(ws + P.rinv);
    void* q = ws + P.q;
    void* k = ws + P.k;
    void* vt = ws + P.vt;
    void* o = ws + P.o;
    uint8_t* o8 = fp8 ? ws + P.o8 : nullptr;
    float* h = (float*)(ws + P.h);
    void* u = ws + P.u;
    uint8_t* u8 = fp8 ? ws + P.u8 : nullptr;
    float* sc = (float*)(ws + P.sc);   // [0] n1 amax, [1] o amax, [2] n2 amax, [3] u amax; [16..19] the sink

    EpiParams ep{};
    ep.M = S; ep.Mpad = Sp; ep.D = D; ep.I = I; ep.F = F; ep.dh = dh;
    ep.q = q; ep.k = k; ep.vt = vt; ep.Sp = Sp;
    const float csoft = (float)(1.4426950408889634 / sqrt((double)dh));   // log2(e) / sqrt(dh)
    ep.rope = rope;
    ep.xin = in;
    ep.h = h;
    ep.u = u;
    ep.hres = h;
    ep.out = out;
    ep.refin = refin;
    ep.kg = KeepGeom{d.H, d.W, keep_count(d.H, d.stride), keep_count(d.W, d.stride), d.stride};
    ep.part = P.part_bytes ? (float*)(ws + P.part) : nullptr;
    ep.part_bytes = P.part_bytes;
    ep.sink = sc + 16;

    // 1-2. RMSNorm1 + QKV (+ rotary)
    if (fp8) {
        HIPCHK(fill_launch(sc, 4, 0.f, st));   // the four running maxima of this block, one launch
        TR("rmsnorm1");
        HIPCHK(rmsnorm_fp8_launch(true, in, nullptr, w.g1, (uint8_t*)n, rinv, sc + 0, S, D, d.eps, st));
        ep.amax_a = sc + 0; ep.s_w = w.s_wqkv;
        TR("gemm_qkv");
        HIPCHK(gemm_mfma(true, EPI_QKV, n, w.wqkv, nullptr, S, 3 * I, D, ep, st));
    } else {
        TR("rmsnorm1");
        HIPCHK(rmsnorm_launch(d.act_dtype, true, in, nullptr, w.g1, n, S, D, d.eps, st));
        TR("gemm_qkv");
        if (f32) HIPCHK(gemm_f32(EPI_QKV, n, w.wqkv, nullptr, S, 3 * I, D, ep, st));
        else HIPCHK(gemm_mfma(false, EPI_QKV, n, w.wqkv, nullptr, S, 3 * I, D, ep, st));
    }
    // 3. attention
    TR("attention");
    if (f32) {
        HIPCHK(attention_f32(q, k, vt, o, S, Sp, nh, dh, csoft, st));
    } else {
        HIPCHK(attention_bf16(q, k, vt, o, S, Sp, nh, dh, csoft, fp8 ? sc + 1 : nullptr, st));
    }
    // 4. O projection + residual -> h (fp32)
    if (fp8) {
        TR("quant_o");
        HIPCHK(quant_launch(true, o, o8, sc + 1, (size_t)S * I, st));
        ep.amax_a = sc + 1; ep.s_w = w.s_wo;
        TR("gemm_o");
        HIPCHK(gemm_mfma(true, EPI_RESID, o8, w.wo, nullptr, S, D, I, ep, st));
    } else if (f32) {
        TR("gemm_o");
        HIPCHK(gemm_f32(EPI_RESID, o, w.wo, nullptr, S, D, I, ep, st));
    } else {
        TR("gemm_o");
        HIPCHK(gemm_mfma(false, EPI_RESID, o, w.wo, nullptr, S, D, I, ep, st));
    }
    // 5-6. RMSNorm2 + gate/up (+ SwiGLU)
    if (fp8) {
        TR("rmsnorm2");
        HIPCHK(rmsnorm_fp8_launch(false, in, h, w.g2, (uint8_t*)n, rinv, sc + 2, S, D, d.eps, st));
        ep.amax_a = sc + 2; ep.s_w = w.s_wgate; ep.s_w2 = w.s_wup; ep.u_amax = sc + 3;
        TR("gemm_gate_up");
        HIPCHK(gemm_mfma(true, EPI_SWIGLU, n, w.wgate, w.wup, S, 2 * F, D, ep, st));
        ep.u_amax = nullptr;
    } else {
        TR("rmsnorm2");
        HIPCHK(rmsnorm_launch(d.act_dtype, false, in, h, w.g2, n, S, D, d.eps, st));
        TR("gemm_gate_up");
        if (f32) HIPCHK(gemm_f32(EPI_SWIGLU, n, w.wgate, w.wup, S, 2 * F, D, ep, st));
        else HIPCHK(gemm_mfma(false, EPI_SWIGLU, n, w.wgate, w.wup, S, 2 * F, D, ep, st));
    }
    // 7. down projection + residual -> outputs / delta
    if (fp8) {
        TR("quant_u");
        HIPCHK(quant_launch(true, u, u8, sc + 3, (size_t)S * F, st));
        ep.amax_a = sc + 3; ep.s_w = w.s_wdown; ep.s_w2 = nullptr;
        TR("gemm_down");
        HIPCHK(gemm_mfma(true, EPI_DOWN, u8, w.wdown, nullptr, S, D, F, ep, st));
    } else if (f32) {
        TR("gemm_down");
        HIPCHK(gemm_f32(EPI_DOWN, u, w.wdown, nullptr, S, D, F, ep, st));
    } else {
        TR("gemm_down");
        HIPCHK(gemm_mfma(false, EPI_DOWN, u, w.wdown, nullptr, S, D, F, ep, st));
    }
    return DIT_OK;
}

int check_weights(const dit_dims& d, const dit_block_weights* w) {
    if (!w) return DIT_EINVAL;
    const void* ps[] = {w->g1, w->wqkv, w->wo, w->g2, w->wgate, w->wup, w->wdown};
    for (const void* p : ps)
        if (!p || !aligned16(p)) return DIT_EINVAL;
    if (d.w_dtype == DIT_FP8_E4M3) {
        const float* ss[] = {w->s_wqkv, w->s_wo, w->s_wgate, w->s_wup, w->s_wdown};
        for (const float* s : ss)
            if (!s) return DIT_EINVAL;
    }
    return DIT_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* dit_status_str(int32_t s) {
    switch (s) {
        case DIT_OK: return "ok";
        case DIT_EINVAL: return "invalid argument";
        case DIT_EUNSUPPORTED: return "unsupported configuration";
        case DIT_EWORKSPACE: return "workspace too small";
        case DIT_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int32_t dit_last_hip_error(void) { return g_last_hip; }

int32_t dit_trace_enable(int32_t capacity) {
    if (capacity < 0) return DIT_EINVAL;
    for (hipEvent_t e : g_tr.ev) (void)hipEventDestroy(e);
    g_tr.ev.clear();
    g_tr.name.clear();
    g_tr.n = 0;
    g_tr.cap = 0;
    for (int i = 0; i < capacity; ++i) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            g_last_hip = (int)err;
            return DIT_EHIP;
        }
        g_tr.ev.push_back(e);
        g_tr.name.push_back("");
    }
    g_tr.cap = capacity;
    return DIT_OK;
}

int32_t dit_trace_count(void) { return g_tr.n; }

int32_t dit_trace_read(int32_t index, const char** name, float* ms) {
    if (index < 0 || index + 1 >= g_tr.n || !name || !ms) return DIT_EINVAL;
    *name = g_tr.name[index];
    HIPCHK(hipEventSynchronize(g_tr.ev[index + 1]));
    HIPCHK(hipEventElapsedTime(ms, g_tr.ev[index], g_tr.ev[index + 1]));
    return DIT_OK;
}

int32_t dit_keep_dims(int32_t H, int32_t W, int32_t stride, int32_t* Hk, int32_t* Wk) {
    if (H < 1 || W < 1 || stride < 1 || !Hk || !Wk) return DIT_EINVAL;
    *Hk = keep_count(H, stride);
    *Wk = keep_count(W, stride);
    return DIT_OK;
}

int32_t dit_keep_index(int32_t T, int32_t H, int32_t W, int32_t stride, int32_t* keep, void* stream) {
    if (T < 1 || H < 1 || W < 1 || stride < 1 || !keep || (long long)T * H * W > (1LL << 30)) return DIT_EINVAL;
    HIPCHK(keep_index_launch(T, H, W, stride, keep_count(H, stride), keep_count(W, stride), keep, (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_nearest_kept_map(int32_t T, int32_t H, int32_t W, int32_t stride, int32_t* nk, void* stream) {
    if (T < 1 || H < 1 || W < 1 || stride < 1 || !nk || (long long)T * H * W > (1LL << 30)) return DIT_EINVAL;
    HIPCHK(nearest_map_launch(T, H, W, stride, keep_count(H, stride), keep_count(W, stride), nk, (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_history_count(int32_t n_hist, int32_t H, int32_t W, int32_t* count) {
    if (n_hist < 0 || H < 1 || W < 1 || !count || (long long)(n_hist + 1) * H * W > (1LL << 30)) return DIT_EINVAL;
    const HistPlan hp = history_plan(n_hist, H, W);
    *count = hp.start[hp.n];
    return DIT_OK;
}

int32_t dit_history_index(int32_t n_hist, int32_t H, int32_t W, int32_t* idx, void* stream) {
    if (n_hist < 0 || H < 1 || W < 1 || (long long)(n_hist + 1) * H * W > (1LL << 30)) return DIT_EINVAL;
    const HistPlan hp = history_plan(n_hist, H, W);
    if (hp.start[hp.n] > 0 && !idx) return DIT_EINVAL;
    HIPCHK(history_index_launch(hp, H, W, idx, (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_block_workspace_size(const dit_dims* dims, int32_t compress_on, size_t* bytes) {
    int r = validate_dims(dims);
    if (r) return r;
    if (!bytes) return DIT_EINVAL;
    const int nv = dims->T * dims->H * dims->W;
    const int nk = dims->T * keep_count(dims->H, dims->stride) * keep_count(dims->W, dims->stride);
    // every control position (a listed subset needs no more)
    *bytes = make_plan(*dims, compress_on ? nk : nv, compress_on != 0, dims->n_ctrl * dims->H * dims->W).total;
    return DIT_OK;
}

}  // extern "C"

namespace dit {

void set_last_hip(int e) { g_last_hip = e; }

// dit_block_forward / dit_block_forward_ctrl after their dims check, on a
// caller-provided workspace (also used by the entry points of other files)
int block_forward_impl(const dit_dims* dims, const void* x_text, const void* x_video, const void* x_ctrl,
                       const int32_t* ctrl_idx, int32_t n_ctrl_tok, const void* x_audio,
                       const dit_block_weights* weights, int32_t compress_on, const int32_t* keep, const int32_t* nk,
                       void* y_text, void* y_video, void* y_ctrl, void* y_audio, void* ws, size_t ws_bytes,
                       void* stream) {
    const dit_dims& d = *dims;
    int r;
    if ((r = check_weights(d, weights))) return r;
    if (!x_video || !y_video || !aligned16(x_video) || !aligned16(y_video)) return DIT_EINVAL;
    if (d.n_text > 0 && (!x_text || !y_text || !aligned16(x_text) || !aligned16(y_text))) return DIT_EINVAL;
    if (d.n_audio > 0 && (!x_audio || !y_audio || !aligned16(x_audio) || !aligned16(y_audio))) return DIT_EINVAL;
    if (d.n_ctrl > 0 && (!x_ctrl || !y_ctrl || !aligned16(x_ctrl) || !aligned16(y_ctrl))) return DIT_EINVAL;
    if (ctrl_idx && (n_ctrl_tok < 1 || n_ctrl_tok > d.n_ctrl * d.H * d.W)) return DIT_EINVAL;
    if (compress_on && (!keep || !nk)) return DIT_EINVAL;
    if (!ws || ((uintptr_t)ws & 255)) return DIT_EINVAL;
    const int nv = d.T * d.H * d.W;
    const int nc = ctrl_idx ? n_ctrl_tok : d.n_ctrl * d.H * d.W;
    const int nkept = d.T * keep_count(d.H, d.stride) * keep_count(d.W, d.stride);
    const Plan P = make_plan(d, compress_on ? nkept : nv, compress_on != 0, nc);
    if (ws_bytes < P.total) return DIT_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* w8 = (uint8_t*)ws;

    SeqIn in{x_text,   x_video, x_ctrl, x_audio, compress_on ? keep : nullptr, ctrl_idx, d.n_text,
             compress_on ? nkept : nv, nc, d.n_audio};
    // compressed: the MFMA path adds each kept row's update onto its video
    // positions in the down projection's epilogue; the fp32 path writes the
    // updates and broadcasts them in a pass of its own
    const bool fused = compress_on && d.act_dtype != DIT_F32;
    SeqOut out{y_text, y_video, y_ctrl, y_audio, compress_on ? (float*)(w8 + P.delta) : nullptr,
               fused ? x_video : nullptr, fused ? y_video : nullptr};
    r = run_block(d, *weights, in, compress_on ? keep : nullptr, ctrl_idx, out, in, w8, P, st);
    if (r) return r;
    if (compress_on && !fused) {
        TR("broadcast_residual");
        HIPCHK(broadcast_residual_launch(false, x_video, w8 + P.delta, false, nk, y_video, nv, d.d_model, st));
    }
    TR("end");
    return DIT_OK;
}

}  // namespace dit

extern "C" {

int32_t dit_block_forward(const dit_dims* dims, const void* x_text, const void* x_video, const void* x_audio,
                          const dit_block_weights* weights, int32_t compress_on, const int32_t* keep,
                          const int32_t* nk, void* y_text, void* y_video, void* y_audio, void* ws, size_t ws_bytes,
                          void* stream) {
    int r = validate_dims(dims);
    if (r) return r;
    if (dims->n_ctrl != 0) return DIT_EINVAL;
    return block_forward_impl(dims, x_text, x_video, nullptr, nullptr, 0, x_audio, weights, compress_on, keep, nk, y_text,
                              y_video, nullptr, y_audio, ws, ws_bytes, stream);
}

int32_t dit_block_forward_ctrl(const dit_dims* dims, const void* x_text, const void* x_video, const void* x_ctrl,
                               const int32_t* ctrl_idx, int32_t n_ctrl_tok, const void* x_audio,
                               const dit_block_weights* weights, int32_t compress_on, const int32_t* keep,
                               const int32_t* nk, void* y_text, void* y_video, void* y_ctrl, void* y_audio, void* ws,
                               size_t ws_bytes, void* stream) {
    int r = validate_dims(dims);
    if (r) return r;
    if (dims->n_ctrl < 1) return DIT_EINVAL;
    return block_forward_impl(dims, x_text, x_video, x_ctrl, ctrl_idx, n_ctrl_tok, x_audio, weights, compress_on, keep,
                              nk, y_text, y_video, y_ctrl, y_audio, ws, ws_bytes, stream);
}

namespace {

// stack workspace with nc control tokens in the sequence: the full-resolution
// and the packed compressed state, then the larger of the two block plans
size_t stack_bytes(const dit_dims& d, int nc) {
    const size_t es = esize(d.act_dtype);
    const int nv = d.T * d.H * d.W;
    const int nkept = d.T * keep_count(d.H, d.stride) * keep_count(d.W, d.stride);
    const size_t Soff = (size_t)d.n_text + nv + nc + d.n_audio, Son = (size_t)d.n_text + nkept + nc + d.n_audio;
    const Plan Pf = make_plan(d, nv, false, nc), Pc = make_plan(d, nkept, true, nc);
    return align256(Soff * d.d_model * es) + align256(Son * d.d_model * es) + std::max(Pf.total, Pc.total);
}

}  // namespace

int32_t dit_stack_workspace_size(const dit_dims* dims, const uint8_t* compressed_host, int32_t n_layers,
                                 size_t* bytes) {
    int r = validate_dims(dims);
    if (r) return r;
    if (!bytes || n_layers < 0 || (n_layers > 0 && !compressed_host)) return DIT_EINVAL;
    // every control position (a listed subset needs no more)
    *bytes = stack_bytes(*dims, dims->n_ctrl * dims->H * dims->W);
    return DIT_OK;
}

namespace {

int stack_impl(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
               const uint8_t* compressed_host, int32_t n_evals, const float* t_video_host,
               const float* t_audio_host, const void* x_text, void* x_video, const void* x_ctrl,
               const int32_t* ctrl_idx, int32_t n_ctrl_tok, void* x_audio, const int32_t* keep, const int32_t* nk,
               void* ws, size_t ws_bytes, void* stream) {
    const dit_dims& d = *dims;
    int r;
    if (n_layers < 0 || n_evals < 0 || (n_layers > 0 && (!layers_host || !compressed_host))) return DIT_EINVAL;
    if (n_evals > 0 && !t_video_host) return DIT_EINVAL;
    bool any_c = false;
    for (int l = 0; l < n_layers; ++l) {
        if ((r = check_weights(d, &layers_host[l]))) return r;
        any_c |= compressed_host[l] != 0;
    }
    if (any_c && (!keep || !nk)) return DIT_EINVAL;
    if (!x_video || !aligned16(x_video)) return DIT_EINVAL;
    if (d.n_text > 0 && (!x_text || !aligned16(x_text))) return DIT_EINVAL;
    if (d.n_audio > 0 && (!x_audio || !aligned16(x_audio))) return DIT_EINVAL;
    if (d.n_ctrl > 0 && (!x_ctrl || !aligned16(x_ctrl))) return DIT_EINVAL;
    if (ctrl_idx && (n_ctrl_tok < 1 || n_ctrl_tok > d.n_ctrl * d.H * d.W)) return DIT_EINVAL;
    if (!ws || ((uintptr_t)ws & 255)) return DIT_EINVAL;
    // the workspace this call carves: its control tokens are the listed ones
    // when ctrl_idx is given (dit_stack_workspace_size covers every position)
    if (ws_bytes < stack_bytes(d, ctrl_idx ? n_ctrl_tok : d.n_ctrl * d.H * d.W)) return DIT_EWORKSPACE;
    if (n_evals == 0) return DIT_OK;

    hipStream_t st = (hipStream_t)stream;
    const size_t es = esize(d.act_dtype);
    const bool bf = d.act_dtype == DIT_BF16;
    const size_t D = d.d_model;
    const int nt = d.n_text, na = d.n_audio;
    const int nv = d.T * d.H * d.W;
    const int nc = ctrl_idx ? n_ctrl_tok : d.n_ctrl * d.H * d.W;
    const int nkept = d.T * keep_count(d.H, d.stride) * keep_count(d.W, d.stride);
    const size_t Soff = (size_t)nt + nv + nc + na, Son = (size_t)nt + nkept + nc + na;
    uint8_t* w8 = (uint8_t*)ws;
    uint8_t* Z = w8;
    uint8_t* Zc = Z + align256(Soff * D * es);
    uint8_t* bws = Zc + align256(Son * D * es);
    const Plan Pf = make_plan(d, nv, false, nc), Pc = make_plan(d, nkept, true, nc);
    float* delta = (float*)(bws + Pc.delta);

    // full-resolution state [text | video | control | audio] and the packed
    // compressed state [text | kept video | control | audio]
    void* Zt = Z;
    void* Zv = Z + (size_t)nt * D * es;
    void* Zk = Z + ((size_t)nt + nv) * D * es;
    void* Za = Z + ((size_t)nt + nv + nc) * D * es;
    void* Zct = Zc;
    void* Zcv = Zc + (size_t)nt * D * es;
    void* Zck = Zc + ((size_t)nt + nkept) * D * es;
    void* Zca = Zc + ((size_t)nt + nkept + nc) * D * es;
    const SeqIn state{Zt, Zv, Zk, Za, nullptr, nullptr, nt, nv, nc, na};

    // which plan's rotary tables and rows the block workspace holds (0: none,
    // 1: the full-resolution plan, 2: the compressed one); the two plans share
    // the workspace, so a change of plan rebuilds them
    int rope_plan = 0;
    for (int ev = 0; ev < n_evals; ++ev) {
        // current full-resolution state: the inputs for the first layer, Z after
        // (listed control tokens are read through ctrl_idx by the first layer, packed after it)
        SeqIn cur{x_text, x_video, x_ctrl, x_audio, nullptr, ctrl_idx, nt, nv, nc, na};
        int l = 0;
        while (l < n_layers) {
            if (!compressed_host[l]) {
                SeqOut out{Zt, Zv, Zk, Za, nullptr, nullptr, nullptr};
                if ((r = run_block(d, layers_host[l], cur, nullptr, ctrl_idx, out, cur, bws, Pf, st, rope_plan == 1)))
                    return r;
                rope_plan = 1;
                cur = state;
                ++l;
                continue;
            }
            int e = l;
            while (e < n_layers && compressed_host[e]) ++e;
            // span [l, e): gather on read at its start, broadcast the summed update at its end
            const SeqIn start{cur.xt, cur.xv, cur.xc, cur.xa, keep, cur.cidx, nt, nkept, nc, na};
            const SeqIn packed{Zct, Zcv, Zck, Zca, nullptr, nullptr, nt, nkept, nc, na};
            for (int i = l; i < e; ++i) {
                const SeqIn& in = (i == l) ? start : packed;
                // the span's last layer adds the summed update onto every
                // position of the full-resolution state (in its epilogue on
                // the MFMA path, in a pass of its own for fp32)
                SeqOut out = (i + 1 < e) ? SeqOut{Zct, Zcv, Zck, Zca, nullptr, nullptr, nullptr}
                                         : SeqOut{Zt, nullptr, Zk, Za, delta, bf ? cur.xv : nullptr, bf ? Zv : nullptr};
                if ((r = run_block(d, layers_host[i], in, keep, ctrl_idx, out, start, bws, Pc, st, rope_plan == 2)))
                    return r;
                rope_plan = 2;
            }
            if (!bf) {
                TR("broadcast_residual");
                HIPCHK(broadcast_residual_launch(false, cur.xv, delta, false, nk, Zv, nv, (int)D, st));
            }
            cur = state;
            l = e;
        }
        const float dtv = (float)((double)t_video_host[ev + 1] - (double)t_video_host[ev]);
        const float* ta = t_audio_host ? t_audio_host : t_video_host;
        const float dta = (float)((double)ta[ev + 1] - (double)ta[ev]);
        // velocity = the stack output (the state itself when there are no layers)
        const void* vv = n_layers ? (const void*)Zv : (const void*)x_video;
        const void* va = n_layers ? (const void*)Za : (const void*)x_audio;
        TR("euler");
        // the first n_fixed frames keep their state (their velocity is not applied)
        const size_t fixed = (size_t)d.n_fixed * d.H * d.W * D;
        if (fixed < (size_t)nv * D)
            HIPCHK(euler_launch(bf, (uint8_t*)x_video + fixed * es, (const uint8_t*)vv + fixed * es,
                                (size_t)nv * D - fixed, dtv, st));
        if (na > 0) HIPCHK(euler_launch(bf, x_audio, va, (size_t)na * D, dta, st));
    }
    TR("end");
    return DIT_OK;
}

}  // namespace

int32_t dit_stack_sample(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                         const uint8_t* compressed_host, int32_t n_evals, const float* t_video_host,
                         const float* t_audio_host, const void* x_text, void* x_video, void* x_audio,
                         const int32_t* keep, const int32_t* nk, void* ws, size_t ws_bytes, void* stream) {
    int r = validate_dims(dims);
    if (r) return r;
    if (dims->n_ctrl != 0) return DIT_EINVAL;
    return stack_impl(dims, layers_host, n_layers, compressed_host, n_evals, t_video_host, t_audio_host, x_text,
                      x_video, nullptr, nullptr, 0, x_audio, keep, nk, ws, ws_bytes, stream);
}

int32_t dit_stack_sample_ctrl(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                              const uint8_t* compressed_host, int32_t n_evals, const float* t_video_host,
                              const float* t_audio_host, const void* x_text, void* x_video, const void* x_ctrl,
                              const int32_t* ctrl_idx, int32_t n_ctrl_tok, void* x_audio, const int32_t* keep,
                              const int32_t* nk, void* ws, size_t ws_bytes, void* stream) {
    int r = validate_dims(dims);
    if (r) return r;
    if (dims->n_ctrl < 1) return DIT_EINVAL;
    return stack_impl(dims, layers_host, n_layers, compressed_host, n_evals, t_video_host, t_audio_host, x_text,
                      x_video, x_ctrl, ctrl_idx, n_ctrl_tok, x_audio, keep, nk, ws, ws_bytes, stream);
}

namespace {

// dims of chunk c >= 1 of a long video: the boundary frame held fixed, every
// earlier frame as control frames at the time offset n_hist
int chunk_hist(const dit_dims& d, int c) { return d.T + (c - 1) * (d.T - 1) - 1; }

dit_dims chunk_dims(const dit_dims& d, int c) {
    dit_dims e = d;
    if (c > 0) {
        e.n_ctrl = e.ctrl_offset = chunk_hist(d, c);
        e.n_fixed = 1;
    }
    return e;
}

int long_video_plan(const dit_dims* dims, const uint8_t* compressed_host, int32_t n_layers, int32_t n_chunks,
                    size_t* idx_bytes, size_t* stack_max) {
    int r = validate_dims(dims);
    if (r) return r;
    const dit_dims& d = *dims;
    if (d.n_ctrl != 0 || d.ctrl_offset != 0 || d.n_fixed != 0) return DIT_EINVAL;
    if (n_chunks < 1 || n_layers < 0 || (n_layers > 0 && !compressed_host)) return DIT_EINVAL;
    if (n_chunks > 1 && d.T < 2) return DIT_EINVAL;
    if ((long long)d.T + (long long)(n_chunks - 1) * (d.T - 1) > (1 << 20)) return DIT_EINVAL;
    size_t ib = 0, sm = stack_bytes(d, 0);
    for (int c = 1; c < n_chunks; ++c) {
        const dit_dims e = chunk_dims(d, c);
        if ((r = validate_dims(&e))) return r;
        int32_t cnt = 0;
        if ((r = dit_history_count(e.n_ctrl, d.H, d.W, &cnt))) return r;
        ib = std::max(ib, align256((size_t)cnt * sizeof(int32_t)));
        sm = std::max(sm, stack_bytes(e, cnt));
    }
    *idx_bytes = ib;
    *stack_max = sm;
    return DIT_OK;
}

}  // namespace

int32_t dit_long_video_workspace_size(const dit_dims* dims, const uint8_t* compressed_host, int32_t n_layers,
                                      int32_t n_chunks, size_t* bytes) {
    if (!bytes) return DIT_EINVAL;
    size_t ib = 0, sm = 0;
    int r = long_video_plan(dims, compressed_host, n_layers, n_chunks, &ib, &sm);
    if (r) return r;
    *bytes = ib + sm;
    return DIT_OK;
}

int32_t dit_long_video_sample(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                              const uint8_t* compressed_host, int32_t n_evals, const float* t_video_host,
                              const float* t_audio_host, const void* x_text, int32_t n_chunks, void* frames,
                              void* x_audio, const int32_t* keep, const int32_t* nk, void* ws, size_t ws_bytes,
                              void* stream) {
    size_t ib = 0, sm = 0;
    int r = long_video_plan(dims, compressed_host, n_layers, n_chunks, &ib, &sm);
    if (r) return r;
    if (!frames || !aligned16(frames) || !ws || ((uintptr_t)ws & 255)) return DIT_EINVAL;
    if (dims->n_audio > 0 && (!x_audio || !aligned16(x_audio))) return DIT_EINVAL;
    if (ws_bytes < ib + sm) return DIT_EWORKSPACE;
    const dit_dims& d = *dims;
    const size_t es = esize(d.act_dtype);
    const size_t frame = (size_t)d.H * d.W * d.d_model * es;
    const size_t aud = (size_t)d.n_audio * d.d_model * es;
    int32_t* idx = (int32_t*)ws;
    uint8_t* sws = (uint8_t*)ws + ib;
    uint8_t* f8 = (uint8_t*)frames;
    uint8_t* a8 = (uint8_t*)x_audio;
    // chunk 0: the first T frames on their own
    if ((r = stack_impl(dims, layers_host, n_layers, compressed_host, n_evals, t_video_host, t_audio_host, x_text,
                        f8, nullptr, nullptr, 0, a8, keep, nk, sws, sm, stream)))
        return r;
    for (int c = 1; c < n_chunks; ++c) {
        const dit_dims e = chunk_dims(d, c);
        const int n_hist = e.n_ctrl;
        int32_t cnt = 0;
        if ((r = dit_history_count(n_hist, d.H, d.W, &cnt))) return r;
        if ((r = dit_history_index(n_hist, d.H, d.W, idx, stream))) return r;
        // window [n_hist, n_hist + T): the last frame made so far, then the T - 1 new ones
        if ((r = stack_impl(&e, layers_host, n_layers, compressed_host, n_evals, t_video_host, t_audio_host, x_text,
                            f8 + (size_t)n_hist * frame, f8, idx, cnt, a8 ? a8 + (size_t)c * aud : nullptr, keep, nk,
                            sws, sm, stream)))
            return r;
    }
    return DIT_OK;
}

int32_t dit_quantize_fp8(const void* src, int32_t src_dtype, int64_t n, uint8_t* dst, float* scale, void* stream) {
    if (!src || !dst || !scale || n <= 0 || n % 4 || !aligned16(src) || ((uintptr_t)dst & 3)) return DIT_EINVAL;
    if (src_dtype != DIT_F32 && src_dtype != DIT_BF16) return DIT_EUNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    const bool bf = src_dtype == DIT_BF16;
    HIPCHK(fill_launch(scale, 1, 0.f, st));
    HIPCHK(amax_launch(bf, src, (size_t)n, scale, st));
    HIPCHK(quant_launch(bf, src, dst, scale, (size_t)n, st));
    HIPCHK(amax_to_scale_launch(scale, st));
    return DIT_OK;
}

int32_t dit_gather_kept(int32_t n_kept, int32_t D, int32_t dtype, const void* x_video, const int32_t* keep, void* out,
                        void* stream) {
    if (n_kept < 0 || D <= 0 || !x_video || !keep || !out || !aligned16(x_video) || !aligned16(out)) return DIT_EINVAL;
    if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EUNSUPPORTED;
    const size_t rowbytes = (size_t)D * esize(dtype);
    if (rowbytes % 16) return DIT_EINVAL;
    if (n_kept == 0) return DIT_OK;
    HIPCHK(gather_rows_launch(x_video, keep, out, n_kept, rowbytes, (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_broadcast_residual(int32_t n_video, int32_t n_kept, int32_t D, int32_t dtype, const void* x_video,
                               const void* delta, int32_t delta_dtype, const int32_t* nk, void* out, void* stream) {
    if (n_video < 0 || n_kept < 1 || D <= 0 || D % 8 || !x_video || !delta || !nk || !out) return DIT_EINVAL;
    if (!aligned16(x_video) || !aligned16(delta) || !aligned16(out)) return DIT_EINVAL;
    if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EUNSUPPORTED;
    if (delta_dtype != DIT_F32 && delta_dtype != DIT_BF16) return DIT_EUNSUPPORTED;
    if (n_video == 0) return DIT_OK;
    HIPCHK(broadcast_residual_launch(dtype == DIT_BF16, x_video, delta, delta_dtype == DIT_BF16, nk, out, n_video, D,
                                     (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_rmsnorm(int32_t M, int32_t D, int32_t in_dtype, int32_t out_dtype, const void* x, const void* g, float eps,
                    void* out, float* rinv, float* amax, void* stream) {
    if (M < 0 || D < 64 || D % 64 || !x || !g || !out || !aligned16(x) || !aligned16(g) || !aligned16(out)) return DIT_EINVAL;
    if (!(eps >= 0.f)) return DIT_EINVAL;
    const bool f32 = in_dtype == DIT_F32 && out_dtype == DIT_F32;
    const bool bf = (in_dtype == DIT_BF16 || in_dtype == DIT_F32) && out_dtype == DIT_BF16;
    const bool f8 = (in_dtype == DIT_BF16 || in_dtype == DIT_F32) && out_dtype == DIT_FP8_E4M3;
    if (!(f32 || bf || f8)) return DIT_EUNSUPPORTED;
    if (f8 && (!rinv || !amax || ((uintptr_t)rinv & 3) || ((uintptr_t)amax & 3))) return DIT_EINVAL;
    if (M == 0) return DIT_OK;
    hipStream_t st = (hipStream_t)stream;
    // rows of a bf16 tensor go through the sequence reader (one segment), fp32 rows through the dense one
    const bool seq = in_dtype == DIT_BF16 || f32;
    const SeqIn in{x, nullptr, nullptr, nullptr, nullptr, nullptr, M, 0, 0, 0};
    const float* dense = seq ? nullptr : (const float*)x;
    if (f8) {
        HIPCHK(fill_launch(amax, 1, 0.f, st));
        HIPCHK(rmsnorm_fp8_launch(seq, in, dense, g, (uint8_t*)out, rinv, amax, M, D, eps, st));
    } else {
        HIPCHK(rmsnorm_launch(f32 ? DIT_F32 : DIT_BF16, seq, in, dense, g, out, M, D, eps, st));
    }
    return DIT_OK;
}

int32_t dit_project_residual_workspace_size(int32_t M, int32_t N, int32_t K, int32_t a_dtype, size_t* bytes) {
    if (M < 0 || N < 128 || K < 128 || N % 128 || K % 128 || !bytes) return DIT_EINVAL;
    if (a_dtype != DIT_BF16 && a_dtype != DIT_FP8_E4M3) return DIT_EUNSUPPORTED;
    *bytes = std::max<size_t>(256, gemm_split_bytes_bound(M, N));
    return DIT_OK;
}

int32_t dit_project_residual(int32_t M, int32_t N, int32_t K, int32_t a_dtype, const void* x_res, const void* a,
                             const float* a_amax, const void* w, const float* w_scale, float* h, void* ws,
                             size_t ws_bytes, void* stream) {
    size_t need = 0;
    int r = dit_project_residual_workspace_size(M, N, K, a_dtype, &need);
    if (r) return r;
    const bool fp8 = a_dtype == DIT_FP8_E4M3;
    if (!x_res || !a || !w || !h || !aligned16(x_res) || !aligned16(a) || !aligned16(w) || !aligned16(h)) return DIT_EINVAL;
    if (fp8 && (!a_amax || !w_scale)) return DIT_EINVAL;
    if (!ws || ((uintptr_t)ws & 255)) return DIT_EINVAL;
    if (ws_bytes < need) return DIT_EWORKSPACE;
    if (M == 0) return DIT_OK;
    EpiParams ep{};
    ep.M = M; ep.Mpad = M; ep.D = N; ep.I = K; ep.F = K; ep.dh = 128;
    ep.xin = SeqIn{x_res, nullptr, nullptr, nullptr, nullptr, nullptr, M, 0, 0, 0};
    ep.h = h;
    ep.amax_a = fp8 ? a_amax : nullptr;
    ep.s_w = fp8 ? w_scale : nullptr;
    ep.part = (float*)ws;
    ep.part_bytes = gemm_split_bytes_bound(M, N);
    HIPCHK(gemm_mfma(fp8, EPI_RESID, a, w, nullptr, M, N, K, ep, (hipStream_t)stream));
    return DIT_OK;
}

int32_t dit_attention_workspace_size(int32_t S, int32_t n_heads, int32_t head_dim, int32_t dtype, size_t* bytes) {
    if (S < 1 || n_heads < 1 || !bytes) return DIT_EINVAL;
    if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EUNSUPPORTED;
    if (head_dim != 128 && !(dtype == DIT_F32 && head_dim == 64)) return DIT_EUNSUPPORTED;
    const size_t Sp = ((size_t)S + 127) / 128 * 128;
    *bytes = 3 * align256(Sp * n_heads * head_dim * esize(dtype));
    return DIT_OK;
}

int32_t dit_attention(int32_t S, int32_t n_heads, int32_t head_dim, int32_t dtype, float scale, const void* q,
                      const void* k, const void* v, void* o, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    int r = dit_attention_workspace_size(S, n_heads, head_dim, dtype, &need);
    if (r) return r;
    if (!q || !k || !v || !o || !ws || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        ((uintptr_t)ws & 255))
        return DIT_EINVAL;
    if (ws_bytes < need) return DIT_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int Sp = (S + 127) / 128 * 128;
    const size_t part = need / 3;
    uint8_t* w8 = (uint8_t*)ws;
    const float c = (float)((double)scale * 1.4426950408889634);
    HIPCHK(attention_pack(dtype == DIT_BF16, q, k, v, w8, w8 + part, w8 + 2 * part, S, Sp, n_heads, head_dim, 1.f, st));
    if (dtype == DIT_BF16) HIPCHK(attention_bf16(w8, w8 + part, w8 + 2 * part, o, S, Sp, n_heads, head_dim, c, nullptr, st));
    else HIPCHK(attention_f32(w8, w8 + part, w8 + 2 * part, o, S, Sp, n_heads, head_dim, c, st));
    return DIT_OK;
}

}  // extern "C"
