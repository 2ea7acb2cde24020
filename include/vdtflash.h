/*
 * vdtflash.h - C ABI of the MI355X (gfx950) Flash DiT block library.
 *
 * One joint text + video + audio diffusion-transformer block of the Flash
 * model, with spatial token compression and its full-resolution residual,
 * and the few-step flow-matching sampler over a stack of such blocks.
 *
 * Sources (the pages this follows):
 *   [TDH-backbone] tokendh.com article on LynnReal-Omni, backbone section:
 *       one shared denoiser over text, video and audio tokens; width 5376,
 *       56 heads of 128, feed-forward width 14336; 3D rotary positions.
 *   [TDH-training] same article, training section: flow matching, separate
 *       video and audio noise clocks, Flash keeps 42 layers (2 full, 26 with
 *       2x spatial token subsampling that keeps boundary rows and columns,
 *       14 full) and 3 evaluations; dropped tokens take the update of the
 *       nearest kept token of the same frame.
 *   [PD-2] PaperDaily review (longzhangge.com), section 2 (Flash): per-frame
 *       subsampling of rows and columns keeping about a quarter of the
 *       positions plus the edge rows and columns, no temporal subsampling,
 *       text and audio never compressed; compressed layers compute updates
 *       for the kept positions and every missing position adds the update of
 *       the nearest kept position of its frame to the full features; low-bit
 *       projections with fused norm, quantisation, rotary embedding and
 *       residual update.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the name ends in _host. The caller
 *     owns every buffer; the library allocates nothing, keeps no pointer
 *     after returning and never synchronises the stream. `stream` is a
 *     hipStream_t (NULL = the default stream).
 *   - Row-major layouts. Token activations are [rows][d_model]; x_video is
 *     [T][H][W][d_model] (raster order of t, h, w). Weights are [out][in].
 *   - Every argument is validated on the host before any launch; on error
 *     nothing is enqueued and a negative dit_status is returned.
 *   - Device pointers must be 16-byte aligned.
 *   - Outputs may alias the corresponding inputs (y_video == x_video etc.).
 *   - Calls are stateless; two calls may run concurrently on different
 *     streams only if each has its own workspace.
 */
#ifndef VDTFLASH_H
#define VDTFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIT_OK = 0,
    DIT_EINVAL = -1,        /* bad pointer, size or dimension */
    DIT_EUNSUPPORTED = -2,  /* valid but not implemented (dtype combination, head_dim, ...) */
    DIT_EWORKSPACE = -3,    /* workspace smaller than the *_workspace_size query */
    DIT_EHIP = -4           /* a HIP launch failed; see dit_last_hip_error() */
} dit_status;

typedef enum {
    DIT_F32 = 0,            /* IEEE binary32 */
    DIT_BF16 = 1,           /* bfloat16 */
    DIT_FP8_E4M3 = 2        /* OCP e4m3 (finite max 448), weights only, per-tensor fp32 scale */
} dit_dtype;

/* Block and grid sizes. Supported combinations (act_dtype, w_dtype):
 * (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * Constraints: d_model % 64 == 0; d_ffn % 64 == 0; head_dim in {64, 128};
 * rope_t + rope_h + rope_w == head_dim, each even; T, H, W >= 1;
 * n_text, n_audio >= 0; stride >= 1; at most 2^30 tokens in the joint
 * sequence. The bf16 / fp8 paths also need d_model, n_heads * head_dim and
 * d_ffn multiples of 128, head_dim 128 and at most 2^23 tokens (their kernels
 * address one head's rows with 32-bit byte offsets), else DIT_EUNSUPPORTED. */
typedef struct {
    int32_t T, H, W;              /* latent video grid */
    int32_t n_text, n_audio;      /* text / audio tokens (never compressed) */
    int32_t d_model;              /* hidden width D */
    int32_t n_heads, head_dim;    /* attention inner width I = n_heads * head_dim */
    int32_t d_ffn;                /* SwiGLU width F */
    int32_t rope_t, rope_h, rope_w; /* rotary band widths inside a head, in this order */
    float rope_base;              /* rotary base (10000) */
    float eps;                    /* RMSNorm epsilon (1e-6) */
    int32_t stride;               /* compression stride (2 in the Flash layers; 1 keeps every token) */
    int32_t act_dtype;            /* dit_dtype of activations and gains */
    int32_t w_dtype;              /* dit_dtype of the projection weights */
    int32_t n_ctrl;               /* control frames on the video's H x W grid (0: none; *_ctrl calls only) */
    int32_t ctrl_offset;          /* target time minus control time, >= 1 with control frames */
    int32_t n_fixed;              /* leading video frames the samplers hold fixed: their Euler update is
                                     skipped, e.g. a long video's shared boundary frame (0..T; the block
                                     itself ignores it) */
} dit_dims;

/* One block's parameters (device pointers). Gains g1, g2 [D] have act_dtype;
 * wqkv [3I][D] (rows: q, then k, then v), wo [D][I], wgate [F][D], wup [F][D],
 * wdown [D][F] have w_dtype. For FP8_E4M3 weights each s_* points to the
 * tensor's fp32 dequantisation scale on the device (W ~= code * scale, as
 * written by dit_quantize_fp8); otherwise the s_* are ignored. */
typedef struct {
    const void *g1, *wqkv, *wo, *g2, *wgate, *wup, *wdown;
    const float *s_wqkv, *s_wo, *s_wgate, *s_wup, *s_wdown;
} dit_block_weights;

/* Kept rows and columns of one frame for a compression stride [PD-2],
 * [TDH-training]: K(n) = {r : r mod stride == 0} U {n - 1}, so
 * |K(n)| = ceil(n / stride) + ((n - 1) mod stride != 0). Host only.
 * Returns DIT_OK and writes *Hk, *Wk, or DIT_EINVAL for H, W, stride < 1. */
int32_t dit_keep_dims(int32_t H, int32_t W, int32_t stride, int32_t* Hk, int32_t* Wk);

/* keep[j] = flat video position t*H*W + h*W + w of kept slot j, for the kept
 * set K(H) x K(W) of every frame in raster order of (t, h, w) [PD-2].
 * keep: int32 [T * Hk * Wk], device. Time is never subsampled. */
int32_t dit_keep_index(int32_t T, int32_t H, int32_t W, int32_t stride, int32_t* keep, void* stream);

/* nk[p] = kept slot (index into keep) of (t, near_H(h), near_W(w)) for every
 * video position p = (t, h, w), where near_n(r) is the kept index nearest to r,
 * ties to the lower index [TDH-training], [PD-2]. nk: int32 [T * H * W], device. */
int32_t dit_nearest_kept_map(int32_t T, int32_t H, int32_t W, int32_t stride, int32_t* nk, void* stream);

/* Bounded long-video history [TDH-long] (tokendh.com article, long-video
 * section), [PD-3] (PaperDaily review, section 3): of the n_hist latent frames
 * generated so far (frame 0 the first), frame 0 stays at full spatial
 * resolution, the two most recent frames are sampled at stride 2 and up to
 * eight frames right before them at stride 4; middle frames beyond that are
 * dropped. A frame at stride s keeps the rows and columns that are multiples
 * of s, so the history never holds more than two full frames of tokens when H
 * and W are multiples of 4. dit_history_count writes the token count (host
 * only); dit_history_index writes idx[j] = flat position f*H*W + h*W + w of
 * history token j in the [n_hist][H][W] grid, frame by frame in raster order
 * (device, int32 [count]); use it as ctrl_idx with the history latents as
 * x_ctrl (n_ctrl = n_hist, ctrl_offset = n_hist for a chunk that follows). */
int32_t dit_history_count(int32_t n_hist, int32_t H, int32_t W, int32_t* count);
int32_t dit_history_index(int32_t n_hist, int32_t H, int32_t W, int32_t* idx, void* stream);

/* Workspace bytes for dit_block_forward with these dims (compress_on 0 / 1);
 * with control frames, for every control position (enough for any ctrl_idx). */
int32_t dit_block_workspace_size(const dit_dims* dims, int32_t compress_on, size_t* bytes);

/* One Flash DiT block [TDH-backbone], [TDH-training], [PD-2].
 * Joint sequence X = [x_text | video tokens | x_audio]; with compress_on the
 * video tokens are x_video[keep[j]] (original coordinates kept for the rotary
 * embedding), otherwise all of x_video in raster order.
 *   n1 = RMSNorm(X) g1; q, k, v = n1 Wqkv^T; rotary embedding on q, k
 *   (video: bands t, h, w; audio: t band at its index; text: none);
 *   o = softmax(q k^T / sqrt(head_dim)) v per head over the whole sequence;
 *   h = X + o Wo^T; y = h + (silu(n2 Wg^T) * (n2 Wu^T)) Wd^T, n2 = RMSNorm(h) g2.
 * Outputs: y_text, y_audio = the text and audio rows of y. Uncompressed:
 * y_video = video rows of y. Compressed: y_video[p] = x_video[p] + (y - X)
 * at slot nk[p], for all T*H*W positions.
 * x_text [n_text][D], x_video [T][H][W][D], x_audio [n_audio][D] and the
 * outputs have act_dtype; keep and nk (from the two calls above, same stride)
 * are required iff compress_on. ws: device workspace of at least the queried
 * size, 256-byte aligned. With FP8 weights, each projection input is
 * quantised to e4m3 with a per-tensor dynamic scale amax / 448 before the
 * product; attention and the residual stream stay bf16 / fp32. */
int32_t dit_block_forward(const dit_dims* dims,
                          const void* x_text, const void* x_video, const void* x_audio,
                          const dit_block_weights* weights, int32_t compress_on,
                          const int32_t* keep, const int32_t* nk,
                          void* y_text, void* y_video, void* y_audio,
                          void* ws, size_t ws_bytes, void* stream);

/* dit_block_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is a static array of the library, 128 MiB on every device the
 * library runs on, held until the process ends. Blocks whose workspace
 * (dit_block_workspace_size) exceeds 128 MiB are refused with
 * DIT_EWORKSPACE before any launch. Uses the current device's array; every
 * call on a GPU shares it, so calls that overlap on one GPU (other streams or
 * threads) race. Outputs as dit_block_forward; allocates nothing. */
int32_t dit_block_forward_noalloc(const dit_dims* dims, const void* x_text, const void* x_video, const void* x_audio,
                                  const dit_block_weights* weights, int32_t compress_on, const int32_t* keep,
                                  const int32_t* nk, void* y_text, void* y_video, void* y_audio, void* stream);

/* The same block with control frames [TDH-backbone] (a reference's time
 * coordinate sits a fixed positive constant before the target's), [PD-1]
 * (aligned control frames and targets keep a stable positive time offset).
 * x_ctrl [n_ctrl][H][W][D] (act_dtype) joins the sequence after the video
 * tokens: X = [x_text | video tokens | x_ctrl | x_audio]. Rotary coordinates:
 * control frame k uses (k, h, w); video tokens use (t + ctrl_offset, h, w) and
 * audio token j the t position j + ctrl_offset (every time position moves
 * together, which leaves the logits among video and audio unchanged). Control
 * tokens are never compressed; y_ctrl [n_ctrl][H][W][D] receives their rows of
 * y (may alias x_ctrl). With ctrl_idx (device int32 [n_ctrl_tok], flat
 * positions in the [n_ctrl][H][W] grid, e.g. from dit_history_index) only
 * those control tokens join the sequence, each with its own coordinates, and
 * y_ctrl receives n_ctrl_tok rows [n_ctrl_tok][D] in that order (then it must
 * not alias x_ctrl); ctrl_idx NULL: every position, n_ctrl_tok ignored.
 * Needs n_ctrl >= 1 and ctrl_offset >= 1; everything else as
 * dit_block_forward, whose dims must have n_ctrl == 0. */
int32_t dit_block_forward_ctrl(const dit_dims* dims,
                               const void* x_text, const void* x_video, const void* x_ctrl,
                               const int32_t* ctrl_idx, int32_t n_ctrl_tok, const void* x_audio,
                               const dit_block_weights* weights, int32_t compress_on,
                               const int32_t* keep, const int32_t* nk,
                               void* y_text, void* y_video, void* y_ctrl, void* y_audio,
                               void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for dit_stack_sample with these dims and layer flags. */
int32_t dit_stack_workspace_size(const dit_dims* dims, const uint8_t* compressed_host, int32_t n_layers,
                                 size_t* bytes);

/* Few-step flow-matching sampler over n_layers blocks [TDH-training], [PD-2].
 * For k = 0 .. n_evals-1: run the layers on [x_text | x_video | x_audio]
 * (layer l compressed iff compressed_host[l]; text re-fed unchanged each
 * evaluation), take the video and audio outputs as the velocity v and update
 *   x_video += (t_video[k+1] - t_video[k]) v_video,
 *   x_audio += (t_audio[k+1] - t_audio[k]) v_audio   (t_audio NULL: t_video).
 * x_video and x_audio are updated in place. A run of consecutive compressed
 * layers gathers the kept tokens once and broadcasts the summed update once,
 * which equals per-layer broadcasting (kept positions are their own nearest).
 * layers_host: host array of n_layers weight sets (device pointers inside).
 * t_video_host / t_audio_host: host arrays of n_evals + 1 clean times. */
int32_t dit_stack_sample(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                         const uint8_t* compressed_host, int32_t n_evals,
                         const float* t_video_host, const float* t_audio_host,
                         const void* x_text, void* x_video, void* x_audio,
                         const int32_t* keep, const int32_t* nk,
                         void* ws, size_t ws_bytes, void* stream);

/* The sampler with control frames (see dit_block_forward_ctrl): every layer
 * runs on [x_text | x_video | control tokens | x_audio], and the control
 * tokens (all of x_ctrl, or those at ctrl_idx) are re-fed unchanged each
 * evaluation, like text. dims must have n_ctrl >= 1. */
int32_t dit_stack_sample_ctrl(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                              const uint8_t* compressed_host, int32_t n_evals,
                              const float* t_video_host, const float* t_audio_host,
                              const void* x_text, void* x_video, const void* x_ctrl,
                              const int32_t* ctrl_idx, int32_t n_ctrl_tok, void* x_audio,
                              const int32_t* keep, const int32_t* nk,
                              void* ws, size_t ws_bytes, void* stream);

/* Chunk-by-chunk long video [TDH-long] (tokendh.com article, long-video
 * section), [PD-3] (PaperDaily review, section 3) on the chunk grid of dims
 * (T frames; dims.n_ctrl, ctrl_offset and n_fixed must be 0). frames
 * [T + (n_chunks - 1) (T - 1)][H][W][D] (act_dtype, device) holds on entry the
 * first chunk's T noise frames, then for each later chunk c its T - 1 new noise
 * frames; on return every frame is denoised. Chunk 0 is dit_stack_sample on
 * frames [0, T). Chunk c >= 1 runs dit_stack_sample_ctrl on the window
 * [n_hist, n_hist + T), n_hist = T + (c - 1)(T - 1) - 1: its first frame (the
 * last frame made so far) is held fixed (n_fixed = 1) and the bounded history
 * of frames [0, n_hist) (dit_history_index) joins as control tokens at time
 * offset n_hist. x_audio [n_chunks][n_audio][D]: one audio segment per chunk,
 * denoised in place. n_chunks >= 1; T >= 2 when n_chunks > 1. Layers,
 * schedules, keep and nk as dit_stack_sample. ws: device workspace of at least
 * dit_long_video_workspace_size bytes, 256-byte aligned (the history index list
 * and the largest chunk's stack workspace, sized for its history tokens). */
int32_t dit_long_video_workspace_size(const dit_dims* dims, const uint8_t* compressed_host, int32_t n_layers,
                                      int32_t n_chunks, size_t* bytes);
int32_t dit_long_video_sample(const dit_dims* dims, const dit_block_weights* layers_host, int32_t n_layers,
                              const uint8_t* compressed_host, int32_t n_evals,
                              const float* t_video_host, const float* t_audio_host,
                              const void* x_text, int32_t n_chunks, void* frames, void* x_audio,
                              const int32_t* keep, const int32_t* nk,
                              void* ws, size_t ws_bytes, void* stream);

/* Per-tensor e4m3 quantisation of a weight tensor [PD-2] (low-bit
 * projections): amax = max |src|, dst = e4m3(saturate(src * (448 / amax))) with
 * round-to-nearest-even, *scale = amax / 448 (fp32, device); amax 0 gives
 * scale 1 and zero codes. src has src_dtype (F32 or BF16), n elements; dst
 * uint8 [n]. Runs on the stream; *scale is valid when the stream reaches it. */
int32_t dit_quantize_fp8(const void* src, int32_t src_dtype, int64_t n, uint8_t* dst, float* scale, void* stream);

/* Row gather of the kept video tokens [PD-2]: out[j] = x_video[keep[j]],
 * rows of D elements of dtype (F32 or BF16). Coalesced, bandwidth bound. */
int32_t dit_gather_kept(int32_t n_kept, int32_t D, int32_t dtype, const void* x_video, const int32_t* keep,
                        void* out, void* stream);

/* Nearest-kept update broadcast with the full-resolution residual [PD-2],
 * [TDH-training]: out[p] = x_video[p] + delta[nk[p]] for p < n_video, rows of
 * D elements (the add in fp32, then the store's rounding); x_video / out have
 * dtype (F32 or BF16), delta [n_kept][D] has delta_dtype (F32 or BF16).
 * out may alias x_video. Bandwidth bound. (Inside dit_block_forward the MFMA
 * path adds the fp32 update in the down projection's epilogue instead.) */
int32_t dit_broadcast_residual(int32_t n_video, int32_t n_kept, int32_t D, int32_t dtype, const void* x_video,
                               const void* delta, int32_t delta_dtype, const int32_t* nk, void* out, void* stream);

/* Multi-head attention over a joint sequence, the block's attention step on
 * its own [TDH-backbone]: o = softmax(q k^T * scale) v per head, unmasked.
 * q, k, v, o are [S][n_heads * head_dim] of dtype (F32 or BF16); no rotary
 * embedding is applied here. ws: workspace of dit_attention_workspace_size. */
int32_t dit_attention_workspace_size(int32_t S, int32_t n_heads, int32_t head_dim, int32_t dtype, size_t* bytes);
int32_t dit_attention(int32_t S, int32_t n_heads, int32_t head_dim, int32_t dtype, float scale,
                      const void* q, const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                      void* stream);

/* The block's normalisation step on its own [PD-2] (the first and second
 * RMSNorm, with the e4m3 quantisation of the low-bit projections' inputs):
 * n[m] = x[m] / sqrt(mean(x[m]^2) + eps) * g for M rows of D elements.
 * x [M][D] has in_dtype (F32 or BF16), g [D] the activation dtype of the
 * combination. Combinations (in_dtype -> out_dtype):
 *   F32 -> F32 (g F32); BF16 -> BF16 and F32 -> BF16 (g BF16);
 *   BF16 -> FP8_E4M3 and F32 -> FP8_E4M3 (g BF16): out receives the e4m3
 *   codes (uint8 [M][D]) of n * (448 / amax) with amax = max |n| over the
 *   whole tensor (the per-tensor scale is amax / 448), round to nearest even,
 *   and the call also writes rinv [M] (fp32 row factors 1 / sqrt(mean + eps))
 *   and *amax (fp32, device; both required for FP8 only, ignored otherwise).
 * n is computed in fp32. D must be a multiple of 64. */
int32_t dit_rmsnorm(int32_t M, int32_t D, int32_t in_dtype, int32_t out_dtype, const void* x, const void* g, float eps,
                    void* out, float* rinv, float* amax, void* stream);

/* The attention output projection with its residual on its own [PD-2]
 * (low-bit projections, fused residual update):
 *   h[m][n] = x_res[m][n] + s * sum_k A[m][k] W[n][k]
 * A [M][K] and W [N][K] both have a_dtype: BF16 (s = 1) or FP8_E4M3 codes
 * (s = (*a_amax / 448) * (*w_scale), both fp32 on the device: A's codes are
 * those of A * 448 / amax, W ~= codes * w_scale). x_res [M][N] is bf16, h
 * [M][N] fp32. N and K multiples of 128. fp32 accumulation on the matrix
 * cores; when the output tiles fill the compute units a whole number of
 * times plus a remainder, the remainder tiles are split along K into slices
 * whose fp32 sums go to the workspace (ws, 256-byte aligned, at least the
 * queried size) and are added in a fixed order. */
int32_t dit_project_residual_workspace_size(int32_t M, int32_t N, int32_t K, int32_t a_dtype, size_t* bytes);
int32_t dit_project_residual(int32_t M, int32_t N, int32_t K, int32_t a_dtype, const void* x_res, const void* a,
                             const float* a_amax, const void* w, const float* w_scale, float* h, void* ws,
                             size_t ws_bytes, void* stream);

/* Profiling trace (process-global, not thread-safe). With capacity > 0 the
 * library records a hipEvent on the call's stream before each kernel group of
 * every later call (names: rope_tables, rmsnorm1, gemm_qkv, attention,
 * gemm_o, rmsnorm2, gemm_gate_up, gemm_down, broadcast_residual, euler,
 * quant_o, quant_u) and one named "end" after each call's last launch, up to
 * `capacity` records; capacity 0 turns tracing off. dit_trace_read(i) waits
 * for record i + 1 and returns the name of record i and the milliseconds from
 * record i to record i + 1. */
int32_t dit_trace_enable(int32_t capacity);
int32_t dit_trace_count(void);
int32_t dit_trace_read(int32_t index, const char** name, float* ms);

const char* dit_status_str(int32_t status);
/* HIP error code of the last failed launch in this process (0 if none). */
int32_t dit_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* VDTFLASH_H */
