// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <algorithm>

#include "common.h"

namespace dit {

struct EpiParams;

hipError_t keep_index_launch(int T, int H, int W, int s, int Hk, int Wk, int32_t* keep, hipStream_t st);
hipError_t nearest_map_launch(int T, int H, int W, int s, int Hk, int Wk, int32_t* nk, hipStream_t st);
hipError_t rope_tables_launch(float2* tab, int n_t, int rt, int n_h, int rh, int n_w, int rw, double base,
                              hipStream_t st);
// rows[m][i] = (cos, sin) of pair i of sequence row m (per-axis tables in r)
hipError_t rope_rows_launch(const Rope& r, float2* rows, int S, int npair, hipStream_t st);
hipError_t rmsnorm_launch(int act, bool seq_input, const SeqIn& seq, const float* dense, const void* g, void* out,
                          int M, int D, float eps, hipStream_t st);
hipError_t rmsnorm_fp8_launch(bool seq_input, const SeqIn& seq, const float* dense, const void* g, uint8_t* out,
                              float* rinv, float* amax, int M, int D, float eps, hipStream_t st);
hipError_t fill_launch(float* p, int n, float v, hipStream_t st);
hipError_t quant_launch(bool bf16, const void* src, uint8_t* dst, const float* amax, size_t n, hipStream_t st);
hipError_t amax_launch(bool bf16, const void* src, size_t n, float* amax, hipStream_t st);
hipError_t amax_to_scale_launch(float* p, hipStream_t st);
hipError_t gather_rows_launch(const void* x, const int32_t* idx, void* out, int n, size_t rowbytes, hipStream_t st);
hipError_t broadcast_residual_launch(bool bf16, const void* x, const void* delta, bool delta_bf16, const int32_t* nk,
                                     void* out, int n_video, int D, hipStream_t st);
hipError_t euler_launch(bool bf16, void* x, const void* v, size_t n, float dt, hipStream_t st);

hipError_t gemm_mfma(bool fp8, int mode, const void* A, const void* W0, const void* W1, int M, int N, int K,
                     const EpiParams& ep, hipStream_t st);
// upper bound of the fp32 partial-tile bytes gemm_mfma uses for a K-split
// tail of the RESID / DOWN modes (0: it never splits); it does not decrease
// with M, and the current device's compute-unit count enters it
size_t gemm_split_bytes_bound(int M, int N);
namespace detail {
// compute units of the current device (cached per device; 256 when it cannot be read)
int device_cus();
}  // namespace detail

// Bounded long-video history: the kept frames and their strides (at most 11)
struct HistPlan {
    int n;                 // frames kept
    int frame[11], stride[11], hk[11], wk[11];
    int start[12];         // first token of each kept frame; start[n] = token count
};
HistPlan history_plan(int n_hist, int H, int W);
hipError_t history_index_launch(const HistPlan& hp, int H, int W, int32_t* idx, hipStream_t st);
hipError_t gemm_f32(int mode, const void* A, const void* W0, const void* W1, int M, int N, int K, const EpiParams& ep,
                    hipStream_t st);

hipError_t attention_bf16(const void* Q, const void* K, const void* Vt, void* O, int S, int Sp, int nh, int dh,
                          float c, float* o_amax, hipStream_t st);
hipError_t attention_f32(const void* Q, const void* K, const void* Vt, void* O, int S, int Sp, int nh, int dh,
                         float c, hipStream_t st);
// record a HIP error for dit_last_hip_error (api.hip)
void set_last_hip(int e);
// dit_block_forward(_ctrl) once dims are validated, on workspace `ws` (api.hip)
int block_forward_impl(const dit_dims* dims, const void* x_text, const void* x_video, const void* x_ctrl,
                       const int32_t* ctrl_idx, int32_t n_ctrl_tok, const void* x_audio,
                       const dit_block_weights* weights, int32_t compress_on, const int32_t* keep, const int32_t* nk,
                       void* y_text, void* y_video, void* y_ctrl, void* y_audio, void* ws, size_t ws_bytes,
                       void* stream);

hipError_t attention_pack(bool bf16, const void* q, const void* k, const void* v, void* Qp, void* Kp, void* Vtp,
                          int S, int Sp, int nh, int dh, float qscale, hipStream_t st);

}  // namespace dit
