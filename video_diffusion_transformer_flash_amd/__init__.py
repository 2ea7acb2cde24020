"""MI355X (gfx950) Flash DiT block: thin Python binding of libvdtflash.so.

Every call marshals torch tensors (device memory) and the current HIP stream
into the C ABI of include/vdtflash.h; all arithmetic runs in the library's
HIP kernels. Outputs and workspaces are allocated with torch (plumbing).
The binding refuses to run without the built library.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import DIT_BF16, DIT_F32, DIT_FP8_E4M3, BlockWeights, Dims, DitError, check  # noqa: F401

__all__ = ["Dims", "make_dims", "keep_dims", "keep_index", "nearest_kept_map", "block_workspace_size",
           "block_forward", "block_forward_noalloc", "stack_workspace_size", "stack_sample", "quantize_fp8",
           "gather_kept", "broadcast_residual", "attention", "rmsnorm", "project_residual", "history_index",
           "long_video_workspace_size", "long_video_sample", "trace_enable", "trace_records", "DitError"]

_ACT = {"f32": DIT_F32, "bf16": DIT_BF16, "fp8": DIT_BF16}
_WT = {"f32": DIT_F32, "bf16": DIT_BF16, "fp8": DIT_FP8_E4M3}
_TORCH = {DIT_F32: torch.float32, DIT_BF16: torch.bfloat16}


def lib():
    return _lib.load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_dims(cfg, stride: int = None) -> Dims:
    """Dims from a dit_synth.BlockDims-like object."""
    return Dims(T=cfg.T, H=cfg.H, W=cfg.W, n_text=cfg.n_text, n_audio=cfg.n_audio, d_model=cfg.d_model,
                n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ffn=cfg.d_ffn, rope_t=cfg.rope[0], rope_h=cfg.rope[1],
                rope_w=cfg.rope[2], rope_base=cfg.rope_base, eps=cfg.eps,
                stride=cfg.stride if stride is None else stride, act_dtype=_ACT[cfg.dtype], w_dtype=_WT[cfg.dtype],
                n_ctrl=getattr(cfg, "n_ctrl", 0), ctrl_offset=getattr(cfg, "ctrl_offset", 0),
                n_fixed=getattr(cfg, "n_fixed", 0))


def keep_dims(H: int, W: int, stride: int = 2):
    hk, wk = ctypes.c_int32(), ctypes.c_int32()
    check(lib().dit_keep_dims(H, W, stride, ctypes.byref(hk), ctypes.byref(wk)), "dit_keep_dims")
    return hk.value, wk.value


def keep_index(T: int, H: int, W: int, stride: int = 2, out=None):
    hk, wk = keep_dims(H, W, stride)
    if out is None:
        out = torch.empty(T * hk * wk, dtype=torch.int32, device="cuda")
    check(lib().dit_keep_index(T, H, W, stride, _ptr(out), _stream()), "dit_keep_index")
    return out


def nearest_kept_map(T: int, H: int, W: int, stride: int = 2, out=None):
    if out is None:
        out = torch.empty(T * H * W, dtype=torch.int32, device="cuda")
    check(lib().dit_nearest_kept_map(T, H, W, stride, _ptr(out), _stream()), "dit_nearest_kept_map")
    return out


def history_index(n_hist: int, H: int, W: int, out=None):
    """Token positions of the bounded long-video history (int32, device)."""
    n = ctypes.c_int32()
    check(lib().dit_history_count(n_hist, H, W, ctypes.byref(n)), "dit_history_count")
    if out is None:
        out = torch.empty(n.value, dtype=torch.int32, device="cuda")
    check(lib().dit_history_index(n_hist, H, W, _ptr(out), _stream()), "dit_history_index")
    return out


def block_workspace_size(dims: Dims, compress: bool) -> int:
    n = ctypes.c_size_t()
    check(lib().dit_block_workspace_size(ctypes.byref(dims), int(compress), ctypes.byref(n)),
          "dit_block_workspace_size")
    return n.value


def _weights_struct(w: dict, dims: Dims = None) -> BlockWeights:
    if dims is not None:
        _check_weights(w, dims)
    g = lambda k: _ptr(w.get(k))  # noqa: E731
    return BlockWeights(g("g1"), g("wqkv"), g("wo"), g("g2"), g("wgate"), g("wup"), g("wdown"), g("s_wqkv"),
                        g("s_wo"), g("s_wgate"), g("s_wup"), g("s_wdown"))


def _check_weights(w: dict, dims: Dims):
    """Host-side check of one block's weights against dims (the library takes
    plain pointers and cannot see a buffer's size or type): every tensor on
    the GPU, contiguous, of the dtype dims names and of its shape's size; e4m3
    weights with their scales. A mismatch would make the kernels read past
    the end of a buffer."""
    D, I, F = dims.d_model, dims.n_heads * dims.head_dim, dims.d_ffn
    wt = {DIT_F32: torch.float32, DIT_BF16: torch.bfloat16, DIT_FP8_E4M3: torch.uint8}[dims.w_dtype]
    want = {"g1": (_TORCH[dims.act_dtype], D), "g2": (_TORCH[dims.act_dtype], D), "wqkv": (wt, 3 * I * D),
            "wo": (wt, D * I), "wgate": (wt, F * D), "wup": (wt, F * D), "wdown": (wt, D * F)}
    if dims.w_dtype == DIT_FP8_E4M3:
        want.update({"s_" + k: (torch.float32, 1) for k in ("wqkv", "wo", "wgate", "wup", "wdown")})
    for k, (dt, n) in want.items():
        t = w.get(k)
        if t is None:
            raise DitError(f"block weights: {k} missing")
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.numel() != n:
            raise DitError(f"block weights: {k} must be a contiguous {dt} GPU tensor of {n} elements "
                           f"(got {t.dtype}, {t.numel()} elements, {t.device})")


def workspace(nbytes: int):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


def block_forward(dims: Dims, x_text, x_video, x_audio, weights: dict, compress: bool, keep=None, nk=None,
                  out=None, ws=None, x_ctrl=None, ctrl_idx=None):
    """One block; returns (y_text, y_video, y_audio), and y_ctrl as a fourth
    element when x_ctrl (control frames, dims.n_ctrl > 0) is given; with
    ctrl_idx (int32 positions in the control grid) only those control tokens
    join and y_ctrl is [len(ctrl_idx), D]. `out` may be the inputs themselves
    (in place)."""
    if out is None:
        out = (torch.empty_like(x_text), torch.empty_like(x_video), torch.empty_like(x_audio))
        if x_ctrl is not None:
            yc = (torch.empty_like(x_ctrl) if ctrl_idx is None else
                  torch.empty((ctrl_idx.numel(), x_ctrl.shape[-1]), dtype=x_ctrl.dtype, device=x_ctrl.device))
            out = out + (yc,)
    need = block_workspace_size(dims, compress)
    if ws is None:
        ws = workspace(need)
    w = _weights_struct(weights, dims)
    if x_ctrl is None:
        st = lib().dit_block_forward(ctypes.byref(dims), _ptr(x_text), _ptr(x_video), _ptr(x_audio), ctypes.byref(w),
                                     int(compress), _ptr(keep), _ptr(nk), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                     _ptr(ws), ws.numel(), _stream())
        check(st, "dit_block_forward")
    else:
        st = lib().dit_block_forward_ctrl(ctypes.byref(dims), _ptr(x_text), _ptr(x_video), _ptr(x_ctrl),
                                          _ptr(ctrl_idx), 0 if ctrl_idx is None else ctrl_idx.numel(),
                                          _ptr(x_audio), ctypes.byref(w), int(compress), _ptr(keep), _ptr(nk),
                                          _ptr(out[0]), _ptr(out[1]), _ptr(out[3]), _ptr(out[2]), _ptr(ws),
                                          ws.numel(), _stream())
        check(st, "dit_block_forward_ctrl")
    return out


def block_forward_noalloc(dims: Dims, x_text, x_video, x_audio, weights: dict, compress: bool, keep=None, nk=None,
                          out=None):
    """One block on the library's static per-device scratch (no workspace is
    allocated; calls that overlap on one GPU race); returns (y_text, y_video,
    y_audio)."""
    if out is None:
        out = (torch.empty_like(x_text), torch.empty_like(x_video), torch.empty_like(x_audio))
    w = _weights_struct(weights, dims)
    st = lib().dit_block_forward_noalloc(ctypes.byref(dims), _ptr(x_text), _ptr(x_video), _ptr(x_audio),
                                         ctypes.byref(w), int(compress), _ptr(keep), _ptr(nk), _ptr(out[0]),
                                         _ptr(out[1]), _ptr(out[2]), _stream())
    check(st, "dit_block_forward_noalloc")
    return out


def stack_workspace_size(dims: Dims, flags) -> int:
    fl = (ctypes.c_uint8 * len(flags))(*[int(f) for f in flags])
    n = ctypes.c_size_t()
    check(lib().dit_stack_workspace_size(ctypes.byref(dims), ctypes.cast(fl, ctypes.c_void_p), len(flags),
                                         ctypes.byref(n)), "dit_stack_workspace_size")
    return n.value


def stack_sample(dims: Dims, layers: list, flags, t_video, t_audio, x_text, x_video, x_audio, keep=None, nk=None,
                 ws=None, x_ctrl=None, ctrl_idx=None):
    """Flow-matching sampler; x_video and x_audio are updated in place
    (control frames x_ctrl, when given, are re-fed every evaluation)."""
    n = len(layers)
    arr = (BlockWeights * max(n, 1))(*[_weights_struct(w, dims) for w in layers])
    fl = (ctypes.c_uint8 * max(n, 1))(*[int(f) for f in flags])
    tv = (ctypes.c_float * len(t_video))(*[float(t) for t in t_video])
    ta = None if t_audio is None else (ctypes.c_float * len(t_audio))(*[float(t) for t in t_audio])
    if ws is None:
        ws = workspace(stack_workspace_size(dims, flags))
    tac = None if ta is None else ctypes.cast(ta, ctypes.c_void_p)
    if x_ctrl is None:
        st = lib().dit_stack_sample(ctypes.byref(dims), arr, n, ctypes.cast(fl, ctypes.c_void_p), len(t_video) - 1,
                                    ctypes.cast(tv, ctypes.c_void_p), tac, _ptr(x_text), _ptr(x_video),
                                    _ptr(x_audio), _ptr(keep), _ptr(nk), _ptr(ws), ws.numel(), _stream())
        check(st, "dit_stack_sample")
    else:
        st = lib().dit_stack_sample_ctrl(ctypes.byref(dims), arr, n, ctypes.cast(fl, ctypes.c_void_p),
                                         len(t_video) - 1, ctypes.cast(tv, ctypes.c_void_p), tac, _ptr(x_text),
                                         _ptr(x_video), _ptr(x_ctrl), _ptr(ctrl_idx),
                                         0 if ctrl_idx is None else ctrl_idx.numel(), _ptr(x_audio), _ptr(keep),
                                         _ptr(nk), _ptr(ws), ws.numel(), _stream())
        check(st, "dit_stack_sample_ctrl")
    return x_video, x_audio


def long_video_workspace_size(dims: Dims, flags, n_chunks: int) -> int:
    fl = (ctypes.c_uint8 * max(len(flags), 1))(*[int(f) for f in flags])
    n = ctypes.c_size_t()
    check(lib().dit_long_video_workspace_size(ctypes.byref(dims), ctypes.cast(fl, ctypes.c_void_p), len(flags),
                                              n_chunks, ctypes.byref(n)), "dit_long_video_workspace_size")
    return n.value


def long_video_sample(dims: Dims, layers: list, flags, t_video, t_audio, x_text, first_video, new_video, audio,
                      keep=None, nk=None, ws=None):
    """Chunk-by-chunk long video on the chunk grid of `dims` (T frames), one
    dit_long_video_sample call: the first chunk denoises first_video
    [T, H, W, D]; each later chunk denoises its block of new_video [T - 1, H,
    W, D] after the last frame made so far (held fixed), with the bounded
    history of every earlier frame as control tokens. audio: one [n_audio, D]
    tensor per chunk, denoised in place. Returns the frames
    [T + (chunks - 1)(T - 1), H, W, D]."""
    T, n_chunks = dims.T, 1 + len(new_video)
    assert len(audio) == n_chunks
    frames = torch.empty((T + len(new_video) * (T - 1),) + tuple(first_video.shape[1:]), dtype=first_video.dtype,
                         device=first_video.device)
    frames[:T].copy_(first_video)
    for c, noise in enumerate(new_video):
        frames[T + c * (T - 1):T + (c + 1) * (T - 1)].copy_(noise)
    aud = torch.stack(list(audio)) if dims.n_audio > 0 else None
    n = len(layers)
    arr = (BlockWeights * max(n, 1))(*[_weights_struct(w, dims) for w in layers])
    fl = (ctypes.c_uint8 * max(n, 1))(*[int(f) for f in flags])
    tv = (ctypes.c_float * len(t_video))(*[float(t) for t in t_video])
    ta = None if t_audio is None else (ctypes.c_float * len(t_audio))(*[float(t) for t in t_audio])
    if ws is None:
        ws = workspace(long_video_workspace_size(dims, flags, n_chunks))
    st = lib().dit_long_video_sample(ctypes.byref(dims), arr, n, ctypes.cast(fl, ctypes.c_void_p), len(t_video) - 1,
                                     ctypes.cast(tv, ctypes.c_void_p),
                                     None if ta is None else ctypes.cast(ta, ctypes.c_void_p), _ptr(x_text),
                                     n_chunks, _ptr(frames), _ptr(aud), _ptr(keep), _ptr(nk), _ptr(ws), ws.numel(),
                                     _stream())
    check(st, "dit_long_video_sample")
    if aud is not None:
        for a, out in zip(audio, aud):
            a.copy_(out)
    return frames


def quantize_fp8(src, codes=None, scale=None):
    """Per-tensor e4m3 quantisation; returns (uint8 codes, fp32 scale [1])."""
    dt = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16}[src.dtype]
    if codes is None:
        codes = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=src.device)
    check(lib().dit_quantize_fp8(_ptr(src), dt, src.numel(), _ptr(codes), _ptr(scale), _stream()), "dit_quantize_fp8")
    return codes, scale


def gather_kept(x_video, keep, out=None):
    D = x_video.shape[-1]
    dt = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16}[x_video.dtype]
    if out is None:
        out = torch.empty((keep.numel(), D), dtype=x_video.dtype, device=x_video.device)
    check(lib().dit_gather_kept(keep.numel(), D, dt, _ptr(x_video), _ptr(keep), _ptr(out), _stream()),
          "dit_gather_kept")
    return out


def broadcast_residual(x_video, delta, nk, out=None):
    """out[p] = x_video[p] + delta[nk[p]] (delta fp32 or bf16 rows)."""
    D = x_video.shape[-1]
    dt = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16}[x_video.dtype]
    ddt = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16}[delta.dtype]
    if out is None:
        out = torch.empty_like(x_video)
    check(lib().dit_broadcast_residual(nk.numel(), delta.shape[0], D, dt, _ptr(x_video), _ptr(delta), ddt, _ptr(nk),
                                       _ptr(out), _stream()), "dit_broadcast_residual")
    return out


def attention(q, k, v, n_heads: int, scale: float, out=None, ws=None):
    """q, k, v [S, n_heads * head_dim] -> softmax(q k^T * scale) v per head."""
    S, I = q.shape
    hd = I // n_heads
    dt = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16}[q.dtype]
    n = ctypes.c_size_t()
    check(lib().dit_attention_workspace_size(S, n_heads, hd, dt, ctypes.byref(n)), "dit_attention_workspace_size")
    if ws is None:
        ws = workspace(n.value)
    if out is None:
        out = torch.empty_like(q)
    check(lib().dit_attention(S, n_heads, hd, dt, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                              ws.numel(), _stream()), "dit_attention")
    return out


_DT = {torch.float32: DIT_F32, torch.bfloat16: DIT_BF16, torch.uint8: DIT_FP8_E4M3}


def rmsnorm(x, g, eps: float, out_dtype: str = "same"):
    """RMSNorm of the rows of x [M, D] with gains g [D]. out_dtype "same" /
    "bf16" / "fp8"; fp8 returns (codes uint8 [M, D], rinv [M], amax [1])."""
    M, D = x.shape
    odt = {"same": _DT[x.dtype], "bf16": DIT_BF16, "fp8": DIT_FP8_E4M3}[out_dtype]
    if odt == DIT_FP8_E4M3:
        out = torch.empty((M, D), dtype=torch.uint8, device=x.device)
        rinv = torch.empty(M, dtype=torch.float32, device=x.device)
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        out = torch.empty((M, D), dtype=_TORCH[odt], device=x.device)
        rinv = amax = None
    check(lib().dit_rmsnorm(M, D, _DT[x.dtype], odt, _ptr(x), _ptr(g), float(eps), _ptr(out), _ptr(rinv), _ptr(amax),
                            _stream()), "dit_rmsnorm")
    return (out, rinv, amax) if odt == DIT_FP8_E4M3 else out


def project_residual(x_res, a, w, a_amax=None, w_scale=None, out=None, ws=None):
    """h = x_res + s * a w^T in fp32 (a, w bf16, or uint8 e4m3 codes with
    device scales a_amax / 448 and w_scale)."""
    M, K = a.shape
    N = w.shape[0]
    dt = _DT[a.dtype]
    n = ctypes.c_size_t()
    check(lib().dit_project_residual_workspace_size(M, N, K, dt, ctypes.byref(n)),
          "dit_project_residual_workspace_size")
    if ws is None:
        ws = workspace(n.value)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    check(lib().dit_project_residual(M, N, K, dt, _ptr(x_res), _ptr(a), _ptr(a_amax), _ptr(w), _ptr(w_scale),
                                     _ptr(out), _ptr(ws), ws.numel(), _stream()), "dit_project_residual")
    return out


def trace_enable(capacity: int):
    """Record a HIP event before every kernel group of later calls (0: off)."""
    check(lib().dit_trace_enable(int(capacity)), "dit_trace_enable")


def trace_records():
    """[(name, ms)] for every traced kernel group so far (waits for them)."""
    out = []
    L = lib()
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    for i in range(L.dit_trace_count() - 1):
        check(L.dit_trace_read(i, ctypes.byref(name), ctypes.byref(ms)), "dit_trace_read")
        if name.value != b"end":
            out.append((name.value.decode(), ms.value))
    return out
