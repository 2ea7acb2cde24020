#!/usr/bin/env python3
"""Benchmark of the Flash DiT block on one MI355X.

Step = one pass of the block's hot path on the 540p / 22-frame latent grid
(T=6, H=34, W=60; 256 text + 132 audio tokens; width 5376, 56 heads of 128,
SwiGLU 14336) with spatial token compression on: the two index builders,
then dit_block_forward (gather-on-read, norm, QKV + rotary, attention, O +
residual, norm, gate/up + SwiGLU, down + residual / update, nearest-kept
broadcast onto all 12240 video positions). Inputs are resident in HBM before
the timed region. The same block with compression off (all 12628 tokens) is
timed as a second line item.

The bandwidth-bound kernels (gather of the kept rows, nearest-kept broadcast
plus residual, the first RMSNorm) are also timed alone on the same shapes:
back-to-back launches that rotate over disjoint buffer sets several times the
256 MB Infinity Cache (so no launch finds its data cached; the number their
HBM roofline fraction is quoted on), and each once more after a 1 GiB read
that flushes the caches (a write flush would leave up to ~290 MB of dirty
lines whose write-back to HBM would then be charged to the kernel under test).

Warm-up: after a short warm-up the first few timed steps run 3-14 % slower
than the rest (measured: 3.19, 3.09, 2.92 ... ms, then 2.80 ms per step after
3 warm-up steps; every step at 2.78-2.84 ms after 10), so 10 untimed steps
come first by default.

Prints one JSON line (see the repository's bench contract).
    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--no-cpu] [--no-off] [--copy-calib]

--copy-calib adds three plain 1 GiB elementwise copies after the timed region:
the reference dispatches that scale rocprofv3's FETCH_SIZE / WRITE_SIZE
counters to bytes (see TRAFFIC).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "Flash DiT block ms & TFLOP/s (% bf16 MFMA peak), 540p/22f, compression on/off"
PEAK_BF16 = 2500.0     # TFLOP/s, dense MFMA, MI355X
PEAK_HBM = 8000.0      # GB/s
HERE = os.path.dirname(os.path.abspath(__file__))

# HBM traffic of the dominant kernel, from two rocprofv3 counter runs of
# `bench.py --no-cpu --no-off --no-sweep --no-stack --no-decoder --no-long --steps 2 --warmup 1 --copy-calib` (FETCH_SIZE,
# then WRITE_SIZE; KiB per dispatch), each divided by what the same counter
# reads per byte of a plain 1 GiB copy. Valid only for the kernel source it was
# taken on (sha256 of the listed files); otherwise reported as null.
TRAFFIC = {
    "gemm_gate_up": {"files": ['video_diffusion_transformer_flash_amd/csrc/gemm_mfma.hip', 'video_diffusion_transformer_flash_amd/csrc/epilogue.h', 'video_diffusion_transformer_flash_amd/csrc/common.h'], "sha": "4559f460bcd4e169",
                     "fetch_bytes": 2725940383, "write_bytes": 107118592,
                     "copy_scale": {"FETCH_SIZE": 1.99994, "WRITE_SIZE": 1.0},
                     "source": "profiles/gemm_gate_up_540p_compressed_hbm_traffic.md"},
    "broadcast_residual": {"files": ['video_diffusion_transformer_flash_amd/csrc/rowops.hip', 'video_diffusion_transformer_flash_amd/csrc/common.h'], "sha": "663a96d5164a6d1f",
                           "fetch_bytes": 169073918, "write_bytes": 131642304,
                           "copy_scale": {"FETCH_SIZE": 1.99992, "WRITE_SIZE": 1.0},
                           "source": "profiles/broadcast_residual_540p_compressed_hbm_traffic.md"},
}


def _src_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    t = TRAFFIC.get(kernel)
    if not t or _src_sha(t["files"]) != t["sha"]:
        return None
    return {"bytes": t["fetch_bytes"] + t["write_bytes"], "fetch_bytes": t["fetch_bytes"],
            "write_bytes": t["write_bytes"], "copy_scale": t["copy_scale"], "source": t["source"]}


def _traffic_bytes(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled), or None."""
    t = traffic_for(kernel)
    return None if t is None else t["bytes"]


def block_flops(d, S):
    """Algorithmic FLOPs (2 per MAC) of one block on S tokens, per kernel."""
    D, I, F = d.d_model, d.inner, d.d_ffn
    return {"gemm_qkv": 2.0 * S * D * 3 * I, "attention": 4.0 * S * S * I, "gemm_o": 2.0 * S * I * D,
            "gemm_gate_up": 2.0 * S * D * 2 * F, "gemm_down": 2.0 * S * F * D}


def hbm_bytes(d, S, Nv, Nk, es=2):
    """Algorithmic bytes of the bandwidth-bound kernels per launch."""
    D = d.d_model
    return {"broadcast_residual": (2 * Nv + Nk) * D * es,      # read x, read the update once, write out
            "rmsnorm1": 2 * S * D * es,                        # read X rows, write n
            "rmsnorm2": S * D * (4 + es)}                      # read h (fp32), write n


def broadcast_bytes_moved(Nv, Nk, D, es=2):
    """Bytes the standalone broadcast kernel moves: its update rows are fp32."""
    return (2 * Nv * es + Nk * 4) * D


def setup(cfg_name, compress):
    import torch
    import video_diffusion_transformer_flash_amd as V
    from dit_synth import CONFIGS, activations, weights
    d = CONFIGS[cfg_name]
    x = activations(d, d.seed)
    w = weights(d, d.seed)
    dev = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    gw = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in w.items()}
    dims = V.make_dims(d)
    s = d.stride
    Hk, Wk = V.keep_dims(d.H, d.W, s)
    keep = torch.empty(d.T * Hk * Wk, dtype=torch.int32, device="cuda")
    nk = torch.empty(d.n_video, dtype=torch.int32, device="cuda")
    out = tuple(torch.empty_like(dev[k]) for k in ("x_text", "x_video", "x_audio"))
    ws = V.workspace(V.block_workspace_size(dims, compress))

    def step():
        if compress:
            V.keep_index(d.T, d.H, d.W, s, out=keep)
            V.nearest_kept_map(d.T, d.H, d.W, s, out=nk)
        V.block_forward(dims, dev["x_text"], dev["x_video"], dev["x_audio"], gw, compress,
                        keep if compress else None, nk if compress else None, out=out, ws=ws)

    S = d.n_text + d.n_audio + (d.T * Hk * Wk if compress else d.n_video)
    return d, step, S, d.T * Hk * Wk, (x, w)


def time_steps(step, steps, warmup, trace=False):
    """Warm up, then time exactly `steps` steps between two synchronisations:
    returns (ms per step over the whole region, median of the per-step times,
    per-kernel-group (ms, launches) from the library's HIP-event trace when
    `trace` is on; the trace records an event between kernel groups, so the
    headline figures come from an untraced run)."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if trace:
        V.trace_enable(steps * 24 + 8)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(st)
    for i in range(steps):
        step()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    med = per_step[len(per_step) // 2]
    recs = V.trace_records() if trace else []
    if trace:
        V.trace_enable(0)
    per = {}
    for name, t in recs:
        a = per.setdefault(name, [0.0, 0])
        a[0] += t
        a[1] += 1
    return ms, med, {k: (v[0] / v[1], v[1]) for k, v in per.items()}


def kernel_table(kern, flops, bytes_):
    out = {}
    for name, (ms, n) in sorted(kern.items(), key=lambda kv: -kv[1][0]):
        e = {"ms": round(ms, 4), "launches": n}
        if name in flops:
            tf = flops[name] / (ms * 1e-3) / 1e12
            e.update({"TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16, 4)})
        if name in bytes_:
            gb = bytes_[name] / (ms * 1e-3) / 1e9
            e.update({"GB/s": round(gb, 1), "frac": round(gb / PEAK_HBM, 4)})
        out[name] = e
    return out


def bandwidth_kernels(d, reps=10, rounds=5):
    """The bandwidth-bound steps alone on the workload's shapes: the gather of
    the kept rows, the nearest-kept broadcast + residual (update rows bf16, as
    the algorithmic bytes count them, and fp32) and the first RMSNorm on the
    joint sequence. Two measurements per kernel, data never cache-resident:
      * rotated: back-to-back launches cycling over disjoint buffer sets that
        together exceed the 256 MB Infinity Cache several times, `rounds`
        passes over the sets between two events (per-launch mean);
      * flushed: one launch after a 1 GiB read that evicts the caches and
        leaves nothing dirty (median of `reps`; includes the event overhead).
    Beside each, torch's own device copy of the same bytes under the flush."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    Hk, Wk = V.keep_dims(d.H, d.W, d.stride)
    Nk, Nv, D = d.T * Hk * Wk, d.n_video, d.d_model
    S = d.n_text + d.n_audio + Nk
    g = torch.Generator(device="cuda").manual_seed(1000 + d.seed)
    keep = V.keep_index(d.T, d.H, d.W, d.stride)
    nk = V.nearest_kept_map(d.T, d.H, d.W, d.stride)
    gain = (1 + 0.1 ** 0.5 * torch.randn(D, device="cuda", generator=g)).bfloat16()

    def sets(n, make):
        return [make() for _ in range(n)]

    bc = sets(4, lambda: (torch.randn(Nv, D, device="cuda", generator=g).bfloat16(),
                          torch.randn(Nk, D, device="cuda", generator=g),
                          torch.empty(Nv, D, dtype=torch.bfloat16, device="cuda")))
    bc16 = [(x, dl.bfloat16(), o) for x, dl, o in bc]
    ga = sets(8, lambda: (torch.randn(Nv, D, device="cuda", generator=g).bfloat16(),
                          torch.empty(Nk, D, dtype=torch.bfloat16, device="cuda")))
    nm = sets(8, lambda: torch.randn(S, D, device="cuda", generator=g).bfloat16())
    fns = {
        "broadcast_residual": [lambda s=s: V.broadcast_residual(s[0], s[1], nk, out=s[2]) for s in bc16],
        "broadcast_residual_fp32_update": [lambda s=s: V.broadcast_residual(s[0], s[1], nk, out=s[2]) for s in bc],
        "gather_kept": [lambda s=s: V.gather_kept(s[0], keep, out=s[1]) for s in ga],
        "rmsnorm1": [lambda s=s: V.rmsnorm(s, gain, d.eps, "bf16") for s in nm],
    }
    # algorithmic bytes: every row read and written once at 2 bytes per element
    byts = {"broadcast_residual": (2 * Nv + Nk) * D * 2, "broadcast_residual_fp32_update": (2 * Nv + Nk) * D * 2,
            "gather_kept": 2 * Nk * D * 2, "rmsnorm1": 2 * S * D * 2}
    moved = dict(byts, broadcast_residual_fp32_update=broadcast_bytes_moved(Nv, Nk, D))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rot = {}
    for name, fl in fns.items():
        for f in fl:
            f()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(rounds):
            for f in fl:
                f()
        e1.record()
        torch.cuda.synchronize()
        rot[name] = e0.elapsed_time(e1) / (rounds * len(fl))
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")   # 1 GiB
    fl_t = {k: [] for k in fns}
    for r in range(reps + 2):
        for name, fl in fns.items():
            flush.amax()
            e0.record()
            fl[0]()
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                fl_t[name].append(e0.elapsed_time(e1))
    cref = {}
    for name, nb in moved.items():
        a = torch.ones(nb // 4, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        ts = []
        for r in range(reps + 2):
            flush.amax()
            e0.record()
            b.copy_(a)
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(e0.elapsed_time(e1))
        cref[name] = sorted(ts)[len(ts) // 2]
        del a, b
    res = {}
    for name in fns:
        ms = rot[name]
        msf = sorted(fl_t[name])[len(fl_t[name]) // 2]
        gbs, gbf = byts[name] / (ms * 1e-3) / 1e9, byts[name] / (msf * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": byts[name], "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM, 4),
                     "bytes_moved": moved[name], "moved_frac": round(moved[name] / (ms * 1e-3) / 1e9 / PEAK_HBM, 4),
                     "flushed_ms": round(msf, 4), "flushed_frac": round(gbf / PEAK_HBM, 4),
                     "torch_copy_same_bytes_flushed_GB/s": round(moved[name] / (cref[name] * 1e-3) / 1e9, 1)}
    del flush, bc, bc16, ga, nm
    return res


def _gpu_block_inputs(d, seed, fp8=False):
    """Seeded synthetic inputs generated on the device (timing only; the parity
    tests use the host generator): activations N(0, 1); weights N(0, 1/fan_in);
    gains 1 + N(0, 0.1); bf16, or e4m3 codes + scale for fp8 projections."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    g = torch.Generator(device="cuda").manual_seed(seed)
    D, I, F = d.d_model, d.inner, d.d_ffn

    def normal(shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std + mean

    x = {"x_text": normal((d.n_text, D)).bfloat16(), "x_video": normal((d.T, d.H, d.W, D)).bfloat16(),
         "x_audio": normal((d.n_audio, D)).bfloat16()}
    shapes = {"wqkv": ((3 * I, D), D), "wo": ((D, I), I), "wgate": ((F, D), D), "wup": ((F, D), D),
              "wdown": ((D, F), F)}
    w = {"g1": normal((D,), 0.1 ** 0.5, 1.0).bfloat16(), "g2": normal((D,), 0.1 ** 0.5, 1.0).bfloat16()}
    for k, (shape, fan_in) in shapes.items():
        t = normal(shape, fan_in ** -0.5)
        if fp8:
            w[k], w["s_" + k] = V.quantize_fp8(t)
        else:
            w[k] = t.bfloat16()
        del t
    return x, w


def sweep(steps=2, warmup=1):
    """768p grid at T = 2, 8, 32 latent frames, compression on and off:
    block latency and TFLOP/s (device-generated inputs of the configuration's
    distributions)."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    from dit_synth import CONFIGS, SWEEP_FRAMES
    res = []
    for T in SWEEP_FRAMES:
        d = CONFIGS["768p"].with_(name=f"768p_T{T}", T=T)
        x, w = _gpu_block_inputs(d, 3000 + T)
        dims = V.make_dims(d)
        Hk, Wk = V.keep_dims(d.H, d.W, d.stride)
        keep = V.keep_index(d.T, d.H, d.W, d.stride)
        nk = V.nearest_kept_map(d.T, d.H, d.W, d.stride)
        out = tuple(torch.empty_like(x[k]) for k in ("x_text", "x_video", "x_audio"))
        for comp in (True, False):
            ws = V.workspace(V.block_workspace_size(dims, comp))

            def step():
                V.block_forward(dims, x["x_text"], x["x_video"], x["x_audio"], w, comp, keep if comp else None,
                                nk if comp else None, out=out, ws=ws)

            ms, _, _ = time_steps(step, steps, warmup)
            S = d.n_text + d.n_audio + (d.T * Hk * Wk if comp else d.n_video)
            tf = sum(block_flops(d, S).values()) / 1e12
            res.append({"T": T, "compress": comp, "tokens": S, "ms": round(ms, 3), "tflop": round(tf, 3),
                        "TFLOP/s": round(tf / (ms * 1e-3), 1), "frac_of_bf16_peak": round(tf / (ms * 1e-3) / PEAK_BF16, 4)})
            del ws
            torch.cuda.empty_cache()
        del x, w, out
        torch.cuda.empty_cache()
    return res


def _stack_setup():
    """The Flash stack's configuration and device-generated fp8 layers: layer
    flags (2 full, 26 compressed, 14 full), the 540p inputs, the index maps and
    the fixed 3-step schedules t_k = u/(u + s(1-u)), u = k/3 (s = 12 video, 3
    audio)."""
    import video_diffusion_transformer_flash_amd as V
    from dit_synth import CONFIGS, FLASH_EVALS, FLASH_LAYERS
    d = CONFIGS["stack"]
    a, b, c = FLASH_LAYERS
    flags = [0] * a + [1] * b + [0] * c
    x, w0 = _gpu_block_inputs(d, 4000, fp8=True)
    layers = [w0] + [_gpu_block_inputs(d.with_(T=1, H=1, W=1, n_text=1, n_audio=1), 4001 + l, fp8=True)[1]
                     for l in range(1, len(flags))]
    dims = V.make_dims(d)
    keep = V.keep_index(d.T, d.H, d.W, d.stride)
    nk = V.nearest_kept_map(d.T, d.H, d.W, d.stride)

    def sched(n, s):
        return [(k / n) / ((k / n) + s * (1 - k / n)) for k in range(n + 1)]

    return d, dims, flags, x, w0, layers, keep, nk, sched(FLASH_EVALS, 12.0), sched(FLASH_EVALS, 3.0)


def long_video_timing(chunks=4):
    """Chunk-by-chunk long video with the Flash stack (fp8, 42 layers, 3
    evaluations per chunk) on the 540p chunk grid: the first chunk denoises 6
    latent frames, each later chunk holds the last frame made so far fixed and
    adds 5 new ones with the bounded history of the earlier frames joined as
    control tokens. Reports the time of the whole video (one
    dit_long_video_sample call), each chunk's time as a stack call of its own,
    and each chunk's history token count."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    d, dims, flags, x, w0, layers, keep, nk, tv, ta = _stack_setup()
    g = torch.Generator(device="cuda").manual_seed(4100)
    new = [torch.randn((d.T - 1, d.H, d.W, d.d_model), generator=g, device="cuda").bfloat16()
           for _ in range(chunks - 1)]
    audio = [x["x_audio"].clone() for _ in range(chunks)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the whole video in one dit_long_video_sample call (the first pass warms up)
    V.long_video_sample(dims, layers, flags, tv, ta, x["x_text"], x["x_video"].clone(), new, audio, keep, nk)
    torch.cuda.synchronize()
    e0.record()
    frames = V.long_video_sample(dims, layers, flags, tv, ta, x["x_text"], x["x_video"].clone(), new, audio, keep, nk)
    e1.record()
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1)
    # the same chunks one stack call each, timed apart (the call above runs exactly these)
    T = d.T
    fr = torch.empty_like(frames)
    fr[:T].copy_(x["x_video"])
    for c, n in enumerate(new):
        fr[T + c * (T - 1):T + (c + 1) * (T - 1)].copy_(n)
    times = []
    for c in range(chunks):
        kw, win = {}, fr[:T]
        dc = V.Dims.from_buffer_copy(dims)
        if c > 0:
            n_hist = T + (c - 1) * (T - 1) - 1
            dc.n_ctrl, dc.ctrl_offset, dc.n_fixed = n_hist, n_hist, 1
            kw = {"x_ctrl": fr[:n_hist], "ctrl_idx": V.history_index(n_hist, d.H, d.W)}
            win = fr[n_hist:n_hist + T]
        torch.cuda.synchronize()
        e0.record()
        V.stack_sample(dc, layers, flags, tv, ta, x["x_text"], win, audio[c], keep, nk, **kw)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    # chunk k > 0 starts after T + (k - 1)(T - 1) frames; all but the boundary are history
    hist = [0] + [int(V.history_index(d.T + k * (d.T - 1) - 1, d.H, d.W).numel()) for k in range(chunks - 1)]
    ok = bool(torch.isfinite(frames.float()).all())
    del layers, w0, frames, new, audio
    torch.cuda.empty_cache()
    return {"workload": f"{chunks} chunks of the 42-layer fp8 stack (3 evaluations each) on the 540p chunk grid "
                        "6x34x60: 6 frames, then 5 new frames per chunk with a fixed boundary frame and the "
                        "bounded history as control tokens", "frames": d.T + (chunks - 1) * (d.T - 1),
            "total_ms": round(total, 1), "chunk_ms": [round(t, 1) for t in times], "history_tokens": hist,
            "outputs_finite": ok}


def stack_timing(reps=3):
    """The Flash-shaped stack: 42 blocks with fp8 projections (layers 1-2 full,
    3-28 compressed, 29-42 full) on the 540p grid, 3 flow-matching Euler
    evaluations on the fixed schedule t_k = u/(u + s(1-u)), u = k/3 (s = 12
    video, 3 audio). Reported against the mixed roofline: GEMM FLOPs at the fp8
    peak plus attention FLOPs at the bf16 peak."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    from dit_synth import FLASH_EVALS
    d, dims, flags, x, w0, layers, keep, nk, tv, ta = _stack_setup()
    ws = V.workspace(V.stack_workspace_size(dims, flags))
    xv0, xa0 = x["x_video"].clone(), x["x_audio"].clone()

    def run():
        x["x_video"].copy_(xv0)
        x["x_audio"].copy_(xa0)
        V.stack_sample(dims, layers, flags, tv, ta, x["x_text"], x["x_video"], x["x_audio"], keep, nk, ws=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    Hk, Wk = V.keep_dims(d.H, d.W, d.stride)
    S_on, S_off = d.n_text + d.n_audio + d.T * Hk * Wk, d.n_text + d.n_audio + d.n_video
    f_on, f_off = block_flops(d, S_on), block_flops(d, S_off)
    gemm = FLASH_EVALS * sum(v for fl in flags for k, v in (f_on if fl else f_off).items() if k != "attention")
    att = FLASH_EVALS * sum((f_on if fl else f_off)["attention"] for fl in flags)
    roof_ms = (gemm / (2 * PEAK_BF16 * 1e12) + att / (PEAK_BF16 * 1e12)) * 1e3
    ok = bool(torch.isfinite(x["x_video"].float()).all() and torch.isfinite(x["x_audio"].float()).all())
    del layers, w0, ws
    torch.cuda.empty_cache()
    return {"workload": "42 blocks (2 full, 26 compressed, 14 full), fp8 e4m3 projections with per-tensor scales, "
                        "540p grid 6x34x60, 3 Euler evaluations", "ms": round(ms, 2), "reps": reps,
            "tflop": round((gemm + att) / 1e12, 1), "TFLOP/s": round((gemm + att) / 1e12 / (ms * 1e-3), 1),
            "mixed_roofline_ms": round(roof_ms, 1), "frac_of_mixed_roofline": round(roof_ms / ms, 4),
            "outputs_finite": ok}


def decoder_timing(reps=3):
    """A stand-in for the distilled light decoder: 26 blocks at its widths
    (hidden 2048, 16 heads of 128, FFN 4 x 2048) over the 540p latent grid
    (6 x 34 x 60 tokens, no text or audio, no compression), bf16, each layer
    with its own weights. The pages give the decoder's depth and widths only
    (its upsampling and convolutions are not described), so this times a
    transformer of that size on the latent tokens, not the decoder itself."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    from dit_synth import CONFIGS, DECODER_LAYERS
    d = CONFIGS["decoder"]
    x, w0 = _gpu_block_inputs(d, 5000)
    one = d.with_(T=1, H=1, W=1)
    layers = [w0] + [_gpu_block_inputs(one, 5001 + l)[1] for l in range(1, DECODER_LAYERS)]
    dims = V.make_dims(d)
    ws = V.workspace(V.block_workspace_size(dims, False))
    xt, xa = x["x_text"], x["x_audio"]
    bufs = [x["x_video"].clone(), torch.empty_like(x["x_video"])]
    yt, ya = torch.empty_like(xt), torch.empty_like(xa)

    def run():
        for l, w in enumerate(layers):
            src, dst = bufs[l % 2], bufs[(l + 1) % 2]
            V.block_forward(dims, xt, src, xa, w, False, None, None, out=(yt, dst, ya), ws=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        bufs[0].copy_(x["x_video"])
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    fl = block_flops(d, d.n_video)
    tf = DECODER_LAYERS * sum(fl.values()) / 1e12
    ok = bool(torch.isfinite(bufs[DECODER_LAYERS % 2].float()).all())
    del layers, w0, ws, bufs
    torch.cuda.empty_cache()
    return {"workload": f"{DECODER_LAYERS} blocks of width 2048 (16 x 128 heads, FFN 8192), 540p latent grid "
                        "6x34x60 (12240 tokens), bf16, uncompressed", "ms": round(ms, 2), "reps": reps,
            "ms_per_layer": round(ms / DECODER_LAYERS, 3), "tflop": round(tf, 2),
            "TFLOP/s": round(tf / (ms * 1e-3), 1), "frac_of_bf16_peak": round(tf / (ms * 1e-3) / PEAK_BF16, 4),
            "attention_share_of_flops": round(fl["attention"] / sum(fl.values()), 3), "outputs_finite": ok}


def copy_calibration(nbytes=1 << 30, reps=3):
    """Plain elementwise copies of a known size (b = a * 1 over fp32, 16-byte
    vector accesses like the library's kernels): the reference dispatches
    that scale the HBM counters to bytes. (A same-dtype copy_ would go to the
    runtime's blit kernel, whose wider requests the fetch counter reads
    differently.)"""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()


def cpu_info():
    """Host cores this process may use and the CPU's identification."""
    info = {"cores": len(os.sched_getaffinity(0)), "cpu_model": "unknown"}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                key = {"cpu family": "cpu_family", "model": "cpu_model_number", "stepping": "cpu_stepping"}.get(k)
                if k == "model name" and info["cpu_model"] == "unknown":
                    info["cpu_model"] = v
                elif key and key not in info:
                    info[key] = v
                elif not line.strip() and info["cpu_model"] != "unknown":
                    break
    except OSError:
        pass
    return info


def cpu_baseline(d, host, compress, reps=2):
    """The fp64 oracle on the host cores: full blocks of the same workload,
    `reps` times in a row (about 10 s of CPU work), mean per block."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    x, w = host
    ow = O.BlockWeights.from_arrays(w)
    t0 = time.time()
    for _ in range(reps):
        O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress)
    dt = (time.time() - t0) / reps
    Hk, Wk = O.keep_dims(d.H, d.W, d.stride)
    S = d.n_text + d.n_audio + (d.T * Hk * Wk if compress else d.n_video)
    tflop = sum(block_flops(d, S).values()) / 1e12
    out = {"value": round(tflop / dt, 4), "unit": "TFLOP/s", "ms": round(dt * 1e3, 1)}
    out.update(cpu_info())
    out.update({"blas_threads": blas, "kind": "oracle",
                "sample": f"{reps} full blocks in a row of the same workload (S={S}, compression "
                          f"{'on' if compress else 'off'}), fp64 numpy oracle, mean per block"})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)   # the first ~5 steps after a short warm-up run 3-14 % slow
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-off", action="store_true", help="skip the compression-off line item")
    ap.add_argument("--copy-calib", action="store_true", help="add 1 GiB reference copies (counter calibration)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 768p frame sweep")
    ap.add_argument("--no-stack", action="store_true", help="skip the 42-layer fp8 stack")
    ap.add_argument("--no-decoder", action="store_true", help="skip the decoder-width 26-layer stand-in")
    ap.add_argument("--no-long", action="store_true", help="skip the chunk-by-chunk long video")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the block on one GPU; sharding across GPUs is designed but not "
              "implemented (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    d, step, S, Nk, host = setup("540p_on", True)
    ms, med, _ = time_steps(step, a.steps, a.warmup)                 # headline: no trace events
    ms_tr, _, kern = time_steps(step, a.steps, 1, trace=True)          # per-kernel groups (HIP events)
    flops = block_flops(d, S)
    tflop = sum(flops.values()) / 1e12
    value = tflop / (ms * 1e-3)
    byts = hbm_bytes(d, S, d.n_video, Nk)
    table = kernel_table(kern, flops, byts)
    dom = max(flops, key=lambda k: kern.get(k, (0, 0))[0] * kern.get(k, (0, 0))[1])
    dom_ms = kern[dom][0]
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": "Flash DiT block, 540p/22f latent grid 6x34x60, compression on "
                               f"(3348 kept video + 256 text + 132 audio = {S} tokens), broadcast to 12240 positions",
                   "tflop_per_step": round(tflop, 4), "frac_of_bf16_peak": round(value / PEAK_BF16, 4)},
        "median_step_ms": round(med, 4),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "flop_per_launch": flops[dom], "launch_ms": round(dom_ms, 4),
                     "traffic": _traffic_bytes(dom), "traffic_detail": traffic_for(dom)},
        "kernels": table,
        "kernels_note": f"HIP events between kernel groups over a second run of {a.steps} steps "
                        f"({round(ms_tr, 4)} ms per step with the events)",
    }
    if a.copy_calib:
        copy_calibration()
    torch.cuda.empty_cache()
    bw = bandwidth_kernels(d)
    bc = bw["broadcast_residual"]
    line["hbm_roofline"] = {"bound": "hbm", "kernel": "broadcast_residual", "achieved": bc["GB/s"],
                            "peak": PEAK_HBM, "unit": "GB/s", "frac": bc["frac"], "bytes_per_launch": bc["bytes"],
                            "launch_ms": bc["ms"], "update_rows": "bf16",
                            "cache": "launches rotate over 4 disjoint buffer sets (1.2 GB), never cache-resident",
                            "traffic": _traffic_bytes("broadcast_residual"),
                            "traffic_detail": traffic_for("broadcast_residual")}
    line["bandwidth_kernels"] = bw
    torch.cuda.empty_cache()
    if not a.no_off:
        d2, step2, S2, _, host2 = setup("540p_off", False)
        ms2, _, _ = time_steps(step2, max(3, a.steps // 2), a.warmup)
        _, _, kern2 = time_steps(step2, max(3, a.steps // 2), 1, trace=True)
        f2 = block_flops(d2, S2)
        tf2 = sum(f2.values()) / 1e12
        line["compress_off"] = {"workload": f"same block, compression off ({S2} tokens)", "ms": round(ms2, 4),
                                "TFLOP/s": round(tf2 / (ms2 * 1e-3), 2),
                                "frac_of_bf16_peak": round(tf2 / (ms2 * 1e-3) / PEAK_BF16, 4),
                                "tflop_per_step": round(tf2, 4),
                                "kernels": kernel_table(kern2, f2, hbm_bytes(d2, S2, d2.n_video, 0))}
        line["on_off_speedup"] = round(ms2 / ms, 3)
        del host2
    # the secondary measurements: an error in one is recorded in its entry and
    # the others and the headline line still come out
    for flag, key, fn in ((a.no_sweep, "sweep_768p", sweep), (a.no_stack, "stack", stack_timing),
                          (a.no_decoder, "decoder_standin", decoder_timing),
                          (a.no_long, "long_video", long_video_timing),
                          (a.no_cpu, "cpu_baseline", lambda: cpu_baseline(d, host, True))):
        if flag:
            continue
        try:
            line[key] = fn()
        except Exception as e:  # noqa: BLE001
            line[key] = {"error": f"{type(e).__name__}: {e}"[:400]}
            print(f"bench.py: {key} failed: {e!r}", file=sys.stderr)
        torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
