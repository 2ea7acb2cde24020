"""Sentinels: the calls write every output element and nothing else, and do
not depend on what their workspace held before.

Outputs are views into buffers pre-filled with NaN that extend past them; the
workspace is pre-filled with 0xFF bytes (a NaN pattern in bf16 and fp32) and
extends past the size the call is given. After the call every output element
is finite, the guard regions past the outputs and past the given workspace
still hold their fill, the inputs are unchanged, and a second call on a
zero-filled workspace gives bit-identical outputs."""
import numpy as np
import pytest

from cases import SMALL_BF16, SMALL_FP8, SPLIT_BF16, STACK_SMALL
from helpers import gpu_weights, inputs, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")

GUARD = 4096   # elements past every output, bytes past the workspace


def nan_view(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[:n].view(*shape)


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy().copy()


def guards_hold(bufs, n_elems):
    for b, n in zip(bufs, n_elems):
        tail = b[n:]
        assert torch.isnan(tail).all().item(), "an output guard was written"


def ws_pair(need):
    ws = torch.full((need + GUARD,), 0xFF, dtype=torch.uint8, device="cuda")
    return ws, ws[:need]


def ws_guard_holds(ws, need):
    assert bool((ws[need:] == 0xFF).all().item()), "the workspace guard was written"


@pytest.mark.parametrize("d", [SMALL_BF16, SMALL_FP8, SPLIT_BF16], ids=lambda d: d.name)
@pytest.mark.parametrize("compress", [False, True])
def test_block_sentinels(d, compress):
    print(f"sentinels block {d.name} compress={compress}", flush=True)
    x, w = inputs(d)
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    before = [bits(t) for t in (xt, xv, xa)]
    gw, _ = gpu_weights(w, d.dtype)
    keep = V.keep_index(d.T, d.H, d.W) if compress else None
    nk = V.nearest_kept_map(d.T, d.H, d.W) if compress else None
    need = V.block_workspace_size(dims, compress)
    outs = [nan_view(t.shape, t.dtype) for t in (xt, xv, xa)]
    ws, wsv = ws_pair(need)
    V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk, out=tuple(o[1] for o in outs), ws=wsv)
    torch.cuda.synchronize()
    for _, y in outs:
        assert torch.isfinite(y.float()).all().item(), "an output element was not written"
    guards_hold([o[0] for o in outs], [o[1].numel() for o in outs])
    ws_guard_holds(ws, need)
    for t, b in zip((xt, xv, xa), before):
        assert np.array_equal(bits(t), b), "an input changed"
    first = [bits(o[1]) for o in outs]
    wsv.zero_()
    V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk, out=tuple(o[1] for o in outs), ws=wsv)
    torch.cuda.synchronize()
    for o, f in zip(outs, first):
        assert np.array_equal(bits(o[1]), f), "the result depends on the workspace's earlier contents"


def test_stack_sentinels():
    d = STACK_SMALL.with_(dtype="bf16")
    flags = [0, 1, 1, 0]
    x, _ = inputs(d)
    layers = [gpu_weights(inputs(d, layer=l)[1], d.dtype)[0] for l in range(len(flags))]
    dims = V.make_dims(d)
    keep, nk = V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W)
    need = V.stack_workspace_size(dims, flags)
    results = []
    for fill in (0xFF, 0x00):
        xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
        t0 = bits(xt)
        ws = torch.full((need + GUARD,), fill, dtype=torch.uint8, device="cuda")
        V.stack_sample(dims, layers, flags, [0.0, 0.25, 1.0], None, xt, xv, xa, keep, nk, ws=ws[:need])
        torch.cuda.synchronize()
        assert bool((ws[need:] == fill).all().item()), "the workspace guard was written"
        assert np.array_equal(bits(xt), t0), "text is an input only"
        assert torch.isfinite(xv.float()).all().item() and torch.isfinite(xa.float()).all().item()
        results.append((bits(xv), bits(xa)))
    assert all(np.array_equal(a, b) for a, b in zip(*results))


def test_project_residual_sentinels():
    M, N, K = 3736, 5376, 7168          # the K-split tail writes its slices to the workspace
    g = np.random.default_rng(5)
    tt = lambda a: torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    xres, a, w = tt(g.standard_normal((M, N))), tt(g.standard_normal((M, K))), tt(g.standard_normal((N, K)) / 85)
    import ctypes
    n = ctypes.c_size_t()
    assert V.lib().dit_project_residual_workspace_size(M, N, K, V.DIT_BF16, ctypes.byref(n)) == 0
    need = n.value
    res = []
    for fill in (0xFF, 0x00):
        ws = torch.full((need + GUARD,), fill, dtype=torch.uint8, device="cuda")
        buf, h = nan_view((M, N), torch.float32)
        V.project_residual(xres, a, w, out=h, ws=ws[:need])
        torch.cuda.synchronize()
        assert torch.isfinite(h).all().item()
        guards_hold([buf], [h.numel()])
        assert bool((ws[need:] == fill).all().item())
        res.append(bits(h))
    assert np.array_equal(res[0], res[1])


def test_weights_checked_against_dims():
    """The binding refuses weights whose dtype or size does not match dims
    (e4m3 codes under bf16 dims, a missing scale, a short tensor) before any
    launch: the library takes plain pointers and would read past the end."""
    d = SMALL_FP8
    x, w = inputs(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gw, _ = gpu_weights(w, d.dtype)
    with pytest.raises(V.DitError, match="wqkv"):
        V.block_forward(V.make_dims(d.with_(dtype="bf16")), xt, xv, xa, gw, False)
    no_scale = {k: v for k, v in gw.items() if k != "s_wdown"}
    with pytest.raises(V.DitError, match="s_wdown"):
        V.block_forward(V.make_dims(d), xt, xv, xa, no_scale, False)
    short = dict(gw, wo=gw["wo"][:-1])
    with pytest.raises(V.DitError, match="wo"):
        V.stack_sample(V.make_dims(d), [gw, short], [0, 0], [0.0, 1.0], None, xt, xv, xa)
