"""The allocation-free block under HIP graph capture (the callers it is for):
dit_block_forward_noalloc recorded once into a graph on the capture stream
and replayed. Every replay, with eager work of the program and
synchronisations between the replays, gives the eager call's outputs bit for
bit (bf16 and fp8, compressed)."""
import pytest

from cases import SMALL_BF16, SMALL_FP8
from helpers import gpu_weights, inputs, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")


@pytest.mark.parametrize("d", [SMALL_BF16, SMALL_FP8], ids=lambda d: d.name)
def test_noalloc_block_replays_in_a_graph(d):
    print(f"graph {d.name}", flush=True)
    x, w = inputs(d)
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gw, _ = gpu_weights(w, d.dtype)
    keep, nk = V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W)
    ref = [t.clone() for t in V.block_forward_noalloc(dims, xt, xv, xa, gw, True, keep, nk)]
    out = tuple(torch.empty_like(t) for t in ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a call on the capture's side stream before capturing
        V.block_forward_noalloc(dims, xt, xv, xa, gw, True, keep, nk, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        V.block_forward_noalloc(dims, xt, xv, xa, gw, True, keep, nk, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), rep
        # eager work of the program between replays: the uncompressed block
        # with its own workspace, and an eager call on the shared scratch
        V.block_forward(dims, xt, xv, xa, gw, False)
        V.block_forward_noalloc(dims, xt, xv, xa, gw, False)
        torch.cuda.synchronize()
