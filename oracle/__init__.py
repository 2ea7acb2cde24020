"""CPU oracle for the Flash DiT block: plain, slow, fp64 numpy.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link anything in this package; only the tests, the smoke check and the
benchmark's CPU-baseline leg do. It shares no code with the HIP library
(video_diffusion_transformer_flash_amd) and imports nothing from it.

Sources (the pages this follows; cited per function):
  * tokendh.com article on LynnReal-Omni: backbone section (block shape,
    tagged joint sequence, 3D rotary positions) and training section (flow
    matching, separate video/audio noise clocks with printed values, Flash
    layer schedule and spatial token compression with a full-resolution
    residual).
  * PaperDaily review (longzhangge.com), section 2 on Flash: 42 layers / 3
    evaluations, per-frame row/column subsampling keeping the edge rows and
    columns, nearest-kept-update residual, low-bit projections with fused
    norm / quantisation / RoPE / residual; section 1: control frames at a
    stable positive time offset; section 3: bounded long-video history.

Readings taken where the pages are silent are stated in each function's
docstring. Pinned by tests/test_oracle_*.py (marked "not gpu"). Functions with
no pin are labelled "parity unpinned".
"""
from .compress import (keep_axis, nearest_axis, keep_dims, keep_index, nearest_kept_map, kept_coords,  # noqa: F401
                       history_frames, history_index)
from .block import (rmsnorm, rope_rotate, attention, swiglu, block_core, block_forward,  # noqa: F401
                    token_coords, BlockWeights)
from .fp8 import e4m3_encode, e4m3_decode, quantize_weight_fp8, E4M3_MAX  # noqa: F401
from .sampler import flow_schedule, stack_sample, flash_layer_flags, long_video_sample  # noqa: F401
