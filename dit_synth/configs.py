"""The block configurations used by the tests and the benchmark.

Shapes follow the pages' Flash block (hidden 5376, 56 heads of 128, SwiGLU
width 14336: tokendh.com article, backbone section) on synthetic latent grids
of the 540p / 22-frame and 768p video shapes, plus a tiny fp32 block. Only
sizes live here; nothing in this file computes any part of the block.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class BlockDims:
    name: str
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    T: int
    H: int
    W: int
    n_text: int
    n_audio: int
    rope: tuple            # (t, h, w) band widths inside one head, sum = head_dim
    dtype: str             # "f32" | "bf16" | "fp8" (fp8 projections, bf16 elsewhere)
    seed: int
    rope_base: float = 10000.0
    eps: float = 1e-6
    stride: int = 2
    n_ctrl: int = 0        # control frames at the video's spatial grid (0: none)
    ctrl_offset: int = 0   # target time minus control time (> 0 with control frames)
    n_fixed: int = 0       # leading video frames the sampler holds fixed (a long video's boundary frame)

    @property
    def inner(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_video(self) -> int:
        return self.T * self.H * self.W

    @property
    def n_ctrl_tokens(self) -> int:
        return self.n_ctrl * self.H * self.W

    def with_(self, **kw) -> "BlockDims":
        return replace(self, **kw)


FLASH = dict(d_model=5376, n_heads=56, head_dim=128, d_ffn=14336, rope=(32, 48, 48))

CONFIGS = {
    # tiny fp32 block, compression on and off
    "tiny": BlockDims("tiny", d_model=256, n_heads=4, head_dim=64, d_ffn=704, T=2, H=9, W=15,
                      n_text=16, n_audio=8, rope=(16, 24, 24), dtype="f32", seed=0),
    # 540p / 22-frame latent grid, bf16, compression off
    "540p_off": BlockDims("540p_off", T=6, H=34, W=60, n_text=256, n_audio=132, dtype="bf16", seed=1, **FLASH),
    # same grid, compression on
    "540p_on": BlockDims("540p_on", T=6, H=34, W=60, n_text=256, n_audio=132, dtype="bf16", seed=2, **FLASH),
    # 768p-shaped grid, compression on and off (frame sweep 2, 8, 32 via with_(T=...))
    "768p": BlockDims("768p", T=6, H=48, W=84, n_text=512, n_audio=132, dtype="bf16", seed=3, **FLASH),
    # 42-layer, 3-evaluation fp8 stack on the 540p grid
    "stack": BlockDims("stack", T=6, H=34, W=60, n_text=256, n_audio=132, dtype="fp8", seed=4, **FLASH),
    # the light decoder's width (hidden 2048, FFN 4x: tokendh.com article,
    # decoder section) as a block over the 540p latent grid alone (no text or
    # audio tokens, no compression): a timing stand-in, since the pages give
    # the decoder's depth and widths but not its layers
    "decoder": BlockDims("decoder", d_model=2048, n_heads=16, head_dim=128, d_ffn=8192, T=6, H=34, W=60, n_text=0,
                         n_audio=0, rope=(32, 48, 48), dtype="bf16", seed=11),
}

# Flash layer schedule: 2 full, 26 compressed, 14 full (tokendh.com article,
# training section; PaperDaily review, section 2).
FLASH_LAYERS = (2, 26, 14)
FLASH_EVALS = 3
SWEEP_FRAMES = (2, 8, 32)
# the distilled student decoder's depth (tokendh.com article, decoder section)
DECODER_LAYERS = 26


def get_config(name: str) -> BlockDims:
    return CONFIGS[name]
