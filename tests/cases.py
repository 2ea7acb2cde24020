"""Block and stack configurations of the parity tests (sizes only).

Shared by the GPU parity tests and tests/golden/make_floors.py, which writes
the noise floors of the low-bit and stack cases (tests/floors.py)."""
from dit_synth import CONFIGS, BlockDims

# small bf16 / fp8 blocks: several GEMM and attention tiles and a ragged tail
SMALL_BF16 = BlockDims("small_bf16", d_model=512, n_heads=4, head_dim=128, d_ffn=1024, T=2, H=9, W=15, n_text=16,
                       n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=5)
SMALL_FP8 = SMALL_BF16.with_(name="small_fp8", dtype="fp8", seed=6)
# full Flash width on a small grid
WIDE_FP8 = BlockDims("wide_fp8", T=2, H=6, W=10, n_text=16, n_audio=8, dtype="fp8", seed=8, d_model=5376, n_heads=56,
                     head_dim=128, d_ffn=14336, rope=(32, 48, 48))
# 9 token x 4 feature tiles of 256 x 256 in the O and down projections when
# uncompressed: fewer tiles than compute units, so those projections run
# entirely as K slices plus the slice-sum pass (compressed: 3 token tiles,
# too few to split, the plain path)
SPLIT_BF16 = BlockDims("split_bf16", d_model=1024, n_heads=8, head_dim=128, d_ffn=2048, T=2, H=32, W=32, n_text=16,
                       n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=9)
SPLIT_FP8 = SPLIT_BF16.with_(name="split_fp8", dtype="fp8", seed=10)
# Many tokens at a narrow width: the QKV and gate/up projections run more than
# two rounds of 256 x 256 tiles with a partial last round.
LONG_BF16 = BlockDims("long_bf16", d_model=256, n_heads=2, head_dim=128, d_ffn=512, T=4, H=96, W=120, n_text=16,
                      n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=21)
LONG_FP8 = BlockDims("long_fp8", d_model=256, n_heads=8, head_dim=128, d_ffn=2048, T=2, H=72, W=76, n_text=16,
                     n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=22)
# The fp8 block at the sizes of the 42-layer stack's layers: the 540p grid
# with fp8 projections, compressed (3736 tokens) and not (12628 tokens)
C5_BLOCK = CONFIGS["stack"]

# stacks
STACK_SMALL = BlockDims("stack_small", d_model=256, n_heads=2, head_dim=128, d_ffn=512, T=2, H=9, W=15, n_text=16,
                        n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=7)
STACK_FLAGS = [0, 1, 1, 1, 0, 1]
STACK_WIDE = BlockDims("stack_wide", d_model=5376, n_heads=56, head_dim=128, d_ffn=14336, T=2, H=6, W=10, n_text=16,
                       n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=9)
STACK_WIDE_FLAGS = [0, 1, 1, 0]
# The Flash schedule (42 layers: 2 full, 26 compressed, 14 full; 3
# evaluations) with fp8 projections, at width 1024 on a 2 x 16 x 30 grid
# (984 tokens, 312 compressed): the structure of the 42-layer stack at a size
# the oracle runs in seconds per evaluation
FLASH42 = BlockDims("flash42_fp8", d_model=1024, n_heads=8, head_dim=128, d_ffn=2816, T=2, H=16, W=30, n_text=16,
                    n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=24)

# control frames, bounded history, long video
CTRL_BF16 = BlockDims("ctrl_bf16", d_model=512, n_heads=4, head_dim=128, d_ffn=1024, T=2, H=9, W=15, n_text=16,
                      n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=11, n_ctrl=2, ctrl_offset=3)
CTRL_F32 = BlockDims("ctrl_f32", d_model=256, n_heads=4, head_dim=64, d_ffn=704, T=2, H=9, W=15, n_text=16,
                     n_audio=8, rope=(16, 24, 24), dtype="f32", seed=12, n_ctrl=1, ctrl_offset=2)
CTRL_FP8 = CTRL_BF16.with_(name="ctrl_fp8", dtype="fp8", seed=13)
CTRL_STACK = CTRL_BF16.with_(name="ctrl_stack", d_model=256, n_heads=2, d_ffn=512, seed=14)
HIST = CTRL_BF16.with_(name="hist_bf16", n_ctrl=12, ctrl_offset=12, seed=15)
HIST_STACK = HIST.with_(name="hist_stack", d_model=256, n_heads=2, d_ffn=512, n_ctrl=5, ctrl_offset=5, seed=16)
LONG_VIDEO = CTRL_BF16.with_(name="long_video", d_model=256, n_heads=2, d_ffn=512, T=3, H=8, W=12, n_ctrl=0,
                             ctrl_offset=0, seed=17)


# fp8 blocks on degenerate grids: (T, H, W, n_text, n_audio); a single token,
# text only beside a 2 x 2 grid, audio beside a one-column grid
DEG_FP8 = [SMALL_FP8.with_(name=f"deg_fp8_{T}x{H}x{W}", T=T, H=H, W=W, n_text=nt, n_audio=na)
           for T, H, W, nt, na in [(1, 1, 1, 0, 0), (1, 2, 2, 3, 0), (2, 3, 1, 0, 5)]]
