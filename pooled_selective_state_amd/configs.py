"""Layer shapes of the workloads the library is tested and measured on.

Each workload is one pooled bidirectional selective-scan layer (or a chain of
them), named by what it is.  Shapes follow the FastVim widths the pages quote
(FastVim-T d_inner 384, FastVim-S 768, Vim-B 1536; 14x14 token grid at 224^2
with patch 16, 64x64 at 1024^2, 128x128 at 2048^2) and the efficiency setting
of the FastVim summary page (section 实验设计: batch 128, float32).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    h: int
    w: int
    E: int
    N: int = 16
    R: int = 12
    K: int = 0  # kept tokens per image; 0 = dense grid
    io_dtype: str = "f32"  # "f32" or "bf16"
    axes: Tuple[int, ...] = (0,)  # pool axis of each chained block (0 = COLS, 1 = ROWS)
    note: str = field(default="", compare=False)

    @property
    def masked(self) -> bool:
        return self.K > 0

    @property
    def nblocks(self) -> int:
        return len(self.axes)

    @property
    def tokens_per_image(self) -> int:
        return self.K if self.masked else self.h * self.w

    def io_bytes(self) -> int:
        """Bytes the layer must move: x and z read once, out written once."""
        elem = 4 if self.io_dtype == "f32" else 2
        n = self.B * self.tokens_per_image * self.E
        return 3 * n * elem * self.nblocks + (self.B * self.K * 4 if self.masked else 0)


TINY = LayerConfig("tiny_224_T", B=2, h=14, w=14, E=384, R=12,
                   note="FastVim-T layer at 224^2, CPU-scale")
SHORT_224_S = LayerConfig("short_224_S_b128", B=128, h=14, w=14, E=768, R=24,
                          note="FastVim-S width, 128*768 length-14 scans per direction")
CHAIN_1024 = LayerConfig("chain2_1024_T_b128", B=128, h=64, w=64, E=384, R=12, axes=(0, 1),
                         note="two FastVim-T blocks at 1024^2: COLS then ROWS on the transposed grid")
HIRES_2048 = LayerConfig("pooled_2048_T_b128", B=128, h=128, w=128, E=384, R=12,
                         note="FastVim-T layer at 2048^2, batch 128, fp32")
MASKED_B = LayerConfig("masked_224_B_b256", B=256, h=14, w=14, E=1536, R=48, K=49, io_dtype="bf16",
                       note="FastMaskVim layer, Vim-B width, 49 of 196 tokens kept")

ALL = (TINY, SHORT_224_S, CHAIN_1024, HIRES_2048, MASKED_B)
BY_NAME = {c.name: c for c in ALL}
