"""Workload shapes for one pipeline stage of patch-level DiT inference.

PipeFusion (gist.science PipeFusion summary, "Core mechanisms" 1-2) cuts the
DiT backbone into contiguous layer groups, one per device, and splits the token
sequence into M non-overlapping patches that flow through a stage one at a time.
One stage here is `num_layers` contiguous transformer blocks of width `hidden`
with `heads` x `head_dim` attention, run over `seq_txt + seq_img` buffer rows.

The five workloads below are synthetic stand-ins for the PixArt / SD3 / Flux.1
stages the summaries evaluate (Experiments section: PixArt 0.6B, SD3 2B,
Flux.1 12B at 1024-4096 px; PixArt at 8192 px).  Values are drawn by
`synth.py`; no trained weights or images are used.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class StageShape:
    name: str
    num_layers: int       # L: contiguous transformer blocks owned by this stage
    hidden: int           # h
    heads: int            # H
    head_dim: int         # d
    mlp_ratio: int        # r (0 = attention sublayer only)
    seq_img: int          # image tokens, split into M patches
    seq_txt: int          # text-prefix rows kept fresh at the front of the buffer
    num_patches: int      # M
    steps: int            # diffusion steps including the single warm-up step
    dtype: str            # "bf16" or "fp32"
    sigma_kv: float       # per-step drift added to every stale K/V value
    w_std: float          # std of weights and biases
    seed: int

    @property
    def seq_kv(self) -> int:
        return self.seq_txt + self.seq_img

    @property
    def patch_rows(self) -> int:
        return self.seq_img // self.num_patches

    def patch_offsets(self):
        """Buffer row offset of patch m: text rows first, then ascending patches."""
        return [self.seq_txt + m * self.patch_rows for m in range(self.num_patches)]

    def flops_per_step(self) -> float:
        """Algorithmic FLOPs of one patched step (projections + attention),
        head_dim counted unpadded; the adaLN GEMV is not counted."""
        h, s = self.hidden, self.seq_kv
        proj = (8 + 4 * self.mlp_ratio) * s * h * h
        attn = 4 * s * s * h
        return float(self.num_layers * (proj + attn))

    def attn_flops_per_step(self) -> float:
        return float(self.num_layers * 4 * self.seq_kv * self.seq_kv * self.hidden)

    def small(self, seq_img: int, num_layers: int | None = None, seq_txt: int | None = None,
              num_patches: int | None = None, seed: int | None = None) -> "StageShape":
        """Same block width / heads / head_dim with a shorter sequence (test-sized)."""
        return dataclasses.replace(
            self, name=self.name + f"-s{seq_img}",
            seq_img=seq_img,
            num_layers=self.num_layers if num_layers is None else num_layers,
            seq_txt=self.seq_txt if seq_txt is None else seq_txt,
            num_patches=self.num_patches if num_patches is None else num_patches,
            seed=(self.seed + 1000) if seed is None else seed)


C1 = StageShape("c1-tiny-fp32", 1, 128, 2, 64, 0, 256, 0, 4, 2, "fp32", 0.05, 1.0 / math.sqrt(128), 1001)
C2 = StageShape("c2-pixart", 4, 1152, 16, 72, 4, 4096, 0, 4, 20, "bf16", 0.02, 0.02, 1002)
C3 = StageShape("c3-sd3", 4, 1536, 24, 64, 4, 16384, 0, 8, 20, "bf16", 0.02, 0.02, 1003)
C4 = StageShape("c4-flux", 8, 3072, 24, 128, 4, 16384, 512, 8, 28, "bf16", 0.02, 0.02, 1004)
C5 = StageShape("c5-long-pixart", 4, 1152, 16, 72, 4, 262144, 0, 16, 4, "bf16", 0.02, 0.02, 1005)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}
