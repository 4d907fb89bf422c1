"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and converts storage formats; it holds no
step of the method.  Recipe (one numpy PCG64 stream per workload, seed from the
shape table):

1. per layer, in order: W_qkv [3h,h], b_qkv [3h], W_o [h,h], b_o [h],
   W1 [rh,h], b1 [rh], W2 [h,rh], b2 [h], W_ada [6h,h], b_ada [6h]
   (all N(0, w_std^2); the MLP entries are skipped when r = 0);
2. x_all [S_kv, h] ~ N(0, 1), the stage input (kept constant across steps);
3. c [h] ~ N(0, 1), the conditioning vector;
4. for each step s >= 1 and each layer: noise_k, noise_v [S_kv, h] ~ N(0, sigma_kv^2),
   the per-step drift of the stale K/V context.

For bf16 workloads weight matrices are rounded once to bf16 (round to nearest
even, via torch's dtype conversion) and both the HIP path and the oracle read
those exact values; biases, x, c and the noise stay fp32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .configs import StageShape

WEIGHT_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2", "w_ada", "b_ada")
MATRIX_NAMES = ("w_qkv", "w_o", "w1", "w2", "w_ada")


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """fp32 array -> fp32 array holding the nearest-even bf16 values (torch conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def layer_shapes(h: int, r: int):
    shapes = {"w_qkv": (3 * h, h), "b_qkv": (3 * h,), "w_o": (h, h), "b_o": (h,),
              "w1": (r * h, h), "b1": (r * h,), "w2": (h, r * h), "b2": (h,),
              "w_ada": (6 * h, h), "b_ada": (6 * h,)}
    return shapes


@dataclasses.dataclass
class StageInputs:
    shape: StageShape
    layers: list          # list of dict name -> fp32 ndarray
    x: np.ndarray         # fp32 [S_kv, h]
    c: np.ndarray         # fp32 [h]
    _rng: np.random.Generator
    _next_step: int = 1

    def next_noise(self):
        """Noise for the next step (s = 1, 2, ... in order): list of (nk, nv) per layer."""
        s = self.shape
        out = []
        for _ in range(s.num_layers):
            nk = self._rng.standard_normal((s.seq_kv, s.hidden), dtype=np.float32) * np.float32(s.sigma_kv)
            nv = self._rng.standard_normal((s.seq_kv, s.hidden), dtype=np.float32) * np.float32(s.sigma_kv)
            out.append((nk, nv))
        self._next_step += 1
        return out


def stage_inputs(shape: StageShape, seed: int | None = None) -> StageInputs:
    rng = np.random.Generator(np.random.PCG64(shape.seed if seed is None else seed))
    h, r = shape.hidden, shape.mlp_ratio
    shapes = layer_shapes(h, r)
    std = np.float32(shape.w_std)
    layers = []
    for _ in range(shape.num_layers):
        lw = {}
        for name in WEIGHT_NAMES:
            shp = shapes[name]
            if r == 0 and name in ("w1", "b1", "w2", "b2"):
                lw[name] = np.zeros(shp, np.float32)
                continue
            a = rng.standard_normal(shp, dtype=np.float32) * std
            if shape.dtype == "bf16" and name in MATRIX_NAMES:
                a = to_bf16_values(a)
            lw[name] = a
        layers.append(lw)
    x = rng.standard_normal((shape.seq_kv, h), dtype=np.float32)
    c = rng.standard_normal((h,), dtype=np.float32)
    return StageInputs(shape, layers, x, c, rng)


@dataclasses.dataclass
class MMDiTInputs:
    layers: list           # image-stream layer dicts: the StageInputs layers plus q_norm, k_norm [d]
    txt_layers: list       # text-stream layer dicts of the same form
    angles: np.ndarray     # fp32 [S_kv, d/2] rotation angles of the buffer rows


def mmdit_inputs(shape: StageShape, inputs: StageInputs, seed: int | None = None) -> MMDiTInputs:
    """Extra inputs of the MM-DiT block options, from generator PCG64(shape.seed + 3000): a
    text-stream layer set drawn like step 1 of the recipe, then per layer q_norm and k_norm of
    the image stream and of the text stream, each [d] ~ 1 + N(0, 0.3^2).

    The rotation angles are rope_angles(shape)."""
    rng = np.random.Generator(np.random.PCG64(shape.seed + 3000 if seed is None else seed))
    h, r, d = shape.hidden, shape.mlp_ratio, shape.head_dim
    shapes = layer_shapes(h, r)
    std = np.float32(shape.w_std)
    txt = []
    for _ in range(shape.num_layers):
        lw = {}
        for name in WEIGHT_NAMES:
            if r == 0 and name in ("w1", "b1", "w2", "b2"):
                lw[name] = np.zeros(shapes[name], np.float32)
                continue
            a = rng.standard_normal(shapes[name], dtype=np.float32) * std
            if shape.dtype == "bf16" and name in MATRIX_NAMES:
                a = to_bf16_values(a)
            lw[name] = a
        txt.append(lw)
    img = [dict(lw) for lw in inputs.layers]
    for sets in (img, txt):
        for lw in sets:
            lw["q_norm"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
            lw["k_norm"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    return MMDiTInputs(img, txt, rope_angles(shape))


def rope_angles(shape: StageShape) -> np.ndarray:
    """fp32 [S_kv, d/2] rotation angles in the published Flux.1 position layout (no random draw):
    a buffer row has a 3-axis position, (0, 0, 0) for every text row and (0, gy, gx) for image
    row gy * gw + gx (gw: the largest divisor of seq_img not above its square root); the d/2
    pairs of a head split into axes of a0 = d // 16 pairs and two of (d/2 - a0) / 2, and pair j
    of an axis with n pairs turns by position * 10000^(-j / n)."""
    d = shape.head_dim
    gw = max(g for g in range(1, int(shape.seq_img ** 0.5) + 1) if shape.seq_img % g == 0)
    a0 = d // 16
    a1 = (d // 2 - a0) // 2
    axes = (a0, a1, d // 2 - a0 - a1)
    pos = np.zeros((shape.seq_kv, 3), np.float64)
    s_img = np.arange(shape.seq_img)
    pos[shape.seq_txt:, 1] = s_img // gw
    pos[shape.seq_txt:, 2] = s_img % gw
    cols = []
    for axis, n in enumerate(axes):
        freq = 10000.0 ** (-np.arange(n, dtype=np.float64) / n)
        cols.append(pos[:, axis:axis + 1] * freq[None, :])
    return np.concatenate(cols, axis=1).astype(np.float32)


def parallel_inputs(shape: StageShape, seed: int | None = None) -> MMDiTInputs:
    """Layer weights of the parallel (Flux.1 single-stream) block, generator PCG64(shape.seed +
    4000), per layer in order: W_qkv [3h,h], b_qkv, W1 [rh,h], b1, W2 [h, h + rh], b2,
    W_ada [3h,h], b_ada [3h] (all N(0, w_std^2), matrices rounded to bf16 for bf16 shapes), then
    q_norm, k_norm [d] ~ 1 + N(0, 0.3^2).  No text-stream set; angles are rope_angles(shape).
    The stage input, condition and drift come from stage_inputs(shape) as for the DiT block."""
    rng = np.random.Generator(np.random.PCG64(shape.seed + 4000 if seed is None else seed))
    h, r, d = shape.hidden, shape.mlp_ratio, shape.head_dim
    shapes = {"w_qkv": (3 * h, h), "b_qkv": (3 * h,), "w1": (r * h, h), "b1": (r * h,), "w2": (h, h + r * h),
              "b2": (h,), "w_ada": (3 * h, h), "b_ada": (3 * h,)}
    std = np.float32(shape.w_std)
    layers = []
    for _ in range(shape.num_layers):
        lw = {}
        for name, shp in shapes.items():
            a = rng.standard_normal(shp, dtype=np.float32) * std
            if shape.dtype == "bf16" and name.startswith("w"):
                a = to_bf16_values(a)
            lw[name] = a
        lw["q_norm"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        lw["k_norm"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        layers.append(lw)
    return MMDiTInputs(layers, [], rope_angles(shape))


def batch_conds(shape: StageShape, c: np.ndarray, batch: int) -> np.ndarray:
    """Conditions of a batch of samples sharing the latent: sample 0 takes `c`; sample b >= 1
    (e.g. the unconditional half of a classifier-free guidance pair) an N(0, 1) vector of its own
    generator, PCG64(shape.seed + 7776 + b).  fp32 [batch, h]."""
    rows = [np.asarray(c, np.float32)] + [randn((shape.hidden,), shape.seed + 7776 + b) for b in range(1, batch)]
    return np.stack(rows)


@dataclasses.dataclass
class DenoiserInputs:
    weights: dict          # name -> fp32 ndarray (pf_denoiser_weights order)
    z: np.ndarray          # fp32 [batch, C, grid_h p, grid_w p]; a batch shares one latent
    y: np.ndarray          # fp32 [batch, h]: one condition embedding per sample
    grid_h: int
    grid_w: int


def denoiser_inputs(shape: StageShape, batch: int = 1, in_channels: int = 4, patch: int = 2, freq_dim: int = 256,
                    seed: int | None = None) -> DenoiserInputs:
    """Random weights of the loop around a stage (generator PCG64(shape.seed + 5000)), drawn in
    the order w_patch, b_patch, w_t1, b_t1, w_t2, b_t2, w_fada, b_fada, w_out, b_out, then z and y.
    Matrices ~ N(0, 1/fan_in) (w_fada ~ N(0, 0.02^2), as the blocks' adaLN), biases ~ N(0, 0.02^2),
    z and y ~ N(0, 1).  The patch grid is square: grid_h = grid_w = sqrt(seq_img)."""
    g = int(round(shape.seq_img ** 0.5))
    if g * g != shape.seq_img:
        raise ValueError("denoiser_inputs needs a square patch grid")
    rng = np.random.Generator(np.random.PCG64(shape.seed + 5000 if seed is None else seed))
    h, k = shape.hidden, in_channels * patch * patch
    dims = {"w_patch": (h, k), "b_patch": (h,), "w_t1": (h, freq_dim), "b_t1": (h,), "w_t2": (h, h), "b_t2": (h,),
            "w_fada": (2 * h, h), "b_fada": (2 * h,), "w_out": (k, h), "b_out": (k,)}
    w = {}
    for name, dim in dims.items():
        std = 0.02 if (name.startswith("b") or name == "w_fada") else 1.0 / np.sqrt(dim[1])
        w[name] = rng.standard_normal(dim, dtype=np.float32) * np.float32(std)
    z1 = rng.standard_normal((in_channels, g * patch, g * patch), dtype=np.float32)
    y = rng.standard_normal((batch, h), dtype=np.float32)
    return DenoiserInputs(w, np.stack([z1] * batch), y, g, g)


def randn(shape, seed: int, std: float = 1.0, bf16: bool = False) -> np.ndarray:
    """Plain seeded N(0, std^2) array (fp32), optionally rounded to bf16 values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return to_bf16_values(a) if bf16 else a


def rand_bits16(shape, seed: int) -> np.ndarray:
    """Seeded arbitrary 16-bit patterns that are finite bf16 values (for byte-copy tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = (a & 0x7F80) == 0x7F80          # inf/nan patterns -> clear one exponent bit
    a[exp_all_ones] &= np.uint16(0xBF7F)
    return a


def rand_bits32(shape, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
    bad = (a & 0x7F800000) == 0x7F800000
    a[bad] &= np.uint32(0xBF7FFFFF)
    return a
