"""fp64 reference ("oracle") for the denoising loop around a pipeline stage.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import or run this module; the
product path never does.  It shares no code with the HIP path: plain numpy float64.

What it computes.  The PipeFusion summaries (gist.science, Korean page 1 and French page
4, "Core mechanisms" 2) place the stage inside a diffusion loop: consecutive steps see
similar inputs, so a step's stale K/V from step T+1 serve as context at step T, and the
pipeline keeps running without bubbles apart from its start-up (the warm-up).  The pages do
not define the loop itself; the plainest DiT reading is taken and listed in the design notes:

* condition c = MLP(sinusoid(t)) + y: a 2-layer timestep MLP (Linear, SiLU, Linear) on the
  [cos, sin] frequency features of t (frequencies 10000^(-k / half)), plus a given
  condition embedding y (the pooled class / text embedding, an input here);
* patch embedding: non-overlapping p x p patches of the latent, row-major over the patch
  grid, flattened channel-major ((c * p + dy) * p + dx), then a linear map, a bias and a
  fixed 2-D sine-cosine position embedding (first half of the width from the patch row,
  second half from the patch column; each half [sin(pos w_k), cos(pos w_k)] with
  w_k = 10000^(-k / (h/4)));
* the stage (oracle.ref.StageOracle) over [text rows, image rows];
* final layer: adaLN (shift, scale) = SiLU(c) W_f^T + b_f, LayerNorm + modulation of the
  image rows, a linear map to p*p*C values per patch, unpatchify -> noise prediction eps;
* classifier-free guidance for a pair (sample 0 conditional, sample 1 unconditional):
  eps = eps_1 + g (eps_0 - eps_1), applied to both samples, which share the latent;
* DDIM update (eta = 0) with a linear beta schedule over T training steps:
  x0 = (z - sqrt(1 - abar_t) eps) / sqrt(abar_t);  z' = sqrt(abar_s) x0 + sqrt(1 - abar_s) eps
  where s is the next (smaller) timestep, and abar of "no next step" is 1.

Pins (tests/test_sampler_oracle.py): closed forms of the sinusoids at position 0, the DDIM
step on an exactly predicted noise, patchify against torch's conv2d, the unpatchify
round trip by brute force, the guidance limits g = 0 and g = 1, and the schedule's first
value and monotonicity.  The loop as a whole (condition, eps, step) is pinned against the
independent loop restatement oracle/brute_sampler.py over three steps (one sample; a guided
pair with a text prefix), by two special cases of the final layer (W_fada = 0 with a zero
and with a constant [shift; scale] bias) and by the guidance roles (g = 1 gives both samples
the conditional prediction, g = 0 the unconditional one); a planted shift/scale swap and a
planted swap of the guidance roles fail those pins.
"""
from __future__ import annotations

import math

import numpy as np

from . import ref

F64 = np.float64


silu = ref.silu


def timestep_features(t: float, dim: int) -> np.ndarray:
    """[cos(t f_0) .. cos(t f_{half-1}), sin(t f_0) .. sin(t f_{half-1})], f_k = 10000^(-k/half)."""
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=F64) / half)
    a = float(t) * f
    return np.concatenate([np.cos(a), np.sin(a)])


def pos_embed_2d(grid_h: int, grid_w: int, hidden: int) -> np.ndarray:
    """[grid_h * grid_w, hidden] fixed sine-cosine position embedding (see module notes)."""
    q = hidden // 4
    w = 10000.0 ** (-np.arange(q, dtype=F64) / q)
    out = np.empty((grid_h * grid_w, hidden), F64)
    for gy in range(grid_h):
        for gx in range(grid_w):
            s = gy * grid_w + gx
            out[s, 0:q] = np.sin(gy * w)
            out[s, q:2 * q] = np.cos(gy * w)
            out[s, 2 * q:3 * q] = np.sin(gx * w)
            out[s, 3 * q:4 * q] = np.cos(gx * w)
    return out


def patchify(z: np.ndarray, p: int) -> np.ndarray:
    """z [C, H, W] -> [(H/p)(W/p), C p p]; patch s = gy * (W/p) + gx, value (c * p + dy) * p + dx."""
    c, hh, ww = z.shape
    gh, gw = hh // p, ww // p
    return (np.asarray(z, F64).reshape(c, gh, p, gw, p).transpose(1, 3, 0, 2, 4).reshape(gh * gw, c * p * p))


def unpatchify(v: np.ndarray, c: int, p: int, gh: int, gw: int) -> np.ndarray:
    """Inverse of patchify: [gh * gw, c p p] -> [c, gh p, gw p]."""
    return np.asarray(v, F64).reshape(gh, gw, c, p, p).transpose(2, 0, 3, 1, 4).reshape(c, gh * p, gw * p)


def alphas_cumprod(train_steps: int, beta_start: float, beta_end: float) -> np.ndarray:
    """abar_t = prod_{i <= t} (1 - beta_i), beta linear from beta_start to beta_end."""
    betas = np.linspace(beta_start, beta_end, train_steps, dtype=F64)
    return np.cumprod(1.0 - betas)


def ddim_step(z, eps, abar_t: float, abar_next: float):
    x0 = (np.asarray(z, F64) - math.sqrt(1.0 - abar_t) * eps) / math.sqrt(abar_t)
    return math.sqrt(abar_next) * x0 + math.sqrt(1.0 - abar_next) * eps


def guide(eps_cond, eps_uncond, g: float):
    return eps_uncond + g * (eps_cond - eps_uncond)


class DenoiserOracle:
    """The loop for `batch` samples (1, or 2 = a guidance pair), each with its own stage
    oracle (own K/V buffers) and the shared weights `w` (dict of fp64-convertible arrays:
    w_patch [h, C p p], b_patch [h], w_t1 [h, F], b_t1, w_t2 [h, h], b_t2, w_fada [2h, h],
    b_fada [2h], w_out [C p p, h], b_out [C p p])."""

    def __init__(self, stages, w, in_channels: int, patch: int, grid_h: int, grid_w: int, freq_dim: int,
                 abar: np.ndarray, seq_txt: int = 0, ln_eps: float = 1e-6):
        self.stages = list(stages)
        self.w = {k: np.asarray(v, F64) for k, v in w.items()}
        self.c, self.p, self.gh, self.gw = in_channels, patch, grid_h, grid_w
        self.freq_dim, self.abar, self.seq_txt, self.ln_eps = freq_dim, abar, seq_txt, ln_eps
        self.hidden = self.w["w_t2"].shape[0]
        self.pos = pos_embed_2d(grid_h, grid_w, self.hidden)

    def condition(self, t: float, y: np.ndarray) -> np.ndarray:
        w = self.w
        tf = timestep_features(t, self.freq_dim)
        th = silu(ref.linear(tf[None], w["w_t1"], w["b_t1"]))
        temb = ref.linear(th, w["w_t2"], w["b_t2"])[0]
        return temb[None] + np.asarray(y, F64)

    def eps(self, z_b, y_b, c_b, stage, warmup, x_txt=None):
        w = self.w
        x_img = ref.linear(patchify(z_b, self.p), w["w_patch"], w["b_patch"]) + self.pos
        x_all = x_img if self.seq_txt == 0 else np.concatenate([np.asarray(x_txt, F64), x_img])
        out = stage.step(x_all, c_b, warmup=warmup)[self.seq_txt:]
        mod = ref.linear(silu(c_b)[None], w["w_fada"], w["b_fada"])[0]
        hsz = self.hidden
        hf = ref.modulate(ref.layer_norm(out, self.ln_eps), mod[:hsz], mod[hsz:])
        v = ref.linear(hf, w["w_out"], w["b_out"])
        return unpatchify(v, self.c, self.p, self.gh, self.gw)

    def step(self, z, y, t: int, t_next: int, warmup: bool, guidance: float = 1.0, x_txt=None):
        """z: [batch, C, H, W] (a pair shares its latent), y: [batch, h].  Returns (z', eps)."""
        c = self.condition(t, y)
        eps = [self.eps(z[b], y[b], c[b], self.stages[b], warmup, None if x_txt is None else x_txt[b])
               for b in range(len(self.stages))]
        if len(eps) == 2:
            g = guide(eps[0], eps[1], guidance)
            eps = [g, g]
        abar_t = float(self.abar[t])
        abar_n = float(self.abar[t_next]) if t_next >= 0 else 1.0
        z_new = np.stack([ddim_step(z[b], eps[b], abar_t, abar_n) for b in range(len(eps))])
        return z_new, np.stack(eps)
