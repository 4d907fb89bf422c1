"""Pure-Python loop restatement of the denoising loop around a stage, for tiny grids.

TEST INFRASTRUCTURE ONLY (see oracle/ref.py).  It restates oracle/sampler.py's
DenoiserOracle step by step with explicit loops, math.fsum and the brute-force stage
(oracle/brute.py), sharing none of sampler.py's helpers, so that a swapped operand, a
wrong index or a swapped role in either one shows up as a mismatch.

The loop (PipeFusion summaries, Korean page 1 and French page 4, "Core mechanisms" 2:
the stage sits inside a diffusion loop whose consecutive steps see similar inputs; the
loop itself is a DiT reading, listed with the design notes):
  c_b   = W_t2 SiLU(W_t1 [cos(t f_j)..., sin(t f_j)...] + b_t1) + b_t2 + y_b,  f_j = 10000^(-j/half)
  x_b   = [x_txt_b; W_patch patch_s(z_b) + b_patch + pos_s]  (patch values (c p + dy) p + dx)
  out_b = the stage step on x_b with condition c_b
  eps_b = unpatchify(W_out (LN(out_b) (1 + scale_b) + shift_b) + b_out),
          (shift_b, scale_b) = the two halves of W_fada SiLU(c_b) + b_fada
  pair:   eps = eps_1 + g (eps_0 - eps_1) for both samples (0 conditional, 1 unconditional)
  DDIM:   z' = sqrt(abar_n) (z - sqrt(1 - abar_t) eps) / sqrt(abar_t) + sqrt(1 - abar_n) eps
"""
from __future__ import annotations

import math

from . import brute


def _silu(a):
    return a / (1.0 + math.exp(-a))


def _mv(w, x, b):
    return [math.fsum(w[j][i] * x[i] for i in range(len(x))) + b[j] for j in range(len(w))]


def abar_table(train_steps, beta_start, beta_end):
    """abar_t = prod_{i <= t} (1 - beta_i), betas evenly spaced from beta_start to beta_end."""
    out, acc = [], 1.0
    for i in range(train_steps):
        beta = beta_start + (beta_end - beta_start) * i / (train_steps - 1)
        acc *= 1.0 - beta
        out.append(acc)
    return out


def condition(w, t, y, freq_dim):
    half = freq_dim // 2
    feats = [0.0] * freq_dim
    for j in range(half):
        f = 10000.0 ** (-j / half)
        feats[j] = math.cos(t * f)
        feats[half + j] = math.sin(t * f)
    th = [_silu(a) for a in _mv(w["w_t1"], feats, w["b_t1"])]
    temb = _mv(w["w_t2"], th, w["b_t2"])
    return [temb[i] + y[i] for i in range(len(y))]


def position_row(gy, gx, hidden):
    q = hidden // 4
    row = [0.0] * hidden
    for k in range(q):
        wk = 10000.0 ** (-k / q)
        row[k] = math.sin(gy * wk)
        row[q + k] = math.cos(gy * wk)
        row[2 * q + k] = math.sin(gx * wk)
        row[3 * q + k] = math.cos(gx * wk)
    return row


def embed(w, z, p, hidden):
    """Rows of the image tokens of one sample's latent z [C][H][W] (nested lists)."""
    C, gh, gw = len(z), len(z[0]) // p, len(z[0][0]) // p
    rows = []
    for gy in range(gh):
        for gx in range(gw):
            vec = [0.0] * (C * p * p)
            for c in range(C):
                for dy in range(p):
                    for dx in range(p):
                        vec[(c * p + dy) * p + dx] = z[c][gy * p + dy][gx * p + dx]
            e = _mv(w["w_patch"], vec, w["b_patch"])
            pos = position_row(gy, gx, hidden)
            rows.append([e[i] + pos[i] for i in range(hidden)])
    return rows


def noise_prediction(w, out_img, c, C, p, gh, gw, eps_ln=1e-6):
    """eps [C][gh p][gw p] from the stage's image-row outputs."""
    h = len(c)
    mod = _mv(w["w_fada"], [_silu(a) for a in c], w["b_fada"])
    shift, scale = mod[:h], mod[h:2 * h]
    eps = [[[0.0] * (gw * p) for _ in range(gh * p)] for _ in range(C)]
    for s, row in enumerate(out_img):
        n = brute.layer_norm_row(row, eps_ln)
        hf = [n[i] * (1.0 + scale[i]) + shift[i] for i in range(h)]
        v = _mv(w["w_out"], hf, w["b_out"])
        gy, gx = divmod(s, gw)
        for ch in range(C):
            for dy in range(p):
                for dx in range(p):
                    eps[ch][gy * p + dy][gx * p + dx] = v[(ch * p + dy) * p + dx]
    return eps


def denoise_step(w, layers, kbufs, vbufs, z, y, t, t_next, abar, *, heads, d, seq_txt, num_patches, mlp_ratio,
                 patch, freq_dim, warmup, guidance=1.0, x_txt=None):
    """One step for every sample b (z[b] nested [C][H][W], y[b] [h]); kbufs[b] / vbufs[b]
    are sample b's per-layer buffers (updated in place).  Returns (z', eps)."""
    nb = len(z)
    C, p = len(z[0]), patch
    gh, gw = len(z[0][0]) // p, len(z[0][0][0]) // p
    hidden = heads * d
    eps = []
    for b in range(nb):
        c = condition(w, t, y[b], freq_dim)
        x_all = ([list(r) for r in x_txt[b]] if seq_txt else []) + embed(w, z[b], p, hidden)
        out = brute.stage_step(layers, kbufs[b], vbufs[b], x_all, c, heads=heads, d=d, seq_txt=seq_txt,
                               num_patches=num_patches, mlp_ratio=mlp_ratio, warmup=warmup)
        eps.append(noise_prediction(w, out[seq_txt:], c, C, p, gh, gw))
    if nb == 2:
        e0, e1 = eps
        g = [[[e1[ch][i][j] + guidance * (e0[ch][i][j] - e1[ch][i][j]) for j in range(len(e0[0][0]))]
              for i in range(len(e0[0]))] for ch in range(C)]
        eps = [g, g]
    a_t = abar[t]
    a_n = abar[t_next] if t_next >= 0 else 1.0
    z_new = []
    for b in range(nb):
        zb = [[[0.0] * len(z[b][0][0]) for _ in range(len(z[b][0]))] for _ in range(C)]
        for ch in range(C):
            for i in range(len(z[b][0])):
                for j in range(len(z[b][0][0])):
                    e = eps[b][ch][i][j]
                    x0 = (z[b][ch][i][j] - math.sqrt(1.0 - a_t) * e) / math.sqrt(a_t)
                    zb[ch][i][j] = math.sqrt(a_n) * x0 + math.sqrt(1.0 - a_n) * e
        z_new.append(zb)
    return z_new, eps
