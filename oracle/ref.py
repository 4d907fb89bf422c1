"""fp64 reference ("oracle") for one pipeline stage of patch-level DiT inference.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory; the
product path never does.  It shares no code with the HIP path: it is plain numpy
float64, slow and written to be checked by eye against the method.

What it computes (sources: the PipeFusion technical summaries on gist.science,
Korean page 1 and French page 4, "Core mechanisms" / "Mecanismes principaux"):

* Dual partitioning (mechanism 1): the stage owns L contiguous transformer
  layers; the token sequence is split into M non-overlapping patches that are
  pushed through those layers one patch at a time.
* Temporal redundancy (mechanism 2): attention of the current step T uses
  "stale" feature maps from step T+1 as context for the parts of the image not
  yet recomputed; a device starts computing on stale activations rather than
  waiting for fresh ones.
* Memory (mechanism 4): each device keeps full-spatial K and V only for its own
  layers, in one buffer per layer.
* The DiT keeps full (non-local) attention (Key contributions, first bullet).

Readings taken where the pages are silent (each listed in the design notes):
the block is a pre-LN adaLN-modulated DiT block with gated residuals, tanh GELU
MLP, LayerNorm eps 1e-6 without affine, biases present, attention scale
1/sqrt(d), non-causal, no mask; the KV buffer is updated in place, so when
patch m runs, rows of patches < m already hold step-T values, its own rows are
fresh and rows of later patches still hold step-(T+1) values; step 0 is a
warm-up that runs all rows as one patch; text-prefix rows (if any) run first as
their own micro-step in every step.

Three precision modes, all fp64 code:
* ``exact``: no intermediate rounding (the plain definition).
* ``bf16``: every tensor the bf16 path stores and feeds to a contraction is
  rounded to bf16 (round to nearest even): the modulated LayerNorm outputs,
  Q/K/V, the KV buffer after drift noise, the attention output and the GELU
  output.  Softmax probabilities are not rounded.
* ``bf16p``: ``bf16`` plus bf16 softmax probabilities, the operand of the
  probability-times-V contraction: the unnormalised weights 2^(s log2(e)) of
  the scaled scores s are rounded to bf16 relative to a power-of-two reference
  (the result does not depend on which power of two: rounding commutes with
  scaling by 2^k), and each row is normalised by the sum of the same rounded
  weights, so the normalised weights of a row sum to one.  It is the bf16-in /
  fp32-accumulate computation with P among the bf16 inputs; comparing it with
  ``bf16`` measures how far bf16 probabilities alone move a stage's output.

Parity status: every function below is pinned in the CPU test-suite by closed
forms, invariants, library special cases or brute force.  The choice of block
(LayerNorm / adaLN / GELU, which the pages do not define) is a reading, so the
block composition is "parity unpinned" with respect to the pages themselves.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Number format
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the fp32
    exponent range.  For |x| in [2^(e-1), 2^e) the spacing is 2^(e-8); below
    the smallest normal 2^-126 the spacing stays 2^-133 (subnormals).  Values
    beyond the largest finite bf16 become inf.  np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=F64)
    out = np.array(x, dtype=F64, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                       # xf = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(xf / q) * q
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


# ---------------------------------------------------------------------------
# Elementwise and row operations of the block
# ---------------------------------------------------------------------------

def layer_norm(x, eps: float = 1e-6) -> np.ndarray:
    """Row LayerNorm without affine: (x - mean) / sqrt(var + eps), biased variance."""
    x = np.asarray(x, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps)


def modulate(y, shift, scale) -> np.ndarray:
    """adaLN modulation: y * (1 + scale) + shift (per column)."""
    return np.asarray(y, F64) * (1.0 + np.asarray(scale, F64)) + np.asarray(shift, F64)


def silu(x) -> np.ndarray:
    x = np.asarray(x, F64)
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x) -> np.ndarray:
    """GELU, tanh approximation: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, F64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gelu_erf(x) -> np.ndarray:
    """GELU, exact form: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    from scipy.special import erf
    x = np.asarray(x, F64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x, w, b=None) -> np.ndarray:
    """nn.Linear convention: y = x @ w.T + b, w stored [out, in]."""
    y = np.asarray(x, F64) @ np.asarray(w, F64).T
    if b is not None:
        y = y + np.asarray(b, F64)
    return y


def adaln(c, w_ada, b_ada) -> np.ndarray:
    """Per-layer modulation vector: SiLU(c) @ W_ada.T + b_ada, returned as [k, h]: k = 6 for
    the DiT block (shift1, scale1, gate1, shift2, scale2, gate2), k = 3 for the parallel block
    (shift, scale, gate)."""
    m = linear(silu(c)[None, :], w_ada, b_ada)[0]
    return m.reshape(-1, np.asarray(w_ada).shape[1])


# ---------------------------------------------------------------------------
# Attention over the full-spatial buffer
# ---------------------------------------------------------------------------

def softmax_rows(s) -> np.ndarray:
    """Two-pass softmax along the last axis: subtract the row max, exponentiate, normalise."""
    s = np.asarray(s, F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v, heads: int, head_dim: int, chunk: int = 256, round_p: bool = False) -> np.ndarray:
    """Full non-causal multi-head attention of the rows of q over every row of k/v.

    Head j uses columns [j*d, (j+1)*d) of q, k and v.  O_j = softmax(Q_j K_j^T / sqrt(d)) V_j.
    Query rows are processed in chunks only to bound memory; each row's arithmetic is unchanged.
    round_p: bf16 probabilities.  With t = s log2(e) the scores in base-2 units, the weights
    w = bf16(2^(t - k)) for the integer k = ceil(max_row t) (any integer gives the same bits,
    barring underflow, since scaling by a power of two commutes with rounding) multiply V, and
    the row is normalised by sum(w), the sum of the same rounded weights.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    n = q.shape[0]
    out = np.empty((n, heads * head_dim), F64)
    scale = 1.0 / math.sqrt(head_dim)
    for j in range(heads):
        cs = slice(j * head_dim, (j + 1) * head_dim)
        kj = k[:, cs]
        vj = v[:, cs]
        for r0 in range(0, n, chunk):
            r1 = min(n, r0 + chunk)
            s = (q[r0:r1, cs] @ kj.T) * scale
            if round_p:
                t = s / math.log(2.0)
                w = bf16_round(np.exp2(t - np.ceil(t.max(axis=-1, keepdims=True))))
                out[r0:r1, cs] = (w @ vj) / w.sum(axis=-1, keepdims=True)
            else:
                out[r0:r1, cs] = softmax_rows(s) @ vj
    return out


# ---------------------------------------------------------------------------
# KV buffer splice
# ---------------------------------------------------------------------------

def rms_norm_heads(x, heads: int, head_dim: int, gamma, eps: float = 1e-6) -> np.ndarray:
    """Per-head RMSNorm of rows of x ([n, heads*d]): each head's d values divided by
    sqrt(mean of their squares + eps), times gamma [d] (shared by the heads)."""
    x = np.asarray(x, F64).reshape(-1, heads, head_dim)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return (x / r * np.asarray(gamma, F64)).reshape(-1, heads * head_dim)


def rope(x, heads: int, head_dim: int, angles) -> np.ndarray:
    """Rotary embedding of rows of x ([n, heads*d]) with per-row angles [n, d/2]: in every head,
    the pair (x[2k], x[2k+1]) is rotated by angles[row, k]."""
    x = np.asarray(x, F64).reshape(-1, heads, head_dim // 2, 2)
    a = np.asarray(angles, F64)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(x)
    out[..., 0] = x[..., 0] * c - x[..., 1] * s
    out[..., 1] = x[..., 0] * s + x[..., 1] * c
    return out.reshape(-1, heads * head_dim)


def splice(dst, src, offset: int):
    """In-place splice of a row block: dst[offset + i, :] = src[i, :] for i < len(src).

    Returns dst (same object).  Rows outside [offset, offset + len(src)) are untouched.
    Works on any dtype (byte-exact for integer views of bf16 / fp32 data).
    """
    n = src.shape[0]
    if offset < 0 or offset + n > dst.shape[0]:
        raise ValueError("splice out of range")
    dst[offset:offset + n, ...] = src
    return dst


# ---------------------------------------------------------------------------
# One pipeline stage
# ---------------------------------------------------------------------------

class StageOracle:
    """L contiguous layers of one stage with their per-layer full-spatial K/V buffers.

    layers: list of dicts with w_qkv [3h,h], b_qkv [3h], w_o [h,h], b_o [h], w1 [rh,h],
    b1 [rh], w2 [h,rh], b2 [h], w_ada [6h,h], b_ada [6h] (any float dtype), plus q_norm and
    k_norm [d] when qk_norm is set.

    Options of the MM-DiT block variants (SD3 / Flux; readings, the pages name the models only):
    * txt_layers: a second weight set of the same form for the text-prefix rows (dual stream);
      the text rows and the image rows then use their own projections, modulation and gates,
      and attention stays joint over every buffer row;
    * qk_norm: per-head RMSNorm of Q and K (after the projection, before RoPE) with the layer's
      (stream's) q_norm / k_norm scales;
    * rope_angles [seq_kv, d/2]: rotary embedding of Q and K, buffer row r's pairs turned by
      rope_angles[r];
    * parallel: the Flux.1 single-stream block, attention and MLP side by side on one modulated
      LayerNorm: h1 = LN(x) (1 + scale) + shift; Q, K, V = h1 W_qkv^T + b_qkv (then norm / rope,
      splice, attention -> o); u = GELU(h1 W1^T + b1); x += gate * ([o, u] W2^T + b2) with
      W2 [h, h + rh] (columns [0, h) act on o); w_ada is [3h, h] (shift, scale, gate) and
      w_o / b_o are not used.
    In bf16 mode Q and K are rounded after the projection and again after norm / rotation (the
    GPU stores them between the two).
    """

    def __init__(self, layers, *, heads: int, head_dim: int, seq_txt: int, seq_img: int,
                 num_patches: int, mlp_ratio: int, ln_eps: float = 1e-6, gelu: str = "tanh",
                 mode: str = "exact", txt_layers=None, qk_norm: bool = False, rope_angles=None,
                 parallel: bool = False):
        if mode not in ("exact", "bf16", "bf16p"):
            raise ValueError(mode)
        if seq_img % num_patches:
            raise ValueError("seq_img must be a multiple of num_patches")
        self.W = [{k: np.asarray(a, F64) for k, a in lw.items()} for lw in layers]
        self.Wt = None if txt_layers is None else [{k: np.asarray(a, F64) for k, a in lw.items()} for lw in txt_layers]
        self.qk_norm = qk_norm
        self.parallel = parallel
        self.rope_angles = None if rope_angles is None else np.asarray(rope_angles, F64)
        self.heads, self.head_dim = heads, head_dim
        self.hidden = heads * head_dim
        self.seq_txt, self.seq_img, self.num_patches = seq_txt, seq_img, num_patches
        self.seq_kv = seq_txt + seq_img
        self.patch_rows = seq_img // num_patches
        self.mlp_ratio = mlp_ratio
        self.ln_eps = ln_eps
        self.gelu = gelu_tanh if gelu == "tanh" else gelu_erf
        self.mode = mode
        self.K = [np.zeros((self.seq_kv, self.hidden), F64) for _ in self.W]
        self.V = [np.zeros((self.seq_kv, self.hidden), F64) for _ in self.W]
        self.mod = None
        self.mod_txt = None
        self.trace = None          # set to a list to record per-layer intermediates

    def _r(self, a):
        return a if self.mode == "exact" else bf16_round(a)

    def set_cond(self, c):
        self.mod = [adaln(c, W["w_ada"], W["b_ada"]) for W in self.W]
        if self.Wt is not None:
            self.mod_txt = [adaln(c, W["w_ada"], W["b_ada"]) for W in self.Wt]

    def _streams(self, rows_global):
        """Index arrays (into rows_global) of the text-stream rows and the image-stream rows."""
        rows_global = np.asarray(rows_global)
        if self.Wt is None:
            return [(np.arange(len(rows_global)), False)]
        txt = rows_global < self.seq_txt
        return [(np.nonzero(txt)[0], True), (np.nonzero(~txt)[0], False)]

    def run_rows(self, offset: int, rows: int, x, sample=None) -> np.ndarray:
        """Push buffer rows [offset, offset+rows) through every layer of the stage.

        In each layer the rows' fresh K/V are spliced into the layer's buffer before
        the rows attend over all seq_kv buffer rows (their own rows are therefore fresh).
        `sample` (indices into the rows) limits the last layer's attention and MLP to
        those rows and returns only their outputs; every buffer update is still complete.
        """
        if self.mod is None:
            raise RuntimeError("set_cond first")
        h, H, d = self.hidden, self.heads, self.head_dim
        x = np.array(x, F64).reshape(rows, h)
        rows_g = offset + np.arange(rows)
        for l in range(len(self.W)):
            def weights(txt):
                return (self.Wt[l], self.mod_txt[l]) if txt else (self.W[l], self.mod[l])
            q_all = np.empty((rows, h), F64)
            u_all = np.empty((rows, self.mlp_ratio * h), F64) if self.parallel else None
            rec = {"layer": l, "offset": offset, "h1": np.empty((rows, h)), "qkv": np.empty((rows, 3 * h))}
            for idx, txt in self._streams(rows_g):
                if len(idx) == 0:
                    continue
                W, mod = weights(txt)
                shift1, scale1 = mod[0], mod[1]
                h1 = self._r(modulate(layer_norm(x[idx], self.ln_eps), shift1, scale1))
                qkv = self._r(linear(h1, W["w_qkv"], W["b_qkv"]))
                q, k, v = qkv[:, :h], qkv[:, h:2 * h], qkv[:, 2 * h:]
                if self.qk_norm:
                    q = rms_norm_heads(q, H, d, W["q_norm"])
                    k = rms_norm_heads(k, H, d, W["k_norm"])
                if self.rope_angles is not None:
                    q = rope(q, H, d, self.rope_angles[rows_g[idx]])
                    k = rope(k, H, d, self.rope_angles[rows_g[idx]])
                if self.qk_norm or self.rope_angles is not None:
                    q, k = self._r(q), self._r(k)
                self.K[l][rows_g[idx]] = k
                self.V[l][rows_g[idx]] = v
                q_all[idx] = q
                rec["h1"][idx], rec["qkv"][idx] = h1, qkv
                if self.parallel and self.mlp_ratio > 0:
                    u_all[idx] = self._r(self.gelu(linear(h1, W["w1"], W["b1"])))
            sel = np.arange(rows)
            if sample is not None and l == len(self.W) - 1:
                sel = np.asarray(sample)
                x = x[sel]
            o = self._r(attention(q_all[sel], self.K[l], self.V[l], H, d, round_p=self.mode == "bf16p"))
            if self.parallel:
                ou = o if self.mlp_ratio == 0 else np.concatenate([o, u_all[sel]], axis=1)
                x_par = np.empty_like(x)
                for idx, txt in self._streams(rows_g[sel]):
                    if len(idx) == 0:
                        continue
                    W, mod = weights(txt)
                    x_par[idx] = x[idx] + mod[2] * linear(ou[idx], W["w2"], W["b2"])
                x = x_par
                rec.update(o=o, u=None if u_all is None else u_all[sel], x_out=x.copy())
                if self.trace is not None:
                    self.trace.append(rec)
                continue
            x_attn = np.empty_like(x)
            for idx, txt in self._streams(rows_g[sel]):
                if len(idx) == 0:
                    continue
                W, mod = weights(txt)
                x_attn[idx] = x[idx] + mod[2] * linear(o[idx], W["w_o"], W["b_o"])
            x = x_attn
            rec.update(o=o, x_attn=x.copy())
            if self.mlp_ratio > 0:
                x_mlp = np.empty_like(x)
                rec["h2"] = np.empty_like(x)
                rec["u"] = np.empty((x.shape[0], self.mlp_ratio * h))
                for idx, txt in self._streams(rows_g[sel]):
                    if len(idx) == 0:
                        continue
                    W, mod = weights(txt)
                    h2 = self._r(modulate(layer_norm(x[idx], self.ln_eps), mod[3], mod[4]))
                    u = self._r(self.gelu(linear(h2, W["w1"], W["b1"])))
                    x_mlp[idx] = x[idx] + mod[5] * linear(u, W["w2"], W["b2"])
                    rec["h2"][idx], rec["u"][idx] = h2, u
                x = x_mlp
            rec["x_out"] = x.copy()
            if self.trace is not None:
                self.trace.append(rec)
        return x

    def micro_steps(self, warmup: bool):
        """(offset, rows) of each micro-step of a step, in execution order."""
        if warmup:
            return [(0, self.seq_kv)]
        out = []
        if self.seq_txt > 0:
            out.append((0, self.seq_txt))
        for m in range(self.num_patches):
            out.append((self.seq_txt + m * self.patch_rows, self.patch_rows))
        return out

    def step(self, x_all, c, warmup: bool = False) -> np.ndarray:
        """One diffusion step of this stage over all seq_kv rows; returns the stage output."""
        self.set_cond(c)
        x_all = np.asarray(x_all, F64)
        out = np.empty((self.seq_kv, self.hidden), F64)
        for off, n in self.micro_steps(warmup):
            out[off:off + n] = self.run_rows(off, n, x_all[off:off + n])
        return out

    def step_sampled(self, x_all, c, rows_global, warmup: bool = False) -> np.ndarray:
        """Like step(), but returns only the outputs of the given buffer rows (sorted,
        unique); the buffers end in the same state as after step()."""
        self.set_cond(c)
        x_all = np.asarray(x_all, F64)
        rows_global = np.asarray(rows_global)
        out = np.empty((len(rows_global), self.hidden), F64)
        for off, n in self.micro_steps(warmup):
            sel = np.nonzero((rows_global >= off) & (rows_global < off + n))[0]
            res = self.run_rows(off, n, x_all[off:off + n], sample=rows_global[sel] - off)
            out[sel] = res
        return out

    def add_noise(self, noise):
        """Step boundary: every stale K/V value drifts by the given per-layer noise."""
        for l, (nk, nv) in enumerate(noise):
            self.K[l] = self._r(self.K[l] + np.asarray(nk, F64))
            self.V[l] = self._r(self.V[l] + np.asarray(nv, F64))
