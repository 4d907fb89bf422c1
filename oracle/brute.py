"""Pure-Python brute-force restatement of the stage for tiny sizes (S <= 16, h <= 8).

TEST INFRASTRUCTURE ONLY (see oracle/ref.py).  Written with explicit loops,
math.exp and math.fsum, independently of the numpy oracle, so that an indexing,
transposition or scaling slip in either one shows up as a mismatch.  Same
readings as oracle/ref.py: pre-LN adaLN block, gated residuals, tanh GELU MLP,
1/sqrt(d) attention scale, in-place K/V splice before attention, ascending patch
order after an optional text prefix (PipeFusion summaries, mechanisms 1, 2, 4).
"""
from __future__ import annotations

import math


def matvec_rows(x, w, b):
    """rows of x times w^T (w is [out][in]) plus b, by loops."""
    out = []
    for row in x:
        o = []
        for j in range(len(w)):
            o.append(math.fsum(row[i] * w[j][i] for i in range(len(row))) + (b[j] if b is not None else 0.0))
        out.append(o)
    return out


def layer_norm_row(row, eps):
    n = len(row)
    mean = math.fsum(row) / n
    var = math.fsum((a - mean) ** 2 for a in row) / n
    return [(a - mean) / math.sqrt(var + eps) for a in row]


def attention(q, k, v, heads, d):
    """q: list of query rows, k/v: list of buffer rows (python lists of floats)."""
    out = []
    for qi in q:
        orow = [0.0] * (heads * d)
        for j in range(heads):
            scores = []
            for kr in k:
                scores.append(math.fsum(qi[j * d + t] * kr[j * d + t] for t in range(d)) / math.sqrt(d))
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = math.fsum(e)
            for t in range(d):
                orow[j * d + t] = math.fsum(e[i] * k_v[j * d + t] for i, k_v in enumerate(v)) / z
        out.append(orow)
    return out


def gelu_tanh(a):
    return 0.5 * a * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a * a * a)))


def silu(a):
    return a / (1.0 + math.exp(-a))


def rms_heads_row(row, heads, d, gamma, eps=1e-6):
    out = []
    for j in range(heads):
        seg = row[j * d:(j + 1) * d]
        r = math.sqrt(math.fsum(a * a for a in seg) / d + eps)
        out.extend(seg[i] / r * gamma[i] for i in range(d))
    return out


def rope_row(row, heads, d, angles):
    out = list(row)
    for j in range(heads):
        for k in range(d // 2):
            a0, a1 = row[j * d + 2 * k], row[j * d + 2 * k + 1]
            cs, sn = math.cos(angles[k]), math.sin(angles[k])
            out[j * d + 2 * k] = a0 * cs - a1 * sn
            out[j * d + 2 * k + 1] = a0 * sn + a1 * cs
    return out


def stage_step(layers, kbuf, vbuf, x_all, c, *, heads, d, seq_txt, num_patches, mlp_ratio,
               warmup, eps=1e-6, txt_layers=None, qk_norm=False, rope_angles=None, parallel=False):
    """One step over all rows; kbuf/vbuf (lists of per-layer row lists) are updated in place.
    txt_layers: weights of the text-prefix rows (dual stream); qk_norm: per-head RMSNorm of Q
    and K with the row's weights' q_norm / k_norm; rope_angles: per buffer row, d/2 angles;
    parallel: attention and MLP on the same modulated row, x += gate * W2 [o, u] + b2."""
    h = heads * d
    S = len(x_all)

    def mods_of(ws):
        out = []
        for W in ws:
            sc = [silu(a) for a in c]
            m = matvec_rows([sc], W["w_ada"], W["b_ada"])[0]
            out.append([m[i * h:(i + 1) * h] for i in range(len(m) // h)])
        return out
    mods = mods_of(layers)
    mods_t = mods_of(txt_layers) if txt_layers is not None else None
    if warmup:
        micro = [(0, S)]
    else:
        P = (S - seq_txt) // num_patches
        micro = ([(0, seq_txt)] if seq_txt else []) + [(seq_txt + m * P, P) for m in range(num_patches)]
    out = [None] * S
    for off, n in micro:
        x = [list(r) for r in x_all[off:off + n]]
        for l in range(len(layers)):
            # every row on its own, with the weights and modulation of its stream
            def wm(i):
                if txt_layers is not None and off + i < seq_txt:
                    return txt_layers[l], mods_t[l]
                return layers[l], mods[l]
            qs, us = [], []
            for i in range(n):
                W, md = wm(i)
                sh1, sc1 = md[0], md[1]
                h1 = [a * (1.0 + sc1[t]) + sh1[t] for t, a in enumerate(layer_norm_row(x[i], eps))]
                if parallel:
                    us.append([gelu_tanh(a) for a in matvec_rows([h1], W["w1"], W["b1"])[0]] if mlp_ratio else [])
                qkv = matvec_rows([h1], W["w_qkv"], W["b_qkv"])[0]
                q, k = qkv[:h], qkv[h:2 * h]
                if qk_norm:
                    q, k = rms_heads_row(q, heads, d, W["q_norm"], eps), rms_heads_row(k, heads, d, W["k_norm"], eps)
                if rope_angles is not None:
                    q, k = rope_row(q, heads, d, rope_angles[off + i]), rope_row(k, heads, d, rope_angles[off + i])
                kbuf[l][off + i] = k
                vbuf[l][off + i] = qkv[2 * h:3 * h]
                qs.append(q)
            o = attention(qs, kbuf[l], vbuf[l], heads, d)
            for i in range(n):
                W, md = wm(i)
                if parallel:
                    y = matvec_rows([list(o[i]) + us[i]], W["w2"], W["b2"])[0]
                    x[i] = [x[i][t] + md[2][t] * y[t] for t in range(h)]
                    continue
                g1, sh2, sc2, g2 = md[2], md[3], md[4], md[5]
                y = matvec_rows([o[i]], W["w_o"], W["b_o"])[0]
                xi = [x[i][t] + g1[t] * y[t] for t in range(h)]
                if mlp_ratio > 0:
                    h2 = [a * (1.0 + sc2[t]) + sh2[t] for t, a in enumerate(layer_norm_row(xi, eps))]
                    u = [gelu_tanh(a) for a in matvec_rows([h2], W["w1"], W["b1"])[0]]
                    y2 = matvec_rows([u], W["w2"], W["b2"])[0]
                    xi = [xi[t] + g2[t] * y2[t] for t in range(h)]
                x[i] = xi
        for i in range(n):
            out[off + i] = x[i]
    return out
