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


def stage_step(layers, kbuf, vbuf, x_all, c, *, heads, d, seq_txt, num_patches, mlp_ratio,
               warmup, eps=1e-6):
    """One step over all rows; kbuf/vbuf (lists of per-layer row lists) are updated in place."""
    h = heads * d
    S = len(x_all)
    mods = []
    for W in layers:
        sc = [silu(a) for a in c]
        m = matvec_rows([sc], W["w_ada"], W["b_ada"])[0]
        mods.append([m[i * h:(i + 1) * h] for i in range(6)])
    if warmup:
        micro = [(0, S)]
    else:
        P = (S - seq_txt) // num_patches
        micro = ([(0, seq_txt)] if seq_txt else []) + [(seq_txt + m * P, P) for m in range(num_patches)]
    out = [None] * S
    for off, n in micro:
        x = [list(r) for r in x_all[off:off + n]]
        for l, W in enumerate(layers):
            sh1, sc1, g1, sh2, sc2, g2 = mods[l]
            h1 = [[a * (1.0 + sc1[i]) + sh1[i] for i, a in enumerate(layer_norm_row(r, eps))] for r in x]
            qkv = matvec_rows(h1, W["w_qkv"], W["b_qkv"])
            for i in range(n):
                kbuf[l][off + i] = qkv[i][h:2 * h]
                vbuf[l][off + i] = qkv[i][2 * h:3 * h]
            o = attention([r[:h] for r in qkv], kbuf[l], vbuf[l], heads, d)
            y = matvec_rows(o, W["w_o"], W["b_o"])
            x = [[x[i][t] + g1[t] * y[i][t] for t in range(h)] for i in range(n)]
            if mlp_ratio > 0:
                h2 = [[a * (1.0 + sc2[i]) + sh2[i] for i, a in enumerate(layer_norm_row(r, eps))] for r in x]
                u = [[gelu_tanh(a) for a in r] for r in matvec_rows(h2, W["w1"], W["b1"])]
                y2 = matvec_rows(u, W["w2"], W["b2"])
                x = [[x[i][t] + g2[t] * y2[i][t] for t in range(h)] for i in range(n)]
        for i in range(n):
            out[off + i] = x[i]
    return out
