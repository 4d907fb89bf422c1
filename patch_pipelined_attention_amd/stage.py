"""Python handle over one libpf stage (memory plumbing around the C ABI).

`Stage` creates the native stage, uploads a layer set, runs steps and patches,
and moves KV-buffer contents between the stage and host arrays.  All data
movement into and out of the stage's buffers goes through `kvbuf_splice`
(into / out of torch-allocated buffers), so no pointer arithmetic happens here.
Nothing in this module computes any part of the stage.
"""
from __future__ import annotations

import numpy as np

from . import binding as B
from .configs import StageShape


def _torch():
    import torch
    return torch


def k8_to_rows(flat: np.ndarray, rows: int, row_elems: int) -> np.ndarray:
    """Host view of a PF_LAYOUT_K8 matrix as [rows, row_elems] (layout change only)."""
    g = (rows + 7) // 8
    return flat[: g * 8 * row_elems].reshape(g, row_elems, 8).transpose(0, 2, 1).reshape(g * 8, row_elems)[:rows]


def rows_to_k8(a: np.ndarray) -> np.ndarray:
    """[rows, row_elems] -> flat PF_LAYOUT_K8 storage (rows padded to a multiple of 8 with zeros)."""
    rows, e = a.shape
    g = (rows + 7) // 8
    pad = np.zeros((g * 8, e), a.dtype)
    pad[:rows] = a
    return np.ascontiguousarray(pad.reshape(g, 8, e).transpose(0, 2, 1)).reshape(-1)


def parallel_block(lw) -> bool:
    """Layer dict of the parallel block (no out-projection of its own)."""
    return "w_o" not in lw


class Stage:
    """`batch` > 1: samples sharing the weights (a classifier-free guidance pair is 2); x is
    then [batch, rows, h] and cond [batch, h], and each sample has its own K/V buffers.

    MM-DiT block options (bf16 stages): qk_norm (per-head RMSNorm of Q and K; each layer dict
    then holds q_norm and k_norm [d]), dual_stream (the text rows use the layer dicts given as
    `txt_layers` to load()), rope (rotation angles given to set_rope()) and parallel (the Flux.1
    single-stream block; layer dicts as synth.parallel_inputs draws them)."""

    def __init__(self, shape: StageShape, gelu: str = "tanh", ln_eps: float = 1e-6, batch: int = 1,
                 qk_norm: bool = False, dual_stream: bool = False, rope: bool = False, parallel: bool = False):
        torch = _torch()
        self.shape = shape
        self.batch = batch
        self.dtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        self.pf_dtype = B.PF_BF16 if shape.dtype == "bf16" else B.PF_FP32
        cfg = B.StageConfig(num_layers=shape.num_layers, hidden=shape.hidden, heads=shape.heads,
                            head_dim=shape.head_dim, mlp_ratio=shape.mlp_ratio, num_patches=shape.num_patches,
                            seq_img=shape.seq_img, seq_txt=shape.seq_txt, dtype=self.pf_dtype,
                            gelu=B.PF_GELU_TANH if gelu == "tanh" else B.PF_GELU_ERF, ln_eps=ln_eps,
                            flags=(B.PF_STAGE_QK_NORM if qk_norm else 0) | (B.PF_STAGE_DUAL_STREAM if dual_stream else 0)
                            | (B.PF_STAGE_ROPE if rope else 0) | (B.PF_STAGE_PARALLEL if parallel else 0),
                            batch=batch)
        self.handle = B.stage_create(cfg)
        self.v_layout = B.PF_LAYOUT_K8 if self.pf_dtype == B.PF_BF16 else B.PF_LAYOUT_ROWS

    # ------------------------------------------------------------------ lifecycle
    def close(self):
        if self.handle is not None:
            _torch().cuda.synchronize()
            B.stage_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ weights
    def load(self, layers, txt_layers=None):
        """layers (and, for a dual-stream stage, txt_layers): lists of dicts of host fp32 arrays
        (synth.StageInputs.layers); matrices go to the stage dtype, vectors stay fp32."""
        torch = _torch()
        keep = []
        for sets, loader in ((layers, B.stage_load_weights), (txt_layers or [], B.stage_load_text_weights)):
            for l, lw in enumerate(sets):
                dev = {}
                for name, a in lw.items():
                    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
                    dt = self.dtype if name.startswith("w") else torch.float32
                    dev[name] = t.to(device="cuda", dtype=dt)
                if self.shape.mlp_ratio == 0:
                    for n in ("w1", "b1") if parallel_block(lw) else ("w1", "b1", "w2", "b2"):
                        dev[n] = None
                loader(self.handle, l, dev)
                keep.append(dev)
        torch.cuda.synchronize()
        del keep

    def set_rope(self, angles):
        """angles: host array [seq_kv, head_dim / 2] (radians; row r turns buffer row r)."""
        torch = _torch()
        t = torch.from_numpy(np.ascontiguousarray(angles, np.float32)).to("cuda")
        B.stage_set_rope(self.handle, t)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ runs
    def run_step(self, x, cond, warmup: bool = False, out=None):
        out = x if out is None else out
        B.stage_run_step(self.handle, x, out, cond, warmup=warmup)
        return out

    def set_cond(self, cond):
        B.stage_set_cond(self.handle, cond)

    def run_patch(self, row_off: int, rows: int, x_in, x_out=None):
        x_out = x_in if x_out is None else x_out
        B.stage_run_patch(self.handle, row_off, rows, x_in, x_out)
        return x_out

    # ------------------------------------------------------------------ KV buffers
    def kv_view(self, layer: int, sample: int = 0) -> B.KVView:
        return B.stage_get_kvbuf(self.handle, layer, sample)

    def _scratch_pair(self):
        torch = _torch()
        s, h = self.shape.seq_kv, self.shape.hidden
        g = (s + 7) // 8
        k = torch.empty((s, h), dtype=self.dtype, device="cuda")
        v = torch.empty((g * 8 * h,) if self.v_layout == B.PF_LAYOUT_K8 else (s, h), dtype=self.dtype, device="cuda")
        view = B.kv_view(k, v, s, h, self.v_layout)
        return k, v, view

    def kv_raw(self, layer: int, sample: int = 0):
        """Device copies (torch) of layer's K ([S,h]) and V (storage layout) buffers."""
        k, v, view = self._scratch_pair()
        B.kvbuf_splice(view, self.kv_view(layer, sample), 0, self.shape.seq_kv)
        return k, v

    def kv_get(self, layer: int, sample: int = 0):
        """Host fp32 arrays [S, h] of layer's K and V (logical rows)."""
        torch = _torch()
        k, v = self.kv_raw(layer, sample)
        torch.cuda.synchronize()
        kh = k.float().cpu().numpy()
        vh = v.float().cpu().numpy()
        if self.v_layout == B.PF_LAYOUT_K8:
            vh = k8_to_rows(vh, self.shape.seq_kv, self.shape.hidden)
        return kh, vh

    def kv_set(self, layer: int, k_rows: np.ndarray, v_rows: np.ndarray, sample: int = 0):
        """Overwrite layer's whole K/V buffer from host arrays (rounded to the stage dtype by torch)."""
        torch = _torch()
        kt = torch.from_numpy(np.ascontiguousarray(k_rows, np.float32)).to(device="cuda", dtype=self.dtype)
        vv = rows_to_k8(np.asarray(v_rows, np.float32)) if self.v_layout == B.PF_LAYOUT_K8 else v_rows
        vt = torch.from_numpy(np.ascontiguousarray(vv, np.float32)).to(device="cuda", dtype=self.dtype)
        view = B.kv_view(kt, vt, self.shape.seq_kv, self.shape.hidden, self.v_layout)
        B.kvbuf_splice(self.kv_view(layer, sample), view, 0, self.shape.seq_kv)
        torch.cuda.synchronize()

    def add_noise(self, noise, sample: int = 0):
        """Step boundary drift: K += nk, V += nv for every layer (fp32 add, then stage dtype)."""
        for l, (nk, nv) in enumerate(noise):
            k, v = self.kv_get(l, sample)
            self.kv_set(l, k + nk, v + nv, sample)
