"""ctypes binding of libpf (include/pf.h): same names as the C entry points.

Argument marshalling only: torch tensors provide device memory (``data_ptr()``)
and the HIP stream (``torch.cuda.current_stream().cuda_stream``); every step of
the stage runs in the library's HIP kernels.  The library is loaded on first use
and its absence is an error (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpf.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pf.h")

PF_OK, PF_ERR_INVALID_ARG, PF_ERR_UNSUPPORTED, PF_ERR_OOM, PF_ERR_STATE, PF_ERR_HIP = range(6)
PF_BF16, PF_FP32 = 0, 1
PF_GELU_TANH, PF_GELU_ERF = 0, 1
PF_LAYOUT_ROWS, PF_LAYOUT_K8 = 0, 1
PF_EPI_STORE, PF_EPI_GELU_TANH, PF_EPI_GELU_ERF, PF_EPI_GATED_RESIDUAL = range(4)
PF_STEP_WARMUP = 1
PF_STAGE_QK_NORM, PF_STAGE_DUAL_STREAM, PF_STAGE_ROPE, PF_STAGE_PARALLEL = 1, 2, 4, 8

STATUS_NAMES = {0: "PF_OK", 1: "PF_ERR_INVALID_ARG", 2: "PF_ERR_UNSUPPORTED", 3: "PF_ERR_OOM",
                4: "PF_ERR_STATE", 5: "PF_ERR_HIP"}


class PFError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class StageConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("mlp_ratio", ctypes.c_int32), ("num_patches", ctypes.c_int32),
                ("seq_img", ctypes.c_int64), ("seq_txt", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("gelu", ctypes.c_int32), ("ln_eps", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("batch", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2", "w_ada", "b_ada", "q_norm", "k_norm")]


class KVView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("row_elems", ctypes.c_int64), ("k_ld", ctypes.c_int64), ("v_ld", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("v_layout", ctypes.c_int32)]


class DenoiserConfig(ctypes.Structure):
    _fields_ = [("in_channels", ctypes.c_int32), ("patch", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("freq_dim", ctypes.c_int32), ("train_steps", ctypes.c_int32),
                ("beta_start", ctypes.c_float), ("beta_end", ctypes.c_float)]


DENOISER_WEIGHT_NAMES = ("w_patch", "b_patch", "w_t1", "b_t1", "w_t2", "b_t2", "w_fada", "b_fada", "w_out", "b_out")


class DenoiserWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in DENOISER_WEIGHT_NAMES]


_lib = None

_P = ctypes.c_void_p
_I32, _I64, _U32, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
_SIGNATURES = {
    "stage_create": [ctypes.POINTER(StageConfig), ctypes.POINTER(_P)],
    "stage_destroy": [_P],
    "stage_load_weights": [_P, _I32, ctypes.POINTER(LayerWeights), _P],
    "stage_load_text_weights": [_P, _I32, ctypes.POINTER(LayerWeights), _P],
    "stage_set_rope": [_P, _P, _P],
    "stage_set_cond": [_P, _P, _P],
    "stage_run_patch": [_P, _I64, _I64, _P, _P, _P],
    "stage_run_step": [_P, _P, _P, _P, _U32, _P],
    "kvbuf_splice": [ctypes.POINTER(KVView), ctypes.POINTER(KVView), _I64, _I64, _P],
    "stage_get_kvbuf": [_P, _I32, ctypes.POINTER(KVView)],
    "stage_get_kvbuf_sample": [_P, _I32, _I32, ctypes.POINTER(KVView)],
    "stage_get_config": [_P, ctypes.POINTER(StageConfig)],
    "stage_profile_begin": [_P, _I32],
    "stage_profile_end": [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)],
    "denoiser_create": [_P, ctypes.POINTER(DenoiserConfig), ctypes.POINTER(_P)],
    "denoiser_destroy": [_P],
    "denoiser_load_weights": [_P, ctypes.POINTER(DenoiserWeights), _P],
    "denoiser_step": [_P, _P, _P, _P, _I32, _I32, _U32, _F, _P],
    "denoiser_run": [_P, _P, _P, _P, ctypes.POINTER(ctypes.c_int32), _I32, _I32, _F, _P],
    "pf_ln_modulate": [_P, _I64, _I32, _P, _P, _F, _P, _I32, _P],
    "pf_gemm": [_P, _I64, _P, _P, _I64, _I64, _I64, _I32, _P, _I64, _P, _I32, _P, ctypes.c_uint64, _P],
    "pf_gemm_qkv_splice": [_P, _I64, _P, _P, _I64, _I64, _P, _I64, ctypes.POINTER(KVView), _I64, _P, ctypes.c_uint64,
                           _P],
    "pf_gemm_residual_ln": [_P, _I64, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _F, _P, _P, ctypes.c_uint64, _P],
    "pf_gemm_workspace_size": [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_uint64)],
    "pf_attention": [_P, _I64, ctypes.POINTER(KVView), _I64, _I64, _I32, _I32, _P, _I64, _P, ctypes.c_uint64, _P],
    "pf_qk_norm_rope": [_P, _I64, ctypes.POINTER(KVView), _I64, _I64, _I32, _I32, _P, _P, _P, _U32, _P],
    "pf_attention_workspace_size": [_I64, _I32, _I32, ctypes.POINTER(ctypes.c_uint64)],
    "pf_attention_noalloc": [_P, _I64, ctypes.POINTER(KVView), _I64, _I64, _I32, _I32, _P, _I64, _P],
    "pf_adaln": [_P, _P, _P, _I32, _P, _I32, _P],
}


def header_functions(path: str = HEADER):
    """Names of the functions include/pf.h declares."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:pf_status|const char\*)\s+(\w+)\s*\(", src, flags=re.M)


def lib():
    """Load libpf.so (built in-tree by patch_pipelined_attention_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m patch_pipelined_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.pf_last_error.argtypes = []
        L.pf_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pf_last_error().decode()


def _check(status: int):
    if status != PF_OK:
        raise PFError(status, last_error())


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _ptr(t):
    if t is None:
        return None
    return t if isinstance(t, int) else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PF_BF16
    if t.dtype == torch.float32:
        return PF_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------- stage calls

def stage_create(cfg: StageConfig) -> ctypes.c_void_p:
    h = _P()
    _check(lib().stage_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def stage_destroy(handle) -> None:
    _check(lib().stage_destroy(handle))


def stage_load_weights(handle, layer: int, w: dict, stream=None) -> None:
    lw = LayerWeights(**{k: _ptr(w.get(k)) for k, _ in LayerWeights._fields_})
    _check(lib().stage_load_weights(handle, layer, ctypes.byref(lw), _stream(stream)))


def stage_load_text_weights(handle, layer: int, w: dict, stream=None) -> None:
    lw = LayerWeights(**{k: _ptr(w.get(k)) for k, _ in LayerWeights._fields_})
    _check(lib().stage_load_text_weights(handle, layer, ctypes.byref(lw), _stream(stream)))


def stage_set_rope(handle, angles, stream=None) -> None:
    _check(lib().stage_set_rope(handle, _ptr(angles), _stream(stream)))


def stage_set_cond(handle, cond, stream=None) -> None:
    _check(lib().stage_set_cond(handle, _ptr(cond), _stream(stream)))


def stage_run_patch(handle, row_off: int, rows: int, x_in, x_out, stream=None) -> None:
    _check(lib().stage_run_patch(handle, row_off, rows, _ptr(x_in), _ptr(x_out), _stream(stream)))


def stage_run_step(handle, x_in, x_out, cond, warmup: bool = False, stream=None) -> None:
    _check(lib().stage_run_step(handle, _ptr(x_in), _ptr(x_out), _ptr(cond),
                                PF_STEP_WARMUP if warmup else 0, _stream(stream)))


def kvbuf_splice(dst: KVView, src: KVView, offset: int, length: int, stream=None) -> None:
    _check(lib().kvbuf_splice(ctypes.byref(dst), ctypes.byref(src), offset, length, _stream(stream)))


def stage_get_kvbuf(handle, layer: int, sample: int = 0) -> KVView:
    v = KVView()
    if sample == 0:
        _check(lib().stage_get_kvbuf(handle, layer, ctypes.byref(v)))
    else:
        _check(lib().stage_get_kvbuf_sample(handle, layer, sample, ctypes.byref(v)))
    return v


# --------------------------------------------------------------------------- components

def pf_ln_modulate(x, shift, scale, eps: float, y, stream=None) -> None:
    rows, hidden = x.shape
    _check(lib().pf_ln_modulate(_ptr(x), rows, hidden, _ptr(shift), _ptr(scale), eps, _ptr(y), _dtype_code(y),
                                _stream(stream)))


def pf_gemm(a, w, bias, epi: int, c, gate=None, m=None, lda=None, ldc=None, workspace=None, stream=None) -> None:
    n, k = w.shape
    m = a.shape[0] if m is None else m
    lda = a.stride(0) if lda is None else lda
    ldc = c.stride(0) if ldc is None else ldc
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pf_gemm(_ptr(a), lda, _ptr(w), _ptr(bias), m, n, k, epi, _ptr(c), ldc, _ptr(gate),
                         _dtype_code(w), _ptr(workspace), ws_bytes, _stream(stream)))


def pf_gemm_qkv_splice(a, w, bias, q, kv: KVView, row_offset: int, m=None, lda=None, ldq=None, workspace=None,
                       stream=None) -> None:
    m = a.shape[0] if m is None else m
    hidden = w.shape[1]
    lda = a.stride(0) if lda is None else lda
    ldq = q.stride(0) if ldq is None else ldq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pf_gemm_qkv_splice(_ptr(a), lda, _ptr(w), _ptr(bias), m, hidden, _ptr(q), ldq, ctypes.byref(kv),
                                    row_offset, _ptr(workspace), ws_bytes, _stream(stream)))


def pf_gemm_residual_ln(a, w, bias, x, gate, shift, scale, eps: float, y, lda=None, workspace=None,
                        stream=None) -> None:
    n, k = w.shape
    m = x.shape[0]
    lda = a.stride(0) if lda is None else lda
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pf_gemm_residual_ln(_ptr(a), lda, _ptr(w), _ptr(bias), m, n, k, _ptr(x), _ptr(gate), _ptr(shift),
                                     _ptr(scale), eps, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def pf_gemm_workspace_size(m: int, n: int, k: int) -> int:
    b = ctypes.c_uint64()
    _check(lib().pf_gemm_workspace_size(m, n, k, ctypes.byref(b)))
    return b.value


def gemm_workspace(m: int, n: int, k: int):
    """torch uint8 device buffer of pf_gemm_workspace_size bytes (None when zero)."""
    import torch
    nb = pf_gemm_workspace_size(m, n, k)
    return torch.empty((nb,), dtype=torch.uint8, device="cuda") if nb else None


def pf_attention(q, kv: KVView, seq_kv: int, rows: int, heads: int, head_dim: int, o, ldq=None, ldo=None,
                 workspace=None, stream=None) -> None:
    ldq = q.stride(0) if ldq is None else ldq
    ldo = o.stride(0) if ldo is None else ldo
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pf_attention(_ptr(q), ldq, ctypes.byref(kv), seq_kv, rows, heads, head_dim, _ptr(o), ldo,
                              _ptr(workspace), ws_bytes, _stream(stream)))


def pf_attention_noalloc(q, kv: KVView, seq_kv: int, rows: int, heads: int, head_dim: int, o, ldq=None, ldo=None,
                         stream=None) -> None:
    ldq = q.stride(0) if ldq is None else ldq
    ldo = o.stride(0) if ldo is None else ldo
    _check(lib().pf_attention_noalloc(_ptr(q), ldq, ctypes.byref(kv), seq_kv, rows, heads, head_dim, _ptr(o), ldo,
                                      _stream(stream)))


def pf_qk_norm_rope(q, kv: KVView, row_offset: int, rows: int, heads: int, head_dim: int, q_gamma=None,
                    k_gamma=None, angles=None, ldq=None, stream=None) -> None:
    """QK-RMSNorm (when both gammas are given) and rotary embedding (when angles are given) of
    q's rows and K rows [row_offset, row_offset + rows) of kv, in place."""
    ldq = q.stride(0) if ldq is None else ldq
    flags = (PF_STAGE_QK_NORM if q_gamma is not None else 0) | (PF_STAGE_ROPE if angles is not None else 0)
    _check(lib().pf_qk_norm_rope(_ptr(q), ldq, ctypes.byref(kv), row_offset, rows, heads, head_dim, _ptr(q_gamma),
                                 _ptr(k_gamma), _ptr(angles), flags, _stream(stream)))


def pf_attention_workspace_size(rows: int, heads: int, head_dim: int) -> int:
    b = ctypes.c_uint64()
    _check(lib().pf_attention_workspace_size(rows, heads, head_dim, ctypes.byref(b)))
    return b.value


def attention_workspace(rows: int, heads: int, head_dim: int):
    """torch uint8 device buffer of pf_attention_workspace_size bytes (None when zero)."""
    import torch
    n = pf_attention_workspace_size(rows, heads, head_dim)
    return torch.empty((n,), dtype=torch.uint8, device="cuda") if n else None


def pf_adaln(cond, w_ada, b_ada, mod, stream=None) -> None:
    hidden = cond.shape[0]
    _check(lib().pf_adaln(_ptr(cond), _ptr(w_ada), _ptr(b_ada), hidden, _ptr(mod), _dtype_code(w_ada),
                          _stream(stream)))


def kv_view(k, v, rows: int, row_elems: int, v_layout: int, k_ld=None, v_ld=None) -> KVView:
    """View over torch tensors k / v (K rows layout; V rows or K8)."""
    return KVView(k=_ptr(k), v=_ptr(v), rows=rows, row_elems=row_elems,
                  k_ld=row_elems if k_ld is None else k_ld, v_ld=row_elems if v_ld is None else v_ld,
                  dtype=_dtype_code(k), v_layout=v_layout)


def stage_profile_begin(handle, max_launches: int) -> None:
    _check(lib().stage_profile_begin(handle, max_launches))


def stage_profile_end(handle):
    """(timed attention launches, their summed duration in ms) since stage_profile_begin."""
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(lib().stage_profile_end(handle, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def stage_get_config(handle) -> StageConfig:
    c = StageConfig()
    _check(lib().stage_get_config(handle, ctypes.byref(c)))
    return c


def denoiser_create(stage_handle, cfg: DenoiserConfig):
    h = ctypes.c_void_p()
    _check(lib().denoiser_create(stage_handle, ctypes.byref(cfg), ctypes.byref(h)))
    return h


def denoiser_destroy(handle) -> None:
    _check(lib().denoiser_destroy(handle))


def denoiser_load_weights(handle, w: dict, stream=None) -> None:
    lw = DenoiserWeights(**{n: _ptr(w[n]) for n in DENOISER_WEIGHT_NAMES})
    _check(lib().denoiser_load_weights(handle, ctypes.byref(lw), _stream(stream)))


def denoiser_step(handle, z, y, t: int, t_next: int, warmup: bool = False, guidance: float = 1.0, x_txt=None,
                  stream=None) -> None:
    _check(lib().denoiser_step(handle, _ptr(z), _ptr(y), _ptr(x_txt), t, t_next, PF_STEP_WARMUP if warmup else 0,
                               guidance, _stream(stream)))


def denoiser_run(handle, z, y, timesteps, warmup_steps: int, guidance: float = 1.0, x_txt=None, stream=None) -> None:
    ts = (ctypes.c_int32 * len(timesteps))(*[int(t) for t in timesteps])
    _check(lib().denoiser_run(handle, _ptr(z), _ptr(y), _ptr(x_txt), ts, len(timesteps), warmup_steps, guidance,
                              _stream(stream)))
