"""C-ABI checks that need no GPU: the library loads, exports every function
include/pf.h declares, and rejects invalid arguments before any HIP call."""
import ctypes

import pytest

from patch_pipelined_attention_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_exports_every_declared_function(lib):
    names = B.header_functions()
    assert len(names) >= 9
    for required in ("stage_create", "stage_load_weights", "stage_run_patch", "stage_run_step", "kvbuf_splice",
                     "stage_destroy", "stage_set_cond", "stage_get_kvbuf", "pf_last_error"):
        assert required in names
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(num_layers=2, hidden=1152, heads=16, head_dim=72, mlp_ratio=4, num_patches=4, seq_img=4096,
                seq_txt=0, dtype=B.PF_BF16, gelu=B.PF_GELU_TANH, ln_eps=1e-6, flags=0)
    base.update(kw)
    return B.StageConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(num_layers=0), B.PF_ERR_INVALID_ARG),
    (dict(head_dim=96, hidden=16 * 96), B.PF_ERR_UNSUPPORTED),
    (dict(hidden=1000), B.PF_ERR_INVALID_ARG),
    (dict(seq_img=4095), B.PF_ERR_INVALID_ARG),
    (dict(num_patches=0), B.PF_ERR_INVALID_ARG),
    (dict(seq_txt=-1), B.PF_ERR_INVALID_ARG),
    (dict(dtype=7), B.PF_ERR_INVALID_ARG),
    (dict(gelu=5), B.PF_ERR_INVALID_ARG),
    (dict(ln_eps=0.0), B.PF_ERR_INVALID_ARG),
    (dict(flags=B.PF_STAGE_QK_NORM, dtype=B.PF_FP32), B.PF_ERR_UNSUPPORTED),   # options are bf16-only
    (dict(flags=B.PF_STAGE_DUAL_STREAM, seq_txt=0), B.PF_ERR_INVALID_ARG),     # dual stream needs text rows
    (dict(flags=B.PF_STAGE_DUAL_STREAM | B.PF_STAGE_PARALLEL, seq_txt=8), B.PF_ERR_UNSUPPORTED),
    (dict(flags=16), B.PF_ERR_INVALID_ARG),             # unknown block option
    (dict(heads=1, hidden=72), B.PF_ERR_UNSUPPORTED),        # bf16 needs hidden % 64 == 0
    (dict(mlp_ratio=-1), B.PF_ERR_INVALID_ARG),
    (dict(batch=-1), B.PF_ERR_INVALID_ARG),
    (dict(batch=9), B.PF_ERR_INVALID_ARG),             # PF_MAX_STAGE_BATCH is 8
])
def test_stage_create_rejects_bad_configs(lib, kw, status):
    cfg = _cfg(**kw)
    h = ctypes.c_void_p(123)
    st = lib.stage_create(ctypes.byref(cfg), ctypes.byref(h))
    assert st == status
    assert h.value is None                     # *out cleared, nothing created
    assert len(B.last_error()) > 0


def test_null_arguments(lib):
    assert lib.stage_create(None, None) == B.PF_ERR_INVALID_ARG
    assert lib.stage_destroy(None) == B.PF_OK
    assert lib.stage_run_patch(None, 0, 1, None, None, None) == B.PF_ERR_INVALID_ARG
    assert lib.stage_get_kvbuf(None, 0, None) == B.PF_ERR_INVALID_ARG
    assert lib.stage_load_text_weights(None, 0, None, None) == B.PF_ERR_INVALID_ARG
    assert lib.stage_set_rope(None, None, None) == B.PF_ERR_INVALID_ARG


def _view(k, v, rows, elems=64, dtype=B.PF_BF16, layout=B.PF_LAYOUT_ROWS, k_ld=None, v_ld=None):
    return B.KVView(k=k, v=v, rows=rows, row_elems=elems, k_ld=k_ld or elems, v_ld=v_ld or elems, dtype=dtype,
                    v_layout=layout)


@pytest.mark.parametrize("case", ["range", "neg", "src_short", "dtype", "elems", "overlap", "null", "layout"])
def test_kvbuf_splice_validation(lib, case):
    # fake, never-dereferenced addresses: validation runs before any device access
    base = 1 << 40
    dst = _view(base, base + (1 << 30), 100)
    src = _view(base + (2 << 30), base + (3 << 30), 50)
    off, n = 10, 20
    if case == "range":
        off, n = 90, 20
    elif case == "neg":
        off = -1
    elif case == "src_short":
        n = 60
    elif case == "dtype":
        src.dtype = B.PF_FP32
    elif case == "elems":
        src.row_elems = 32
    elif case == "overlap":
        src.k = base + 64 * 2 * 15          # inside dst.K's rows [10, 30)
    elif case == "null":
        dst.v = None
    elif case == "layout":
        dst.v_layout = 9
    st = lib.kvbuf_splice(ctypes.byref(dst), ctypes.byref(src), off, n, None)
    assert st == B.PF_ERR_INVALID_ARG, B.last_error()


def test_kvbuf_splice_zero_length_is_noop_without_device(lib):
    base = 1 << 40
    dst = _view(base, base + (1 << 30), 100)
    src = _view(base + (2 << 30), base + (3 << 30), 50)
    assert lib.kvbuf_splice(ctypes.byref(dst), ctypes.byref(src), 100, 0, None) == B.PF_OK


def test_component_validation(lib):
    base = 1 << 40
    # gemm: bf16 n must be a multiple of 64
    assert lib.pf_gemm(base, 128, base, base, 10, 100, 128, 0, base, 100, None, B.PF_BF16, None, 0, None) == B.PF_ERR_UNSUPPORTED
    assert lib.pf_gemm(base, 128, base, base, 10, 128, 128, 9, base, 128, None, B.PF_BF16, None, 0, None) == B.PF_ERR_INVALID_ARG
    # gated residual needs a gate
    assert lib.pf_gemm(base, 128, base, base, 10, 128, 128, 3, base, 128, None, B.PF_BF16, None, 0, None) == B.PF_ERR_INVALID_ARG
    # attention: head_dim 80 unsupported, bf16 needs K8 V
    kv = _view(base, base + (1 << 30), 1000, elems=160, layout=B.PF_LAYOUT_K8)
    assert lib.pf_attention(base, 480, ctypes.byref(kv), 1000, 10, 2, 80, base, 160, None, 0, None) == B.PF_ERR_UNSUPPORTED
    kv2 = _view(base, base + (1 << 30), 1000, elems=128, layout=B.PF_LAYOUT_ROWS)
    assert lib.pf_attention(base, 384, ctypes.byref(kv2), 1000, 10, 2, 64, base, 128, None, 0, None) == B.PF_ERR_UNSUPPORTED
    assert lib.pf_attention(base, 384, ctypes.byref(kv), 1001, 10, 2, 64, base, 128, None, 0, None) == B.PF_ERR_INVALID_ARG
    # misaligned workspace
    assert lib.pf_attention(base, 384, ctypes.byref(kv), 1000, 10, 2, 64, base, 128, base + 8, 1 << 20, None) == B.PF_ERR_INVALID_ARG
    # workspace size query: 8 splits of fp32 slice results plus fp32 (m, l) per split
    n = ctypes.c_uint64()
    assert lib.pf_attention_workspace_size(1024, 16, 72, ctypes.byref(n)) == B.PF_OK
    assert n.value == 4 * 8 * 1024 * 1152 + 4 * 2 * 8 * 1024 * 16
    # misaligned pointer
    assert lib.pf_ln_modulate(base + 4, 3, 64, base, base, 1e-6, base, 0, None) == B.PF_ERR_INVALID_ARG


def test_memory_formula():
    """The stage holds one K and one V buffer per own layer: 2 * L * S_kv * h elements (PipeFusion mechanism 4)."""
    from patch_pipelined_attention_amd.configs import CONFIGS
    c3 = CONFIGS["c3"]
    per_layer = 2 * c3.seq_kv * c3.hidden * 2
    assert per_layer == 100_663_296               # 100.7 MB per layer for the SD3-shaped stage
    c5 = CONFIGS["c5"]
    assert 2 * c5.seq_kv * c5.hidden * 2 == 1_207_959_552   # ~1.2 GB per layer at 262144 tokens
