"""Teacher-forced parity of each HIP kernel (through its component entry point)
against the fp64 oracle, fed the same bf16 / fp32 inputs, at sizes that span
several tiles with ragged tails."""
import math

import numpy as np
import pytest

from oracle import ref
from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth
from patch_pipelined_attention_amd.stage import rows_to_k8

from _util import assert_close, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ LayerNorm + modulation

@pytest.mark.parametrize("rows,hidden", [(1, 128), (77, 1152), (300, 1536), (5, 3072), (64, 4096), (3, 6144)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ln_modulate(rows, hidden, dtype):
    torch = torch_cuda()
    x = synth.randn((rows, hidden), 1 + rows, std=3.0) + 2.0
    shift = synth.randn((hidden,), 2 + rows, std=0.5)
    scale = synth.randn((hidden,), 3 + rows, std=0.5)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty((rows, hidden), dtype=tdt, device="cuda")
    B.pf_ln_modulate(dev(torch, x), dev(torch, shift), dev(torch, scale), 1e-6, y)
    want = ref.modulate(ref.layer_norm(x, 1e-6), shift, scale)
    if dtype == "bf16":
        want = ref.bf16_round(want)
        assert_close(host(y), want, f"ln_mod bf16 {rows}x{hidden}")
    else:
        assert_close(host(y), want, f"ln_mod fp32 {rows}x{hidden}", max_abs_tol=1e-4, rel_tol=1e-5)


# ------------------------------------------------------------------ GEMM

GEMM_SHAPES = [(1, 64, 64), (77, 192, 128), (128, 128, 1152), (300, 1152, 1152), (1000, 3456, 1152),
               (130, 576, 4608), (1024, 1152, 4608), (4100, 4608, 1152)]


@pytest.mark.parametrize("split", [False, True], ids=["whole", "ksplit"])
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [B.PF_EPI_STORE, B.PF_EPI_GELU_TANH, B.PF_EPI_GELU_ERF, B.PF_EPI_GATED_RESIDUAL])
def test_gemm_bf16(m, n, k, epi, split):
    """Small grids split k when given a workspace (default tile choice: 128 x 128 here)."""
    torch = torch_cuda()
    ws = B.gemm_workspace(m, n, k) if split else None
    seed = m * 7 + n * 11 + k * 13 + epi
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.5)
    y = ref.linear(a, w, bias)
    if epi == B.PF_EPI_GATED_RESIDUAL:
        x0 = synth.randn((m, n), seed + 3)
        gate = synth.randn((n,), seed + 4)
        c = dev(torch, x0)
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  gate=dev(torch, gate), workspace=ws)
        want = x0 + gate * y
    else:
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  workspace=ws)
        act = {B.PF_EPI_STORE: lambda v: v, B.PF_EPI_GELU_TANH: ref.gelu_tanh, B.PF_EPI_GELU_ERF: ref.gelu_erf}[epi]
        want = ref.bf16_round(act(y))
    assert_close(host(c), want, f"gemm bf16 {m}x{n}x{k} epi={epi}")


@pytest.mark.parametrize("kernel", ["256", "128d", "128x64", "256x128"], ids=["deep256", "deep128", "t128x64", "t256x128"])
@pytest.mark.parametrize("split", [False, True], ids=["whole", "ksplit"])
@pytest.mark.parametrize("m,n,k", [(77, 192, 128), (300, 1344, 1152), (257, 640, 4608)])
@pytest.mark.parametrize("epi", [B.PF_EPI_STORE, B.PF_EPI_GELU_TANH, B.PF_EPI_GATED_RESIDUAL])
def test_gemm_bf16_deep_ring(m, n, k, epi, split, kernel, monkeypatch):
    """The kernels other than the default, forced through PF_GEMM_TILE (deep rings: 256 x 256
    with 4 stages, 128 x 128 with 8, 256 features x 128 tokens with 3 and two workgroups per CU;
    and 128 features x 64 tokens with the 2-stage ring): ragged
    m and n (partial tiles in both), k from fewer tiles than the ring holds to a long ring, with
    and without the k split."""
    torch = torch_cuda()
    monkeypatch.setenv("PF_GEMM_TILE", kernel)
    ws = B.gemm_workspace(m, n, k) if split else None
    seed = m * 5 + n * 3 + k + epi
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.5)
    y = ref.linear(a, w, bias)
    if epi == B.PF_EPI_GATED_RESIDUAL:
        x0 = synth.randn((m, n), seed + 3)
        gate = synth.randn((n,), seed + 4)
        c = dev(torch, x0)
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  gate=dev(torch, gate), workspace=ws)
        want = x0 + gate * y
    else:
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  workspace=ws)
        act = {B.PF_EPI_STORE: lambda v: v, B.PF_EPI_GELU_TANH: ref.gelu_tanh}[epi]
        want = ref.bf16_round(act(y))
    assert_close(host(c), want, f"gemm bf16 deep ring {kernel} {m}x{n}x{k} epi={epi}")


def test_gemm_bf16_long_k_default_plan():
    """The Flux-shaped MLP down projection (2048 x 3072 x 12288, gated residual) with the
    workspace the stage gives it (the default plan: 128 x 128 tiles, a 192-step k loop).
    Checked on 64 sampled rows (the full fp64 product is too slow for the oracle)."""
    torch = torch_cuda()
    m, n, k = 2048, 3072, 12288
    ws = B.gemm_workspace(m, n, k)
    seed = 4242
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.5)
    x0 = synth.randn((m, n), seed + 3)
    gate = synth.randn((n,), seed + 4)
    c = dev(torch, x0)
    B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias),
              B.PF_EPI_GATED_RESIDUAL, c, gate=dev(torch, gate), workspace=ws)
    rows = np.random.default_rng(seed).choice(m, 64, replace=False)
    want = x0[rows] + gate * ref.linear(a[rows], w, bias)
    assert_close(host(c)[rows], want, "gemm bf16 2048x3072x12288 gated residual, sampled rows")


def test_gemm_bf16_split_workspace_reuse():
    """One workspace serves k-split GEMMs of different shapes in turn (the stage's pattern:
    QKV, out-projection, QKV again): results match the oracle, and a repeated call reproduces
    its output bit for bit (slices are summed in a fixed order)."""
    torch = torch_cuda()
    shapes = [(1024, 3456, 1152, B.PF_EPI_STORE), (1024, 1152, 1152, B.PF_EPI_GATED_RESIDUAL)]
    sizes = [B.pf_gemm_workspace_size(m, n, k) for m, n, k, _ in shapes]
    ws = torch.empty((max(sizes),), dtype=torch.uint8, device="cuda") if max(sizes) else None
    outs = []
    for rep, (m, n, k, epi) in enumerate(shapes + shapes[:1]):
        seed = 900 + m + n + k
        a = synth.randn((m, k), seed, std=1.0, bf16=True)
        w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
        bias = synth.randn((n,), seed + 2, std=0.5)
        if epi == B.PF_EPI_GATED_RESIDUAL:
            x0 = synth.randn((m, n), seed + 3)
            gate = synth.randn((n,), seed + 4)
            c = dev(torch, x0)
            B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                      gate=dev(torch, gate), workspace=ws)
            want = x0 + gate * ref.linear(a, w, bias)
        else:
            c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                      workspace=ws)
            want = ref.bf16_round(ref.linear(a, w, bias))
        got = host(c)
        assert_close(got, want, f"gemm split reuse {m}x{n}x{k} call {rep}")
        outs.append(got)
    assert np.array_equal(outs[0], outs[2]), "repeated split GEMM is not bit-identical"


def test_gemm_bf16_strided_operands():
    torch = torch_cuda()
    m, n, k, lda, ldc = 200, 128, 192, 256, 384
    a = synth.randn((m, lda), 5, bf16=True)
    w = synth.randn((n, k), 6, std=0.07, bf16=True)
    bias = synth.randn((n,), 7)
    c = torch.zeros((m, ldc), dtype=torch.bfloat16, device="cuda")
    B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), B.PF_EPI_STORE, c,
              lda=lda, ldc=ldc, m=m)
    got = host(c)
    assert_close(got[:, :n], ref.bf16_round(ref.linear(a[:, :k], w, bias)), "gemm strided")
    assert np.all(got[:, n:] == 0)


@pytest.mark.parametrize("m,n,k", [(1, 8, 8), (70, 128, 128), (64, 384, 128)])
@pytest.mark.parametrize("epi", [B.PF_EPI_STORE, B.PF_EPI_GELU_TANH, B.PF_EPI_GATED_RESIDUAL])
def test_gemm_fp32(m, n, k, epi):
    torch = torch_cuda()
    a = synth.randn((m, k), 11 + m)
    w = synth.randn((n, k), 12 + n, std=1 / math.sqrt(k))
    bias = synth.randn((n,), 13)
    y = ref.linear(a, w, bias)
    if epi == B.PF_EPI_GATED_RESIDUAL:
        x0 = synth.randn((m, n), 14)
        gate = synth.randn((n,), 15)
        c = dev(torch, x0)
        B.pf_gemm(dev(torch, a), dev(torch, w), dev(torch, bias), epi, c, gate=dev(torch, gate))
        want = x0 + gate * y
    else:
        c = torch.empty((m, n), dtype=torch.float32, device="cuda")
        B.pf_gemm(dev(torch, a), dev(torch, w), dev(torch, bias), epi, c)
        want = ref.gelu_tanh(y) if epi == B.PF_EPI_GELU_TANH else y
    assert_close(host(c), want, f"gemm fp32 {m}x{n}x{k}", max_abs_tol=1e-4, rel_tol=1e-5)


# ------------------------------------------------------------------ attention

def _kv_bf16(torch, K, V):
    S, h = K.shape
    kt = dev(torch, K, torch.bfloat16)
    vt = dev(torch, rows_to_k8(V.astype(np.float32)), torch.bfloat16)
    return kt, vt, B.kv_view(kt, vt, S, h, B.PF_LAYOUT_K8)


ATTN_CASES = [(64, 2, 64, 1), (64, 2, 100, 50), (64, 3, 1000, 129), (72, 2, 64, 128), (72, 2, 777, 300),
              (72, 4, 2053, 77), (128, 2, 65, 128), (128, 2, 1500, 200), (128, 1, 8, 3), (64, 2, 4133, 257),
              (72, 1, 3000, 600), (128, 3, 2500, 513)]


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
@pytest.mark.parametrize("D,H,S,rows", ATTN_CASES)
def test_attention_bf16(D, H, S, rows, split):
    """`split` passes a workspace, letting small query grids split the key range (merge kernel)."""
    torch = torch_cuda()
    h = H * D
    seed = D * 1000 + S + rows
    q = synth.randn((rows, 3 * h), seed, std=1.0, bf16=True)      # Q inside a qkv-shaped row (ld = 3h)
    K = synth.randn((S, h), seed + 1, std=1.0, bf16=True)
    V = synth.randn((S, h), seed + 2, std=1.0, bf16=True)
    kt, vt, kv = _kv_bf16(torch, K, V)
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    ws = B.attention_workspace(rows, H, D) if split else None
    print(f"[attn] D={D} H={H} S={S} rows={rows} split={split}", flush=True)
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, rows, H, D, o, workspace=ws)
    want = ref.attention(q[:, :h], K, V, H, D)
    assert_close(host(o), ref.bf16_round(want), f"attention bf16 D={D} S={S} rows={rows} vs bf16-in")
    assert_close(host(o), want, f"attention bf16 D={D} S={S} rows={rows} vs exact")


@pytest.mark.parametrize("cfg", ["c3", "c4", "c5"])
def test_attention_full_size_sampled(cfg):
    """One patch's attention at a stage's full size and launch configuration (the patch rows
    against the whole S_kv-row buffer, with the stage's split workspace): SD3 (d = 64), Flux
    (d = 128, text prefix included in S_kv) and long-sequence PixArt (d = 72, 262144 keys).
    Checked on 48 sampled query rows (first, last, tile edges, random) against the oracle over
    the full key range."""
    from patch_pipelined_attention_amd.configs import CONFIGS
    torch = torch_cuda()
    shape = CONFIGS[cfg]
    P, S, H, D = shape.patch_rows, shape.seq_kv, shape.heads, shape.head_dim
    h = H * D
    seed = 7000 + S + D
    q = synth.randn((P, 3 * h), seed, std=1.0, bf16=True)
    K = synth.randn((S, h), seed + 1, std=1.0, bf16=True)
    V = synth.randn((S, h), seed + 2, std=1.0, bf16=True)
    kt, vt, kv = _kv_bf16(torch, K, V)
    o = torch.empty((P, h), dtype=torch.bfloat16, device="cuda")
    ws = B.attention_workspace(P, H, D)
    print(f"[attn] full size {cfg}: P={P} S={S} H={H} D={D}", flush=True)
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, P, H, D, o, workspace=ws)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 511, 512, P - 1], rng.choice(P, 41, replace=False)]))
    got = host(o)[rows]
    want = ref.attention(q[rows, :h], K, V, H, D)
    assert_close(got, ref.bf16_round(want), f"attention {cfg} full size, sampled rows vs bf16-in")
    assert_close(got, want, f"attention {cfg} full size, sampled rows vs exact")


@pytest.mark.parametrize("D", [64, 72, 128])
def test_attention_bf16_closed_forms(D):
    torch = torch_cuda()
    H, S, rows = 2, 300, 70
    h = H * D
    K = synth.randn((S, h), 51, bf16=True)
    V = synth.randn((S, h), 52, bf16=True)
    q = synth.randn((rows, h), 53, bf16=True)
    # V = 1 -> every output is exactly 1 up to P rounding (softmax rows sum to one)
    kt, vt, kv = _kv_bf16(torch, K, np.ones_like(V))
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, rows, H, D, o)
    assert np.abs(host(o) - 1.0).max() <= 8e-3
    # Q = 0 -> uniform weights -> column mean of V
    kt, vt, kv = _kv_bf16(torch, K, V)
    B.pf_attention(torch.zeros((rows, h), dtype=torch.bfloat16, device="cuda"), kv, S, rows, H, D, o)
    assert_close(host(o), np.broadcast_to(V.mean(axis=0), (rows, h)), f"attention Q=0 D={D}", max_abs_tol=4e-3,
                 rel_tol=None)
    # one dominant key per head -> that V row
    K2 = np.zeros_like(K)
    q2 = np.zeros((rows, h), np.float32)
    for j in range(H):
        K2[17 + j, j * D] = 8.0
        q2[:, j * D] = 8.0 * math.sqrt(D) / 8.0 * 8.0     # logit 64 for the dominant key, 0 for the rest
    kt, vt, kv = _kv_bf16(torch, K2, V)
    B.pf_attention(dev(torch, q2, torch.bfloat16), kv, S, rows, H, D, o)
    got = host(o)
    for j in range(H):
        np.testing.assert_allclose(got[:, j * D:(j + 1) * D], np.broadcast_to(V[17 + j, j * D:(j + 1) * D], (rows, D)),
                                   atol=1e-6)


@pytest.mark.parametrize("D,S,rows", [(64, 256, 64), (64, 100, 33), (128, 70, 5)])
def test_attention_fp32(D, S, rows):
    torch = torch_cuda()
    H = 2
    h = H * D
    q = synth.randn((rows, h), 61 + S)
    K = synth.randn((S, h), 62 + S)
    V = synth.randn((S, h), 63 + S)
    kt, vt = dev(torch, K), dev(torch, V)
    kv = B.kv_view(kt, vt, S, h, B.PF_LAYOUT_ROWS)
    o = torch.empty((rows, h), dtype=torch.float32, device="cuda")
    B.pf_attention(dev(torch, q), kv, S, rows, H, D, o)
    assert_close(host(o), ref.attention(q, K, V, H, D), f"attention fp32 D={D}", max_abs_tol=1e-4, rel_tol=1e-5)


# ------------------------------------------------------------------ adaLN

@pytest.mark.parametrize("hidden,dtype", [(128, "fp32"), (1152, "bf16"), (3072, "bf16")])
def test_adaln(hidden, dtype):
    torch = torch_cuda()
    c = synth.randn((hidden,), 71)
    w = synth.randn((6 * hidden, hidden), 72, std=0.02, bf16=(dtype == "bf16"))
    b = synth.randn((6 * hidden,), 73, std=0.02)
    mod = torch.empty((6 * hidden,), dtype=torch.float32, device="cuda")
    B.pf_adaln(dev(torch, c), dev(torch, w, torch.bfloat16 if dtype == "bf16" else torch.float32), dev(torch, b), mod)
    assert_close(host(mod), ref.adaln(c, w, b).reshape(-1), f"adaln {hidden}", max_abs_tol=1e-4, rel_tol=1e-5)
