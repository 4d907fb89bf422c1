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
    """Small grids split k when given a workspace.  Tiles: 128 x 128, except 4100 x 4608 x 1152
    (33 x 24 tiles of 192 features x 128 tokens, more than 1.5 per CU: whole, ragged last tile row)."""
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


@pytest.mark.parametrize("m,n,k", [(1024, 1152, 1152), (1024, 1152, 4608), (2048, 1536, 6144), (100, 3072, 3072),
                                   (2048, 3072, 12288), (77, 192, 128), (2432, 3456, 1152), (8192, 1152, 1152)])
@pytest.mark.parametrize("split", [False, True], ids=["whole", "ksplit"])
def test_gemm_residual_ln_is_bit_identical(m, n, k, split):
    """The gated-residual projection followed by the modulated LayerNorm of its rows, as one call
    (pf_gemm_residual_ln: with a workspace the k-split's reduce pass also computes the LayerNorm)
    gives the same bits as pf_gemm with the same workspace followed by pf_ln_modulate, and both
    match the oracle.  2432 x 3456 x 1152 (513 tiles) takes the remainder split, whose reduce pass
    covers only the split tiles, and 8192 x 1152 x 1152 runs whole with 192 x 128 tiles; in both
    the LayerNorm runs as its own launch."""
    torch = torch_cuda()
    seed = m + 3 * n + 7 * k
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=0.02, bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.02)
    x0 = synth.randn((m, n), seed + 3)
    gate = synth.randn((n,), seed + 4, std=0.5)
    shift = synth.randn((n,), seed + 5, std=0.4)
    scale = synth.randn((n,), seed + 6, std=0.4)
    ws = B.gemm_workspace(m, n, k) if split else None
    ad, wd, bd, gd = dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), dev(torch, gate)
    sd, scd = dev(torch, shift), dev(torch, scale)
    x1, x2 = dev(torch, x0), dev(torch, x0)
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    print(f"[gemm+ln] {m}x{n}x{k} split={split}", flush=True)
    B.pf_gemm_residual_ln(ad, wd, bd, x1, gd, sd, scd, 1e-6, y1, workspace=ws)
    B.pf_gemm(ad, wd, bd, B.PF_EPI_GATED_RESIDUAL, x2, gate=gd, workspace=ws)
    B.pf_ln_modulate(x2, sd, scd, 1e-6, y2)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2), "residual differs from the unfused pair"
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "LayerNorm output differs from the unfused pair"
    rows = np.arange(m) if m <= 128 else np.random.default_rng(seed).choice(m, 48, replace=False)
    xw = x0[rows] + gate * ref.linear(a[rows], w, bias)
    assert_close(host(x1)[rows], xw, f"gemm+ln {m}x{n}x{k} residual", max_abs_tol=1e-3, rel_tol=1e-5)
    assert_close(host(y1)[rows], ref.bf16_round(ref.modulate(ref.layer_norm(host(x1)[rows]), shift, scale)),
                 f"gemm+ln {m}x{n}x{k} LayerNorm of the updated rows")


@pytest.mark.parametrize("epi", [B.PF_EPI_STORE, B.PF_EPI_GELU_TANH, B.PF_EPI_GELU_ERF, B.PF_EPI_GATED_RESIDUAL])
@pytest.mark.parametrize("m,n,k", [(2689, 4608, 1536), (16384, 1152, 4608), (10000, 960, 128)])
def test_gemm_bf16_wide_tiles(m, n, k, epi):
    """Grids the plan runs whole with 192-feature x 128-token tiles (n % 192 == 0, at least 1.5
    tiles per CU): 2689 rows end in a tile row of one token (rows past m clamped on load, never
    stored), 16384 x 1152 x 4608 is the long-sequence PixArt-shaped MLP down projection, and
    n = 960 is a multiple of 192 but not of 128 (79 x 5 tiles, a two-step k loop).
    Checked against the oracle on sampled rows, the first and last rows included."""
    torch = torch_cuda()
    assert B.pf_gemm_workspace_size(m, n, k) == 0, "wide-tile grids run whole"
    seed = 5300 + m + n + k + epi
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.5)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 127, 128, m - 2, m - 1], rng.choice(m, 40, replace=False)]))
    y = ref.linear(a[rows], w, bias)
    ws = B.gemm_workspace(m, n, k)
    print(f"[gemm] wide tiles {m}x{n}x{k} epi={epi}", flush=True)
    if epi == B.PF_EPI_GATED_RESIDUAL:
        x0 = synth.randn((m, n), seed + 3)
        gate = synth.randn((n,), seed + 4)
        c = dev(torch, x0)
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  gate=dev(torch, gate), workspace=ws)
        got = host(c)[rows]
        want = x0[rows] + gate * y
    else:
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  workspace=ws)
        act = {B.PF_EPI_STORE: lambda v: v, B.PF_EPI_GELU_TANH: ref.gelu_tanh, B.PF_EPI_GELU_ERF: ref.gelu_erf}[epi]
        want = ref.bf16_round(act(y))
        got = host(c)[rows]
    assert_close(got, want, f"gemm bf16 {m}x{n}x{k} epi={epi} wide tiles, sampled rows")


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


@pytest.mark.parametrize("epi", [B.PF_EPI_STORE, B.PF_EPI_GELU_TANH, B.PF_EPI_GATED_RESIDUAL])
@pytest.mark.parametrize("m,n,k,tail", [(2304, 4096, 1536, 2048), (2432, 3456, 1152, 2304)])
def test_gemm_bf16_remainder_split(m, n, k, tail, epi):
    """Shapes whose last round of 128 x 128 tiles would hold only a few tiles on 512 workgroup
    slots (576 tiles: one round + 64; 513 tiles: one round + 1; neither has enough 192 x 128
    tiles for the wide tile: n = 4096 is no multiple of 192, 342 tiles), so the plan runs the full round
    as whole tiles and splits k for the remaining tiles only, which a reduce pass over those
    tiles finishes.  Checked against the oracle on sampled rows from both parts: the split tiles
    are the last in the grouped tile order, so token rows from `tail` on lie in split tiles for
    part of their columns."""
    torch = torch_cuda()
    ws = B.gemm_workspace(m, n, k)
    seed = 6100 + m + n + k + epi
    a = synth.randn((m, k), seed, std=1.0, bf16=True)
    w = synth.randn((n, k), seed + 1, std=1.0 / math.sqrt(k), bf16=True)
    bias = synth.randn((n,), seed + 2, std=0.5)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, tail - 1, tail, m - 1], rng.choice(tail, 20, replace=False),
                                     tail + rng.choice(m - tail, 24, replace=False)]))
    y = ref.linear(a[rows], w, bias)
    print(f"[gemm] remainder split {m}x{n}x{k} epi={epi}", flush=True)
    if epi == B.PF_EPI_GATED_RESIDUAL:
        x0 = synth.randn((m, n), seed + 3)
        gate = synth.randn((n,), seed + 4)
        c = dev(torch, x0)
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  gate=dev(torch, gate), workspace=ws)
        want = x0[rows] + gate * y
    else:
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        B.pf_gemm(dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias), epi, c,
                  workspace=ws)
        want = ref.bf16_round(ref.gelu_tanh(y) if epi == B.PF_EPI_GELU_TANH else y)
    assert_close(host(c)[rows], want, f"gemm bf16 {m}x{n}x{k} epi={epi} remainder split, sampled rows")


def test_gemm_split_plan_rules():
    """The k-split plan on a 256-CU MI355X: grids of at least 384 tiles of 192 x 128 (n % 192 == 0)
    run whole with that tile; otherwise, with 128 x 128 tiles, grids with fewer tiles than CUs split
    k (the workspace size is that of the split), grids with a tile for every CU run whole unless a
    small last round is left (then only its tiles split), and grids of full rounds run whole."""
    torch_cuda()
    mnk = lambda m, n, k: B.pf_gemm_workspace_size(m, n, k)
    assert mnk(2048, 1536, 1536) > 0          # 192 tiles: split
    assert mnk(1024, 1152, 4608) > 0          # 72 tiles: split
    assert mnk(2048, 3072, 12288) == 0        # 384 tiles: every CU has one, whole
    assert mnk(2048, 3072, 3072) == 0         # 384 tiles
    assert mnk(2048, 12288, 3072) == 0        # 1536 tiles: three full rounds
    assert mnk(2304, 4096, 1536) > 0          # 576 tiles: 64 left after a full round, those split
    assert mnk(2048, 4608, 1536) == 0         # 384 tiles of 192 x 128 (1.5 per CU): whole
    assert mnk(16384, 1152, 4608) == 0        # 768 tiles of 192 x 128
    assert mnk(2432, 3456, 1152) > 0          # 342 tiles of 192 x 128 (too few): 513 of 128, remainder split


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
    want_p = ref.attention(q[:, :h], K, V, H, D, round_p=True)
    assert_close(host(o), ref.bf16_round(want_p), f"attention bf16 D={D} S={S} rows={rows} vs bf16p")
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
    want_p = ref.attention(q[rows, :h], K, V, H, D, round_p=True)
    assert_close(got, ref.bf16_round(want_p), f"attention {cfg} full size, sampled rows vs bf16p")
    assert_close(got, want, f"attention {cfg} full size, sampled rows vs exact")


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
@pytest.mark.parametrize("D", [64, 72, 128])
def test_attention_bf16_single_key(D, split):
    """One key: every softmax row is the single weight 1, so each query's output is that key's V
    row.  The weight is bf16(2^(t - ceil t)) and the row sum the same value, so acc / l = v up to
    fp32 rounding, which bf16 rounds back to v: the output equals V[0] bit for bit, whatever Q."""
    torch = torch_cuda()
    H, rows = 3, 70
    h = H * D
    q = synth.randn((rows, h), 910 + D, std=3.0, bf16=True)
    K = synth.randn((1, h), 911 + D, bf16=True)
    V = synth.randn((1, h), 912 + D, bf16=True)
    kt, vt, kv = _kv_bf16(torch, K, V)
    ws = torch.empty((B.pf_attention_workspace_size(rows, H, D) or 1,), dtype=torch.uint8, device="cuda") \
        if split else None
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    print(f"[attention] single key D={D} split={split}", flush=True)
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, 1, rows, H, D, o, workspace=ws)
    got = host(o)
    assert np.array_equal(got, np.broadcast_to(V[0], got.shape)), "output differs from the single key's V row"


def test_degenerate_sizes_are_no_ops_or_errors():
    """Zero query rows (attention) and zero token rows (GEMM) launch nothing and leave the
    output untouched; an empty key range has no softmax and is rejected."""
    torch = torch_cuda()
    D, H = 64, 2
    h = H * D
    K = synth.randn((40, h), 920, bf16=True)
    V = synth.randn((40, h), 921, bf16=True)
    kt, vt, kv = _kv_bf16(torch, K, V)
    q = torch.zeros((4, h), dtype=torch.bfloat16, device="cuda")
    o = torch.full((4, h), 7.0, dtype=torch.bfloat16, device="cuda")
    B.pf_attention(q, kv, 40, 0, H, D, o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "rows = 0 wrote the output"
    with pytest.raises(B.PFError) as ei:
        B.pf_attention(q, kv, 0, 4, H, D, o)
    assert ei.value.status == B.PF_ERR_INVALID_ARG
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((128,), dtype=torch.float32, device="cuda")
    c = torch.full((4, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    B.pf_gemm(a, w, bias, B.PF_EPI_STORE, c, m=0)
    torch.cuda.synchronize()
    assert bool((c == 5.0).all()), "m = 0 wrote the output"


@pytest.mark.parametrize("D", [64, 72, 128])
def test_attention_bf16_closed_forms(D):
    torch = torch_cuda()
    H, S, rows = 2, 300, 70
    h = H * D
    K = synth.randn((S, h), 51, bf16=True)
    V = synth.randn((S, h), 52, bf16=True)
    q = synth.randn((rows, h), 53, bf16=True)
    # V = 1 -> every output is 1: the rounded weights are normalised by their own sum, so only
    # fp32 summation order separates l from the P.V row sums (far below one bf16 ulp of 1)
    kt, vt, kv = _kv_bf16(torch, K, np.ones_like(V))
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, rows, H, D, o)
    assert np.abs(host(o) - 1.0).max() <= 2.0 ** -8
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


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
@pytest.mark.parametrize("D", [64, 72, 128])
def test_attention_bf16_rescale_in_late_tiles(D, split):
    """Row maxima that rise after the first key tile, so the kernel raises its reference and
    rescales O and l in the middle of the key loop (and, with the split workspace, inside later
    slices, whose references the merge then combines).  S = 2100 keys = 66 tiles, the last one
    partial; 3 heads x 70 query rows fill 3 workgroups, so with the workspace the key range splits
    into 8 slices of 9 tiles (slice 1 = keys 288..575, slice 5 = keys 1440..1727).
      head 0: a ramp along one K column, 4 per key in base-2 score units over every 3 tiles for
              the rows with a positive query component (the reference rises again and again)
              and falling for the others (maximum in tile 0);
      head 1: one key of logit +40 in slice 1 (key 300) and one of +60 in slice 5 (key 1500);
      head 2: one key of logit +50 in the last, partial tile (key 2099).
    Checked against the bf16p oracle at the contract's tolerances and the exact oracle."""
    torch = torch_cuda()
    H, S, rows = 3, 2100, 70
    h = H * D
    seed = 8100 + D
    q = synth.randn((rows, h), seed, std=1.0)
    K = synth.randn((S, h), seed + 1, std=1.0)
    V = synth.randn((S, h), seed + 2, std=1.0, bf16=True)
    sq = math.sqrt(D)
    # head 0: ramp; logit slope q0 * a / sqrt(D) per key with q0 = +-4, a chosen for ~0.083 base-2 units per key
    q[:, 0] = np.where(np.arange(rows) % 2 == 0, 4.0, -4.0)
    K[:, 0] = np.arange(S) * (0.083 / math.log2(math.e)) * sq / 4.0
    # head 1: q = 8 along its first column; dominant keys at 300 (+40) and 1500 (+60)
    q[:, D] = 8.0
    K[300, D] = 40.0 * sq / 8.0
    K[1500, D] = 60.0 * sq / 8.0
    # head 2: dominant key in the last, partial tile (+50)
    q[:, 2 * D] = 8.0
    K[S - 1, 2 * D] = 50.0 * sq / 8.0
    q = synth.to_bf16_values(q).astype(np.float64)
    K = synth.to_bf16_values(K).astype(np.float64)
    kt, vt, kv = _kv_bf16(torch, K, V)
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    ws = B.attention_workspace(rows, H, D) if split else None
    print(f"[attn] rescale D={D} split={split}", flush=True)
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, rows, H, D, o, workspace=ws)
    got = host(o)
    want_p = ref.attention(q, K, V, H, D, round_p=True)
    want = ref.attention(q, K, V, H, D)
    assert_close(got, ref.bf16_round(want_p), f"attention rescale D={D} split={split} vs bf16p")
    assert_close(got, want, f"attention rescale D={D} split={split} vs exact")
    # the cases really exercise what they name: head 1 ends on key 1500, head 2 on key 2099
    np.testing.assert_allclose(got[:, D:2 * D], np.broadcast_to(V[1500, D:2 * D], (rows, D)), atol=1e-2)
    np.testing.assert_allclose(got[:, 2 * D:], np.broadcast_to(V[S - 1, 2 * D:], (rows, D)), atol=1e-2)


# Shapes whose work a 256-CU MI355X runs on the grouped stream-K schedule (each group of
# workgroups, one per query tile, takes an equal stretch of the (head, key tile) line, so
# stretches start and end inside heads and run over head boundaries): the key tiles per
# stretch are 59 (d = 64, 157 tiles per head), 54 (d = 72, 94 tiles) and 45 (d = 128, 129
# tiles), never a multiple of the tiles per head; every S ends in a partial tile.
SK_CASES = [(64, 24, 5000, 1664), (72, 24, 3000, 2688), (128, 8, 4100, 2688)]


@pytest.mark.parametrize("D,H,S,rows", SK_CASES)
def test_attention_bf16_stream_k(D, H, S, rows):
    """Key ranges cut into pieces that the merge pass recombines, with row maxima that move
    between pieces: head 0 has a key of logit +50 in the last, partial tile, head 1 one of +40
    a third of the way in and one of +60 two thirds of the way in (different pieces for the
    queries of every query tile), the other heads random logits.  Checked on 64 sampled query
    rows against the bf16p and the exact oracle."""
    torch = torch_cuda()
    h = H * D
    seed = 9100 + D
    q = synth.randn((rows, h), seed, std=1.0)
    K = synth.randn((S, h), seed + 1, std=1.0)
    V = synth.randn((S, h), seed + 2, std=1.0, bf16=True)
    sq = math.sqrt(D)
    q[:, 0] = 8.0
    K[S - 1, 0] = 50.0 * sq / 8.0
    q[:, D] = 8.0
    K[S // 3, D] = 40.0 * sq / 8.0
    K[2 * S // 3, D] = 60.0 * sq / 8.0
    q = synth.to_bf16_values(q).astype(np.float64)
    K = synth.to_bf16_values(K).astype(np.float64)
    kt, vt, kv = _kv_bf16(torch, K, V)
    o = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    print(f"[attn] stream-K D={D} H={H} S={S} rows={rows}", flush=True)
    B.pf_attention(dev(torch, q, torch.bfloat16), kv, S, rows, H, D, o, workspace=B.attention_workspace(rows, H, D))
    rng = np.random.default_rng(seed)
    sel = np.unique(np.concatenate([[0, 1, 511, 512, rows - 1], rng.choice(rows, 59, replace=False)]))
    got = host(o)[sel]
    want_p = ref.attention(q[sel], K, V, H, D, round_p=True)
    want = ref.attention(q[sel], K, V, H, D)
    assert_close(got, ref.bf16_round(want_p), f"attention stream-K D={D} vs bf16p")
    assert_close(got, want, f"attention stream-K D={D} vs exact")
    np.testing.assert_allclose(got[:, :D], np.broadcast_to(V[S - 1, :D], (len(sel), D)), atol=1e-2)
    np.testing.assert_allclose(got[:, D:2 * D], np.broadcast_to(V[2 * S // 3, D:2 * D], (len(sel), D)), atol=1e-2)


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
