"""KV-buffer splice on the GPU: bit-exact against the oracle's slice assignment,
every layout pair, edge offsets/lengths, canaries around the destination, and
invalid calls that must leave the destination untouched."""
import numpy as np
import pytest

from oracle import ref
from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth

from _util import torch_cuda

pytestmark = pytest.mark.gpu


def _k8_index(rows_idx, cols_idx, E):
    return ((rows_idx // 8) * E + cols_idx) * 8 + (rows_idx % 8)


def _to_dev(torch, a, dt):
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)).cuda()
    return t.view(dt)


def _to_host(torch, t, np_dtype):
    torch.cuda.synchronize()
    if np_dtype == np.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


CASES = [(100, 0, 100), (100, 0, 1), (100, 7, 1), (100, 99, 1), (100, 3, 7), (100, 8, 16), (100, 13, 50),
         (100, 40, 0), (1030, 256, 256), (1030, 1, 1029)]


@pytest.mark.parametrize("E", [64, 1152])
@pytest.mark.parametrize("R,off,n", CASES)
def test_splice_qkv_rows_into_k_rows_and_v_k8_bit_exact(E, R, off, n):
    torch = torch_cuda()
    seed = 100 + R + off * 7 + n * 13 + E
    CAN = 3                                          # canary rows before and after K
    k_store = synth.rand_bits16((R + 2 * CAN, E), seed)
    g = (R + 7) // 8
    v_store = synth.rand_bits16((g * 8 * E + 64,), seed + 1)      # + canary tail
    src = synth.rand_bits16((max(n, 1), 3 * E), seed + 2)
    k_dev = _to_dev(torch, k_store, torch.bfloat16)
    v_dev = _to_dev(torch, v_store, torch.bfloat16)
    s_dev = _to_dev(torch, src, torch.bfloat16)
    esz = 2
    dst = B.KVView(k=k_dev.data_ptr() + CAN * E * esz, v=v_dev.data_ptr(), rows=R, row_elems=E, k_ld=E, v_ld=E,
                   dtype=B.PF_BF16, v_layout=B.PF_LAYOUT_K8)
    srcv = B.KVView(k=s_dev.data_ptr() + E * esz, v=s_dev.data_ptr() + 2 * E * esz, rows=max(n, 1), row_elems=E,
                    k_ld=3 * E, v_ld=3 * E, dtype=B.PF_BF16, v_layout=B.PF_LAYOUT_ROWS)
    print(f"[splice] E={E} R={R} off={off} n={n}", flush=True)
    B.kvbuf_splice(dst, srcv, off, n)
    k_after = _to_host(torch, k_dev, np.uint16)
    v_after = _to_host(torch, v_dev, np.uint16)

    k_want = k_store.copy()
    ref.splice(k_want[CAN:CAN + R], src[:n, E:2 * E], off)
    np.testing.assert_array_equal(k_after, k_want)

    v_want = v_store.copy()
    if n:
        r, c = np.meshgrid(np.arange(off, off + n), np.arange(E), indexing="ij")
        v_want[_k8_index(r, c, E)] = src[:n, 2 * E:3 * E]
    np.testing.assert_array_equal(v_after, v_want)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("R,off,n", [(64, 0, 64), (77, 5, 33), (77, 76, 1), (300, 100, 200)])
def test_splice_rows_to_rows_strided_bit_exact(dtype, R, off, n):
    torch = torch_cuda()
    E, ld = 128, 136
    if dtype == "bf16":
        npd, tdt, pdt, esz = np.uint16, torch.bfloat16, B.PF_BF16, 2
        gen = synth.rand_bits16
    else:
        npd, tdt, pdt, esz = np.uint32, torch.float32, B.PF_FP32, 4
        gen = synth.rand_bits32
    dk, dv = gen((R + 2, ld), 7 + R), gen((R + 2, ld), 8 + R)
    sk, sv = gen((n, E), 9 + n), gen((n, E), 10 + n)
    t = [_to_dev(torch, a, tdt) for a in (dk, dv, sk, sv)]
    dst = B.KVView(k=t[0].data_ptr() + ld * esz, v=t[1].data_ptr() + ld * esz, rows=R, row_elems=E, k_ld=ld, v_ld=ld,
                   dtype=pdt, v_layout=B.PF_LAYOUT_ROWS)
    src = B.KVView(k=t[2].data_ptr(), v=t[3].data_ptr(), rows=n, row_elems=E, k_ld=E, v_ld=E, dtype=pdt,
                   v_layout=B.PF_LAYOUT_ROWS)
    B.kvbuf_splice(dst, src, off, n)
    for dev_t, before, s in ((t[0], dk, sk), (t[1], dv, sv)):
        want = before.copy()
        ref.splice(want[1:1 + R, :E], s, off)
        np.testing.assert_array_equal(_to_host(torch, dev_t, npd), want)


@pytest.mark.parametrize("R,off,n", [(64, 0, 64), (100, 8, 40), (100, 3, 50)])
def test_splice_k8_sources(R, off, n):
    """K8 -> K8 (checkpoint restore) and K8 -> rows (read-back) take the element path; still bit exact."""
    torch = torch_cuda()
    E = 64
    gs = (n + 7) // 8
    src_v = synth.rand_bits16((gs * 8 * E,), 31 + n)
    src_k = synth.rand_bits16((n, E), 32 + n)
    gd = (R + 7) // 8
    dst_v = synth.rand_bits16((gd * 8 * E,), 33 + R)
    dst_k = synth.rand_bits16((R, E), 34 + R)
    rows_v = synth.rand_bits16((R, E), 35 + R)
    t = [_to_dev(torch, a, torch.bfloat16) for a in (src_k, src_v, dst_k, dst_v, rows_v)]
    src = B.KVView(k=t[0].data_ptr(), v=t[1].data_ptr(), rows=n, row_elems=E, k_ld=E, v_ld=E, dtype=B.PF_BF16,
                   v_layout=B.PF_LAYOUT_K8)
    dst = B.KVView(k=t[2].data_ptr(), v=t[3].data_ptr(), rows=R, row_elems=E, k_ld=E, v_ld=E, dtype=B.PF_BF16,
                   v_layout=B.PF_LAYOUT_K8)
    B.kvbuf_splice(dst, src, off, n)
    src_v_rows = src_v[_k8_index(*np.meshgrid(np.arange(n), np.arange(E), indexing="ij"), E)]
    want_v = dst_v.copy()
    r, c = np.meshgrid(np.arange(off, off + n), np.arange(E), indexing="ij")
    want_v[_k8_index(r, c, E)] = src_v_rows
    np.testing.assert_array_equal(_to_host(torch, t[3], np.uint16), want_v)
    want_k = dst_k.copy()
    ref.splice(want_k, src_k, off)
    np.testing.assert_array_equal(_to_host(torch, t[2], np.uint16), want_k)
    # K8 -> rows
    dst2 = B.KVView(k=t[2].data_ptr(), v=t[4].data_ptr(), rows=R, row_elems=E, k_ld=E, v_ld=E, dtype=B.PF_BF16,
                    v_layout=B.PF_LAYOUT_ROWS)
    B.kvbuf_splice(dst2, src, off, n)
    want_rows = rows_v.copy()
    ref.splice(want_rows, src_v_rows, off)
    np.testing.assert_array_equal(_to_host(torch, t[4], np.uint16), want_rows)


def test_invalid_splice_writes_nothing():
    torch = torch_cuda()
    E, R = 64, 40
    buf = synth.rand_bits16((R, E), 41)
    t = _to_dev(torch, buf, torch.bfloat16)
    tv = _to_dev(torch, synth.rand_bits16((R, E), 42), torch.bfloat16)
    dst = B.KVView(k=t.data_ptr(), v=tv.data_ptr(), rows=R, row_elems=E, k_ld=E, v_ld=E, dtype=B.PF_BF16,
                   v_layout=B.PF_LAYOUT_ROWS)
    src = B.KVView(k=t.data_ptr() + 10 * E * 2, v=tv.data_ptr() + 10 * E * 2, rows=20, row_elems=E, k_ld=E,
                   v_ld=E, dtype=B.PF_BF16, v_layout=B.PF_LAYOUT_ROWS)
    with pytest.raises(B.PFError) as ei:
        B.kvbuf_splice(dst, src, 5, 20)          # overlapping source and destination
    assert ei.value.status == B.PF_ERR_INVALID_ARG
    with pytest.raises(B.PFError):
        B.kvbuf_splice(dst, src, 30, 20)         # past the end
    np.testing.assert_array_equal(_to_host(torch, t, np.uint16), buf)


@pytest.mark.parametrize("m,off,split", [(1024, 1024, False), (77, 1003, False), (300, 8, True), (1, 4095, True),
                                         (2432, 1003, True), (3000, 1001, False), (3002, 1000, False)],
                         ids=["patch", "ragged", "ksplit", "one-row-ksplit", "remainder-split", "wide-tiles",
                              "wide-tiles-aligned"])
def test_fused_qkv_splice_matches_gemm_then_splice(m, off, split):
    """The stage's QKV projection writes K and V straight into the buffer (pf_gemm_qkv_splice).
    Its Q and every byte of the buffer must equal the unfused path, pf_gemm(PF_EPI_STORE) then
    kvbuf_splice of the K and V columns (itself bit-exact against the oracle's slice
    assignment above): same rows replaced, including partial 8-row groups of the K8 layout,
    and nothing else touched.  2432 rows make 513 tiles of 128 x 128: one full round of 512
    slots plus one tile, which the plan runs as k slices finished by a reduce pass.  3000 rows
    make 24 x 18 tiles of 192 features x 128 tokens, which run whole with that tile (offsets 1000
    and 1001: whole and partial 8-row groups of the K8 layout at both ends of the range)."""
    import math
    from _util import dev
    torch = torch_cuda()
    E, R = 1152, 4096
    seed = 7000 + m + off
    a = synth.randn((m, E), seed, bf16=True)
    w = synth.randn((3 * E, E), seed + 1, std=1.0 / math.sqrt(E), bf16=True)
    bias = synth.randn((3 * E,), seed + 2, std=0.5)
    k0 = synth.rand_bits16((R, E), seed + 3)
    v0 = synth.rand_bits16((R * E,), seed + 4)
    bufs = [(_to_dev(torch, k0, torch.bfloat16), _to_dev(torch, v0, torch.bfloat16)) for _ in range(2)]
    views = [B.KVView(k=k.data_ptr(), v=v.data_ptr(), rows=R, row_elems=E, k_ld=E, v_ld=E, dtype=B.PF_BF16,
                      v_layout=B.PF_LAYOUT_K8) for k, v in bufs]
    ws = B.gemm_workspace(m, 3 * E, E) if split else None
    if split:
        assert ws is not None, "shape expected to split k"
    a_d, w_d, b_d = dev(torch, a, torch.bfloat16), dev(torch, w, torch.bfloat16), dev(torch, bias)
    print(f"[fused qkv splice] m={m} off={off} split={split}", flush=True)
    q = torch.empty((m, E), dtype=torch.bfloat16, device="cuda")
    B.pf_gemm_qkv_splice(a_d, w_d, b_d, q, views[0], off, workspace=ws)
    qkv = torch.empty((m, 3 * E), dtype=torch.bfloat16, device="cuda")
    B.pf_gemm(a_d, w_d, b_d, B.PF_EPI_STORE, qkv, workspace=ws)
    src = B.KVView(k=qkv.data_ptr() + E * 2, v=qkv.data_ptr() + 2 * E * 2, rows=m, row_elems=E, k_ld=3 * E,
                   v_ld=3 * E, dtype=B.PF_BF16, v_layout=B.PF_LAYOUT_ROWS)
    B.kvbuf_splice(views[1], src, off, m)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), qkv[:, :E].contiguous().view(torch.int16)), "Q differs"
    for i, name in ((0, "K"), (1, "V")):
        got, want = bufs[0][i].view(torch.int16), bufs[1][i].view(torch.int16)
        assert torch.equal(got, want), f"{name} buffer differs from gemm + kvbuf_splice"
    # rows outside the patch keep their old bits (the unfused path is checked against the oracle above)
    k_after = _to_host(torch, bufs[0][0], np.uint16)
    assert np.array_equal(k_after[:off], k0[:off]) and np.array_equal(k_after[off + m:], k0[off + m:])
