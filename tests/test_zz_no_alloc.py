"""The allocation-free attention entry point (pf_attention_noalloc: split partials in the
library's static device scratch) against pf_attention with a workspace, bit for bit, on two
calls in a row, the second smaller; and its size limit."""
import numpy as np
import pytest

from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth
from patch_pipelined_attention_amd.stage import rows_to_k8

from _util import dev, torch_cuda

pytestmark = pytest.mark.gpu


def _case(torch, rows, S, H, D, seed):
    h = H * D
    q = dev(torch, synth.randn((rows, 3 * h), seed, bf16=True), torch.bfloat16)
    k = dev(torch, synth.randn((S, h), seed + 1, bf16=True), torch.bfloat16)
    v = dev(torch, rows_to_k8(synth.randn((S, h), seed + 2, bf16=True)), torch.bfloat16)
    return q, k, v, B.kv_view(k, v, S, h, B.PF_LAYOUT_K8)


@pytest.mark.parametrize("first,second", [((1024, 4096, 16, 72), (300, 2100, 3, 64)),
                                          ((2048, 16384, 24, 64), (70, 5000, 2, 128))])
def test_attention_noalloc_matches_workspace_entry_point(first, second):
    torch = torch_cuda()
    for i, (rows, S, H, D) in enumerate((first, second)):
        print(f"[noalloc] call {i}: rows={rows} S={S} H={H} D={D}", flush=True)
        q, k, v, kv = _case(torch, rows, S, H, D, 500 + 10 * i + D)
        h = H * D
        o_ref = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
        o = torch.full((rows, h), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.pf_attention(q, kv, S, rows, H, D, o_ref, ldq=3 * h, workspace=B.attention_workspace(rows, H, D))
        B.pf_attention_noalloc(q, kv, S, rows, H, D, o, ldq=3 * h)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"call {i} differs from pf_attention"


def test_attention_noalloc_rejects_splits_beyond_the_scratch():
    """6144 query rows x 24 heads x 128 over 32768 keys, split 4 ways, need 307 MB of partials:
    rejected before any launch (the output keeps its contents)."""
    torch = torch_cuda()
    rows, S, H, D = 6144, 32768, 24, 128
    h = H * D
    q = torch.zeros((rows, h), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((S, h), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((S * h,), dtype=torch.bfloat16, device="cuda")
    kv = B.kv_view(k, v, S, h, B.PF_LAYOUT_K8)
    o = torch.full((rows, h), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.PFError) as e:
        B.pf_attention_noalloc(q, kv, S, rows, H, D, o)
    assert e.value.status == B.PF_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
