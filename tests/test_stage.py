"""Stage-level parity of the HIP path against the fp64 oracle, plus the properties
the PipeFusion summaries fix: (a) fresh == stale context reproduces unpartitioned
full attention, (b) a micro-step changes only its own buffer rows, stale step-(T+1)
rows elsewhere; determinism; call-order errors."""
import dataclasses

import numpy as np
import pytest

from oracle import ref
from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth
from patch_pipelined_attention_amd.configs import C1, C2, C3, C4, C5
from patch_pipelined_attention_amd.stage import Stage

from _util import MAX_ABS, REL_L2, assert_bf16_close, assert_close, dev, host, max_abs, torch_cuda

pytestmark = pytest.mark.gpu


def _oracle(shape, inputs, mode):
    return ref.StageOracle(inputs.layers, heads=shape.heads, head_dim=shape.head_dim, seq_txt=shape.seq_txt,
                           seq_img=shape.seq_img, num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio,
                           mode=mode)


SMALL = {
    "c2s": C2.small(seq_img=400, num_layers=2),                          # D=72, P=100: ragged tiles
    "c3s": C3.small(seq_img=1024, num_layers=2),                         # D=64, M=8, P=128
    "c4s": C4.small(seq_img=256, num_layers=2, seq_txt=40),              # D=128, ragged text prefix
    "c5s": C5.small(seq_img=2048, num_layers=1, num_patches=16),         # D=72, M=16
}


def stage_output_max_abs_tol(want_b, want_p):
    """Max-abs gate for a stage output against the bf16-in oracle: the contract's 2e-2, or twice
    the deviation that rounding the softmax weights to bf16 alone causes in the oracle (bf16p vs
    bf16), whichever is larger.  Deep, wide stages amplify that rounding through later bf16
    rounding points (rounding flips), so no bf16 flash-attention path can sit closer."""
    return max(MAX_ABS, 2.0 * max_abs(want_p, want_b))


def _run_chain(shape, steps, check_exact=True):
    torch = torch_cuda()
    inputs = synth.stage_inputs(shape)
    bf16 = shape.dtype == "bf16"
    orc_b = _oracle(shape, inputs, "bf16") if bf16 else None
    orc_p = _oracle(shape, inputs, "bf16p") if bf16 else None
    orc_e = _oracle(shape, inputs, "exact")
    with Stage(shape) as st:
        st.load(inputs.layers)
        x = dev(torch, inputs.x)
        c = dev(torch, inputs.c)
        out = torch.empty_like(x)
        for s in range(steps):
            warm = s == 0
            if s > 0:
                noise = inputs.next_noise()
                st.add_noise(noise)
                orc_e.add_noise(noise)
                if orc_b:
                    orc_b.add_noise(noise)
                    orc_p.add_noise(noise)
            print(f"[stage] {shape.name} step {s} warmup={warm}", flush=True)
            st.run_step(x, c, warmup=warm, out=out)
            got = host(out)
            want_e = orc_e.step(inputs.x, inputs.c, warmup=warm)
            if bf16:
                want_b = orc_b.step(inputs.x, inputs.c, warmup=warm)
                want_p = orc_p.step(inputs.x, inputs.c, warmup=warm)
                tol = stage_output_max_abs_tol(want_b, want_p)
                assert_close(want_p, want_b, f"{shape.name} step {s} bf16p oracle vs bf16-in oracle (floor)",
                             max_abs_tol=None, rel_tol=None)
                assert_close(got, want_b, f"{shape.name} step {s} vs bf16-in oracle", max_abs_tol=tol)
                if check_exact:
                    assert_close(got, want_e, f"{shape.name} step {s} vs exact oracle", max_abs_tol=None)
                for l in range(shape.num_layers):
                    k, v = st.kv_get(l)
                    fk = 2.0 * max_abs(orc_p.K[l], orc_b.K[l])
                    fv = 2.0 * max_abs(orc_p.V[l], orc_b.V[l])
                    assert_bf16_close(k, orc_b.K[l], f"{shape.name} step {s} K[{l}]", floor=fk)
                    assert_bf16_close(v, orc_b.V[l], f"{shape.name} step {s} V[{l}]", floor=fv)
            else:
                assert_close(got, want_e, f"{shape.name} step {s} vs exact oracle", max_abs_tol=1e-3, rel_tol=1e-5)
                for l in range(shape.num_layers):
                    k, v = st.kv_get(l)
                    assert_close(k, orc_e.K[l], f"{shape.name} step {s} K[{l}]", max_abs_tol=1e-4, rel_tol=1e-5)
                    assert_close(v, orc_e.V[l], f"{shape.name} step {s} V[{l}]", max_abs_tol=1e-4, rel_tol=1e-5)


def test_c1_tiny_fp32_all_steps():
    _run_chain(C1, C1.steps)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_bf16_stage_chain(name):
    _run_chain(SMALL[name], 3)


def _run_pair_chain(shape, steps):
    """A classifier-free guidance pair through one batched stage: both samples share the
    latent rows and the weights, each has its own condition (the second stands in for the
    unconditional embedding), its own drift between steps and its own K/V buffers.  Each
    sample must match its own oracle stage, which never sees the other sample."""
    torch = torch_cuda()
    inputs = synth.stage_inputs(shape)
    conds = list(synth.batch_conds(shape, inputs.c, 2))
    bf16 = shape.dtype == "bf16"
    orc_b = [_oracle(shape, inputs, "bf16" if bf16 else "exact") for _ in range(2)]
    orc_p = [_oracle(shape, inputs, "bf16p") for _ in range(2)] if bf16 else None
    S, h, L = shape.seq_kv, shape.hidden, shape.num_layers
    with Stage(shape, batch=2) as st:
        st.load(inputs.layers)
        x = dev(torch, np.stack([inputs.x, inputs.x]))
        c = dev(torch, np.stack(conds))
        out = torch.empty_like(x)
        for s in range(steps):
            warm = s == 0
            if s > 0:
                for b in range(2):
                    seed = shape.seed + 100 * s + 10 * b
                    noise = [(synth.randn((S, h), seed + 2 * l, std=shape.sigma_kv),
                              synth.randn((S, h), seed + 2 * l + 1, std=shape.sigma_kv)) for l in range(L)]
                    st.add_noise(noise, sample=b)
                    orc_b[b].add_noise(noise)
                    if bf16:
                        orc_p[b].add_noise(noise)
            print(f"[stage pair] {shape.name} step {s} warmup={warm}", flush=True)
            st.run_step(x, c, warmup=warm, out=out)
            got = host(out)
            for b in range(2):
                want = orc_b[b].step(inputs.x, conds[b], warmup=warm)
                if bf16:
                    want_p = orc_p[b].step(inputs.x, conds[b], warmup=warm)
                    tol = stage_output_max_abs_tol(want, want_p)
                    assert_close(got[b], want, f"{shape.name} pair step {s} sample {b} vs bf16-in oracle",
                                 max_abs_tol=tol)
                    for l in range(L):
                        k, v = st.kv_get(l, sample=b)
                        assert_bf16_close(k, orc_b[b].K[l], f"pair step {s} sample {b} K[{l}]",
                                          floor=2.0 * max_abs(orc_p[b].K[l], orc_b[b].K[l]))
                        assert_bf16_close(v, orc_b[b].V[l], f"pair step {s} sample {b} V[{l}]",
                                          floor=2.0 * max_abs(orc_p[b].V[l], orc_b[b].V[l]))
                else:
                    assert_close(got[b], want, f"{shape.name} pair step {s} sample {b} vs exact oracle",
                                 max_abs_tol=1e-3, rel_tol=1e-5)
                    for l in range(L):
                        k, v = st.kv_get(l, sample=b)
                        assert_close(k, orc_b[b].K[l], f"pair step {s} sample {b} K[{l}]", max_abs_tol=1e-4,
                                     rel_tol=1e-5)
                        assert_close(v, orc_b[b].V[l], f"pair step {s} sample {b} V[{l}]", max_abs_tol=1e-4,
                                     rel_tol=1e-5)
            # the two samples really differ (different conditions reach every row)
            assert max_abs(got[0], got[1]) > 1e-3


@pytest.mark.parametrize("name", ["c1", "c2s", "c4s"])
def test_cfg_pair_stage_chain(name):
    shape = C1 if name == "c1" else SMALL[name]
    _run_pair_chain(shape, 3)


@pytest.mark.parametrize("name", ["c2s", "c2-full-L1", "c4-full-L1"])
def test_cfg_pair_patch_matches_single_stages(name):
    """stage_run_patch on a pair equals the same micro-step on two single-sample stages, each
    with that sample's condition and buffer contents (up to the fp32 summation order of
    projections that see twice the rows, and of the key-range split: at full size the pair's
    batched attention splits the keys in fewer slices than a single sample's)."""
    torch = torch_cuda()
    shape = {"c2s": SMALL["c2s"], "c2-full-L1": dataclasses.replace(C2, num_layers=1),
             "c4-full-L1": dataclasses.replace(C4, num_layers=1)}[name]
    inputs = synth.stage_inputs(shape)
    conds = list(synth.batch_conds(shape, inputs.c, 2))
    P, off = shape.patch_rows, shape.patch_offsets()[1]
    x_patch = inputs.x[off:off + P]
    with Stage(shape, batch=2) as pair, Stage(shape) as s0, Stage(shape) as s1:
        singles = [s0, s1]
        for st in (pair, s0, s1):
            st.load(inputs.layers)
        # fill every buffer with a warm-up step of its own condition
        x_all = dev(torch, inputs.x)
        pair.run_step(dev(torch, np.stack([inputs.x, inputs.x])), dev(torch, np.stack(conds)), warmup=True,
                      out=torch.empty((2, shape.seq_kv, shape.hidden), device="cuda"))
        for b, st in enumerate(singles):
            st.run_step(x_all, dev(torch, conds[b]), warmup=True, out=torch.empty_like(x_all))
        pair.set_cond(dev(torch, np.stack(conds)))
        got = host(pair.run_patch(off, P, dev(torch, np.stack([x_patch, x_patch]))))
        for b, st in enumerate(singles):
            st.set_cond(dev(torch, conds[b]))
            want = host(st.run_patch(off, P, dev(torch, x_patch)))
            # rel-L2 is the contract tolerance; max-abs only bounds gross errors, because at
            # h = 3072 the large adaLN gates turn one-ulp bf16 flips into ~0.1 single-element moves
            assert_close(got[b], want, f"pair patch sample {b} vs single stage", max_abs_tol=0.25)
            for l in range(shape.num_layers):
                kp, vp = pair.kv_get(l, sample=b)
                ks, vs = st.kv_get(l)
                assert_bf16_close(kp, ks, f"pair patch sample {b} K[{l}] vs single stage")
                assert_bf16_close(vp, vs, f"pair patch sample {b} V[{l}] vs single stage")


def test_property_a_single_patch_overwrites_stale_context():
    """M = 1: the patch splices every row before attending, so any stale content is irrelevant."""
    torch = torch_cuda()
    shape = dataclasses.replace(C3.small(seq_img=512, num_layers=2), num_patches=1)
    inputs = synth.stage_inputs(shape)
    with Stage(shape) as st:
        st.load(inputs.layers)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        warm = host(st.run_step(x, c, warmup=True, out=torch.empty_like(x)))
        rng = np.random.default_rng(3)
        for l in range(shape.num_layers):
            k, v = st.kv_get(l)
            st.kv_set(l, k + 30 * rng.standard_normal(k.shape), v + 30 * rng.standard_normal(v.shape))
        patched = host(st.run_step(x, c, warmup=False, out=torch.empty_like(x)))
        np.testing.assert_array_equal(patched, warm)


@pytest.mark.parametrize("shape", [C2, C3, C4], ids=lambda s: s.name)
def test_property_a_no_drift_full_size(shape):
    """At full size and in the benchmark's launch configuration: with no drift between steps
    (fresh == stale) a patched step reproduces the warm-up (unpartitioned) step.  The first
    layer's K/V buffers see the same inputs; they agree to within one bf16 ulp per element
    (plus a tiny absolute floor for sums that cancel), since a patch-sized QKV projection may
    split its k range across workgroups (fp32 partial sums added in another order) while the
    warm-up pass does not.  The outputs agree up to
    fp32 summation order too: a patch's attention also splits the key range and merges the
    partials, and later bf16 rounding points turn last-bit differences into occasional
    one-ulp flips."""
    torch = torch_cuda()
    shape = dataclasses.replace(shape, num_layers=min(shape.num_layers, 2))
    inputs = synth.stage_inputs(shape)
    with Stage(shape) as st:
        st.load(inputs.layers)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        print(f"[stage] {shape.name} full-size property (a)", flush=True)
        warm = st.run_step(x, c, warmup=True, out=torch.empty_like(x)).clone()
        k0, v0 = st.kv_raw(0)
        out = torch.empty_like(x)
        st.run_step(x, c, warmup=False, out=out)
        torch.cuda.synchronize()
        k1, v1 = st.kv_raw(0)
        for name, a, b in (("K", k0, k1), ("V", v0, v1)):
            a, b = a.float(), b.float()
            # one bf16 ulp of either value, plus an absolute floor for results that cancel to
            # near zero, where a reordered fp32 sum (|error| ~ 1e-7 of the summed magnitudes)
            # exceeds the ulp of the result itself
            tol = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 2.0 ** -19
            d = (a - b).abs()
            bad = d > tol
            assert not bool(bad.any()), (f"layer-0 {name}: {int(bad.sum())} elements beyond one bf16 ulp, "
                                         f"max |diff| {float(d.max()):.3g} at |value| "
                                         f"{float(a.flatten()[int(d.argmax())].abs()):.3g}")
        assert bool(torch.isfinite(out).all())
        # rel-L2 is the contract tolerance; max-abs only bounds gross errors here, because at
        # h = 3072 the large adaLN gates turn one-ulp bf16 flips into ~0.1 single-element moves
        assert_close(host(out), host(warm), f"{shape.name} patched vs warm-up (no drift)", max_abs_tol=0.25)


@pytest.mark.parametrize("shape", [C2, C3, C4], ids=lambda s: s.name)
def test_full_size_one_layer_sampled_parity(shape):
    """Full sequence length and width, one layer: warm-up and one drifted patched step,
    checked against the oracle on sampled rows of every patch."""
    torch = torch_cuda()
    shape = dataclasses.replace(shape, num_layers=1, name=shape.name + "-L1")
    inputs = synth.stage_inputs(shape)
    orc = _oracle(shape, inputs, "bf16")
    orc_p = _oracle(shape, inputs, "bf16p")
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(shape.seq_kv, 96, replace=False),
                                     [0, shape.seq_kv - 1] + list(shape.patch_offsets())]))
    with Stage(shape) as st:
        st.load(inputs.layers)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        out = torch.empty_like(x)
        for s in range(2):
            if s == 1:
                noise = inputs.next_noise()
                st.add_noise(noise)
                orc.add_noise(noise)
                orc_p.add_noise(noise)
            print(f"[stage] {shape.name} sampled step {s}", flush=True)
            st.run_step(x, c, warmup=(s == 0), out=out)
            got = host(out)[rows]
            want = orc.step_sampled(inputs.x, inputs.c, rows, warmup=(s == 0))
            want_p = orc_p.step_sampled(inputs.x, inputs.c, rows, warmup=(s == 0))
            assert_close(want_p, want, f"{shape.name} step {s} bf16p vs bf16-in oracle (floor)", max_abs_tol=None,
                         rel_tol=None)
            assert_close(got, want, f"{shape.name} step {s} sampled rows vs bf16-in oracle",
                         max_abs_tol=stage_output_max_abs_tol(want, want_p))
            k, v = st.kv_get(0)
            assert_bf16_close(k, orc.K[0], f"{shape.name} step {s} K buffer")
            assert_bf16_close(v, orc.V[0], f"{shape.name} step {s} V buffer")


def test_property_b_micro_steps_touch_only_their_rows():
    torch = torch_cuda()
    shape = SMALL["c4s"]
    inputs = synth.stage_inputs(shape)
    orc = _oracle(shape, inputs, "bf16")
    orc_p = _oracle(shape, inputs, "bf16p")
    with Stage(shape) as st:
        st.load(inputs.layers)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        st.run_step(x, c, warmup=True, out=torch.empty_like(x))
        orc.step(inputs.x, inputs.c, warmup=True)
        orc_p.step(inputs.x, inputs.c, warmup=True)
        noise = inputs.next_noise()
        st.add_noise(noise)
        orc.add_noise(noise)
        orc_p.add_noise(noise)
        st.set_cond(c)
        orc.set_cond(inputs.c)
        orc_p.set_cond(inputs.c)
        xo = x.clone()
        h = shape.hidden
        for off, n in orc.micro_steps(False):
            before = [st.kv_get(l) for l in range(shape.num_layers)]
            st.run_patch(off, n, x[off:off + n], xo[off:off + n])
            orc.run_rows(off, n, inputs.x[off:off + n])
            orc_p.run_rows(off, n, inputs.x[off:off + n])
            rs = slice(off, off + n)
            for l in range(shape.num_layers):
                k, v = st.kv_get(l)
                outside = np.ones(shape.seq_kv, bool)
                outside[rs] = False
                np.testing.assert_array_equal(k[outside], before[l][0][outside])
                np.testing.assert_array_equal(v[outside], before[l][1][outside])
                fk = 2.0 * max_abs(orc_p.K[l][rs], orc.K[l][rs])
                fv = 2.0 * max_abs(orc_p.V[l][rs], orc.V[l][rs])
                assert_bf16_close(k[rs], orc.K[l][rs], f"fresh K rows [{off},{off + n}) layer {l}", floor=fk)
                assert_bf16_close(v[rs], orc.V[l][rs], f"fresh V rows [{off},{off + n}) layer {l}", floor=fv)
        assert h == shape.hidden


def test_deterministic_bytes():
    torch = torch_cuda()
    shape = SMALL["c2s"]
    inputs = synth.stage_inputs(shape)
    outs = []
    for _ in range(2):
        with Stage(shape) as st:
            st.load(inputs.layers)
            x, c = dev(torch, inputs.x), dev(torch, inputs.c)
            st.run_step(x, c, warmup=True, out=torch.empty_like(x))
            outs.append(st.run_step(x, c, warmup=False, out=torch.empty_like(x)).clone())
    assert torch.equal(outs[0], outs[1])


def test_call_order_and_range_errors():
    torch = torch_cuda()
    shape = C1
    inputs = synth.stage_inputs(shape)
    with Stage(shape) as st:
        x = dev(torch, inputs.x)
        c = dev(torch, inputs.c)
        with pytest.raises(B.PFError) as ei:
            st.run_step(x, c, warmup=True)
        assert ei.value.status == B.PF_ERR_STATE
        st.load(inputs.layers)
        with pytest.raises(B.PFError) as ei:
            B.stage_run_patch(st.handle, 0, 64, x, x)          # condition not set yet
        assert ei.value.status == B.PF_ERR_STATE
        st.set_cond(c)
        for off, n in [(-1, 4), (0, 0), (250, 7)]:
            with pytest.raises(B.PFError) as ei:
                B.stage_run_patch(st.handle, off, n, x, x)
            assert ei.value.status == B.PF_ERR_INVALID_ARG
        with pytest.raises(B.PFError):
            B.stage_get_kvbuf(st.handle, 1)
        view = st.kv_view(0)
        assert view.rows == shape.seq_kv and view.row_elems == shape.hidden
        assert view.v_layout == B.PF_LAYOUT_ROWS and view.dtype == B.PF_FP32
