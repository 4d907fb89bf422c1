"""MM-DiT block options of the stage (the SD3 / Flux.1 models of the PipeFusion experiments):
dual-stream text weights, per-head QK-RMSNorm and rotary Q/K, each alone and together, and the
parallel (Flux.1 single-stream) block, against the fp64 oracle stage with the same options
(bf16-in mode with bf16 probabilities), over a warm-up step and patched steps with drifted stale context; guidance
pairs; the QK step as a component; call-order errors."""
import dataclasses

import numpy as np
import pytest

from oracle import ref
from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth
from patch_pipelined_attention_amd.configs import C2, C3, C4
from patch_pipelined_attention_amd.stage import Stage

from _util import (assert_bf16_close, assert_close, bf16_ulp, chain_elementwise, chain_max_abs_tol, dev, host, max_abs,
                   pair_norms, torch_cuda)
from test_stage import check_stage_output

pytestmark = pytest.mark.gpu

SHAPES = {
    "c3s": C3.small(seq_img=1024, num_layers=2, seq_txt=77),    # D=64, M=8, ragged text prefix
    "c4s": C4.small(seq_img=256, num_layers=2, seq_txt=40),     # D=128
    "c2s": C2.small(seq_img=400, num_layers=2, seq_txt=24),     # D=72, P=100
}

# (shape, qk_norm, dual_stream, rope)
CASES = {
    "c4s-all": ("c4s", True, True, True),
    "c4s-dual": ("c4s", False, True, False),
    "c3s-qknorm": ("c3s", True, False, False),
    "c3s-dual-qknorm": ("c3s", True, True, False),
    "c2s-rope": ("c2s", False, False, True),
    "c2s-all": ("c2s", True, True, True),
}


def k_bound(k_want, qk_norm, rope):
    """Element bound for the K buffer (see assert_bf16_close): one ulp for the plain projection
    output, three for K normalised or rotated after it, scaled by the pair norm when rotated."""
    if not (qk_norm or rope):
        return {}
    return {"ulps": 3, "scale": pair_norms(k_want) if rope else None}


def _oracle(shape, mm, mode, qk_norm, dual, rope):
    return ref.StageOracle(mm.layers, heads=shape.heads, head_dim=shape.head_dim, seq_txt=shape.seq_txt,
                           seq_img=shape.seq_img, num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio,
                           mode=mode, txt_layers=mm.txt_layers if dual else None, qk_norm=qk_norm,
                           rope_angles=mm.angles if rope else None)


def _stage(shape, mm, qk_norm, dual, rope, batch=1):
    st = Stage(shape, batch=batch, qk_norm=qk_norm, dual_stream=dual, rope=rope)
    st.load(mm.layers, mm.txt_layers if dual else None)
    if rope:
        st.set_rope(mm.angles)
    return st


@pytest.mark.parametrize("case", sorted(CASES))
def test_mmdit_stage_chain(case):
    name, qk_norm, dual, rope = CASES[case]
    shape = SHAPES[name]
    torch = torch_cuda()
    inputs = synth.stage_inputs(shape)
    mm = synth.mmdit_inputs(shape, inputs)
    orc_b = _oracle(shape, mm, "bf16", qk_norm, dual, rope)
    orc_p = _oracle(shape, mm, "bf16p", qk_norm, dual, rope)
    orc_e = _oracle(shape, mm, "exact", qk_norm, dual, rope)
    with _stage(shape, mm, qk_norm, dual, rope) as st:
        x = dev(torch, inputs.x)
        c = dev(torch, inputs.c)
        out = torch.empty_like(x)
        for s in range(3):
            warm = s == 0
            if s > 0:
                noise = inputs.next_noise()
                st.add_noise(noise)
                orc_b.add_noise(noise)
                orc_p.add_noise(noise)
                orc_e.add_noise(noise)
            print(f"[mmdit] {case} step {s} warmup={warm}", flush=True)
            st.run_step(x, c, warmup=warm, out=out)
            got = host(out)
            want = orc_b.step(inputs.x, inputs.c, warmup=warm)
            want_p = orc_p.step(inputs.x, inputs.c, warmup=warm)
            want_e = orc_e.step(inputs.x, inputs.c, warmup=warm)
            check_stage_output(got, want_p, f"{case} step {s}", want, want_e, hidden=shape.hidden)
            for l in range(shape.num_layers):
                k, v = st.kv_get(l)
                ew = chain_elementwise(l, shape.hidden)
                assert_bf16_close(k, orc_p.K[l], f"{case} step {s} K[{l}]", elementwise=ew,
                                  **k_bound(orc_p.K[l], qk_norm, rope))
                assert_bf16_close(v, orc_p.V[l], f"{case} step {s} V[{l}]", elementwise=ew)


def test_mmdit_options_change_the_output():
    """Each option reaches the output: the same inputs through the plain block and through each
    single option differ well beyond the parity tolerance (guards against an option that is
    accepted and silently ignored)."""
    torch = torch_cuda()
    shape = SHAPES["c4s"]
    inputs = synth.stage_inputs(shape)
    mm = synth.mmdit_inputs(shape, inputs)
    outs = {}
    for opt in [(False, False, False), (True, False, False), (False, True, False), (False, False, True)]:
        with _stage(shape, mm, *opt) as st:
            x = dev(torch, inputs.x)
            out = torch.empty_like(x)
            st.run_step(x, dev(torch, inputs.c), warmup=True, out=out)
            outs[opt] = host(out)
    base = outs[(False, False, False)]
    for opt, o in outs.items():
        if opt != (False, False, False):
            print(f"[mmdit] option {opt}: max_abs vs plain {max_abs(o, base):.3e}", flush=True)
            assert max_abs(o, base) > 0.1


def test_mmdit_guidance_pair_all_options():
    """A guidance pair with every option: each sample matches its own oracle stage."""
    torch = torch_cuda()
    shape = SHAPES["c4s"]
    inputs = synth.stage_inputs(shape)
    mm = synth.mmdit_inputs(shape, inputs)
    conds = list(synth.batch_conds(shape, inputs.c, 2))
    orc_p = [_oracle(shape, mm, "bf16p", True, True, True) for _ in range(2)]
    S, h, L = shape.seq_kv, shape.hidden, shape.num_layers
    with _stage(shape, mm, True, True, True, batch=2) as st:
        x = dev(torch, np.stack([inputs.x, inputs.x]))
        c = dev(torch, np.stack(conds))
        out = torch.empty_like(x)
        for s in range(2):
            warm = s == 0
            if s > 0:
                for b in range(2):
                    seed = shape.seed + 100 * s + 10 * b
                    noise = [(synth.randn((S, h), seed + 2 * l, std=shape.sigma_kv),
                              synth.randn((S, h), seed + 2 * l + 1, std=shape.sigma_kv)) for l in range(L)]
                    st.add_noise(noise, sample=b)
                    orc_p[b].add_noise(noise)
            print(f"[mmdit pair] step {s} warmup={warm}", flush=True)
            st.run_step(x, c, warmup=warm, out=out)
            got = host(out)
            for b in range(2):
                want_p = orc_p[b].step(inputs.x, conds[b], warmup=warm)
                check_stage_output(got[b], want_p, f"pair step {s} sample {b}", hidden=shape.hidden)
                for l in range(L):
                    k, _ = st.kv_get(l, sample=b)
                    assert_bf16_close(k, orc_p[b].K[l], f"pair step {s} sample {b} K[{l}]",
                                      elementwise=chain_elementwise(l, shape.hidden), **k_bound(orc_p[b].K[l], True, True))
            assert max_abs(got[0], got[1]) > 1e-3


def test_mmdit_patch_across_the_text_boundary():
    """A stage_run_patch whose rows straddle the end of the text prefix runs each part with its
    own stream's weights: it matches the oracle's micro-step over the same rows."""
    torch = torch_cuda()
    shape = SHAPES["c4s"]
    inputs = synth.stage_inputs(shape)
    mm = synth.mmdit_inputs(shape, inputs)
    orc = _oracle(shape, mm, "bf16p", True, True, True)
    with _stage(shape, mm, True, True, True) as st:
        x = dev(torch, inputs.x)
        out = torch.empty_like(x)
        st.run_step(x, dev(torch, inputs.c), warmup=True, out=out)
        orc.step(inputs.x, inputs.c, warmup=True)
        off, n = shape.seq_txt - 17, 50
        xp = dev(torch, inputs.x[off:off + n])
        st.run_patch(off, n, xp)
        got = host(xp)
        want = orc.run_rows(off, n, inputs.x[off:off + n])
        check_stage_output(got, want, "straddling micro-step", hidden=shape.hidden)
        for l in range(shape.num_layers):
            k, _ = st.kv_get(l)
            assert_bf16_close(k, orc.K[l], f"straddling micro-step K[{l}]", elementwise=chain_elementwise(l, shape.hidden),
                              **k_bound(orc.K[l], True, True))


# parallel (Flux.1 single-stream) block: (shape, qk_norm, rope, mlp_ratio)
PARALLEL = {
    "c4s-par": ("c4s", True, True, 4),
    "c3s-par-qknorm": ("c3s", True, False, 4),
    "c2s-par-rope": ("c2s", False, True, 4),
    "c2s-par-attn-only": ("c2s", True, True, 0),
}


def _parallel_chain(shape, par, qk_norm, rope, batch):
    torch = torch_cuda()
    inputs = synth.stage_inputs(shape)
    conds = synth.batch_conds(shape, inputs.c, batch)
    kw = dict(heads=shape.heads, head_dim=shape.head_dim, seq_txt=shape.seq_txt, seq_img=shape.seq_img,
              num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio, qk_norm=qk_norm,
              rope_angles=par.angles if rope else None, parallel=True)
    orc_p = [ref.StageOracle(par.layers, mode="bf16p", **kw) for _ in range(batch)]
    S, h, L = shape.seq_kv, shape.hidden, shape.num_layers
    with Stage(shape, batch=batch, qk_norm=qk_norm, rope=rope, parallel=True) as st:
        st.load(par.layers)
        if rope:
            st.set_rope(par.angles)
        x = dev(torch, np.stack([inputs.x] * batch) if batch > 1 else inputs.x)
        c = dev(torch, conds if batch > 1 else inputs.c)
        out = torch.empty_like(x)
        for s in range(3 if batch == 1 else 2):
            warm = s == 0
            if s > 0:
                for b in range(batch):
                    seed = shape.seed + 100 * s + 10 * b
                    noise = [(synth.randn((S, h), seed + 2 * l, std=shape.sigma_kv),
                              synth.randn((S, h), seed + 2 * l + 1, std=shape.sigma_kv)) for l in range(L)]
                    st.add_noise(noise, sample=b)
                    orc_p[b].add_noise(noise)
            print(f"[parallel] {shape.name} r={shape.mlp_ratio} batch {batch} step {s} warmup={warm}", flush=True)
            st.run_step(x, c, warmup=warm, out=out)
            got = host(out).reshape(batch, S, h)
            for b in range(batch):
                want_p = orc_p[b].step(inputs.x, conds[b], warmup=warm)
                check_stage_output(got[b], want_p, f"parallel step {s} sample {b}", hidden=shape.hidden)
                for l in range(L):
                    k, v = st.kv_get(l, sample=b)
                    ew = chain_elementwise(l, shape.hidden)
                    assert_bf16_close(k, orc_p[b].K[l], f"parallel step {s} sample {b} K[{l}]", elementwise=ew,
                                      **k_bound(orc_p[b].K[l], qk_norm, rope))
                    assert_bf16_close(v, orc_p[b].V[l], f"parallel step {s} sample {b} V[{l}]", elementwise=ew)
        if batch > 1:
            assert max_abs(got[0], got[1]) > 1e-3


@pytest.mark.parametrize("case", sorted(PARALLEL))
def test_parallel_block_stage_chain(case):
    """The parallel block (attention and MLP side by side, one fused output projection) against
    the oracle's, over a warm-up step and two drifted patched steps."""
    name, qk_norm, rope, r = PARALLEL[case]
    shape = dataclasses.replace(SHAPES[name], mlp_ratio=r)
    _parallel_chain(shape, synth.parallel_inputs(shape), qk_norm, rope, 1)


def test_parallel_block_guidance_pair():
    shape = SHAPES["c4s"]
    _parallel_chain(shape, synth.parallel_inputs(shape), True, True, 2)


@pytest.mark.parametrize("d,heads,rows,off,norm,rope", [
    (64, 3, 130, 5, True, True),      # ragged rows, both steps
    (72, 2, 77, 0, True, False),      # norm only
    (128, 4, 33, 60, False, True),    # rotation only, last buffer rows
    (64, 2, 0, 7, True, True),        # empty
])
def test_qk_norm_rope_component(d, heads, rows, off, norm, rope):
    """pf_qk_norm_rope on bf16 inputs against the oracle's per-head RMSNorm and rotation in
    fp64 (teacher-forced: one rounding, so within one bf16 ulp of the rounded exact value);
    V, the K rows outside the range and the K / V columns of the query rows stay bit-identical."""
    torch = torch_cuda()
    h, S = heads * d, 93 + max(rows, 0)
    rng = np.random.default_rng(d + rows)
    qkv = synth.to_bf16_values(rng.standard_normal((max(rows, 1), 3 * h)).astype(np.float32) * 2.0)
    if rows > 1:
        qkv[1, d:2 * d] = 0.0                                   # an all-zero head: RMS -> sqrt(eps)
    kb = synth.to_bf16_values(rng.standard_normal((S, h)).astype(np.float32) * 0.5)
    vb = synth.to_bf16_values(rng.standard_normal((S, h)).astype(np.float32))
    gq = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    gk = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    ang = rng.uniform(-50.0, 50.0, (S, d // 2)).astype(np.float32)
    q_t = dev(torch, qkv, torch.bfloat16)
    k_t = dev(torch, kb, torch.bfloat16)
    v_t = dev(torch, vb, torch.bfloat16)
    view = B.kv_view(k_t, v_t, S, h, B.PF_LAYOUT_ROWS)
    print(f"[qk_norm_rope] d={d} heads={heads} rows={rows} off={off} norm={norm} rope={rope}", flush=True)
    B.pf_qk_norm_rope(q_t, view, off, rows, heads, d, q_gamma=dev(torch, gq) if norm else None,
                      k_gamma=dev(torch, gk) if norm else None, angles=dev(torch, ang) if rope else None)
    got_q, got_k, got_v = host(q_t), host(k_t), host(v_t)
    np.testing.assert_array_equal(got_v, vb)
    keep = np.ones(S, bool)
    keep[off:off + rows] = False
    np.testing.assert_array_equal(got_k[keep], kb[keep])
    if rows == 0:
        np.testing.assert_array_equal(got_q, qkv)
        return
    np.testing.assert_array_equal(got_q[:, h:], qkv[:, h:])

    def expect(x, g):
        y = ref.rms_norm_heads(x, heads, d, g) if norm else np.asarray(x, np.float64)
        return ref.rope(y, heads, d, ang[off:off + rows]) if rope else y
    for what, got, want in (("Q", got_q[:, :h], expect(qkv[:, :h], gq)),
                            ("K", got_k[off:off + rows], expect(kb[off:off + rows], gk))):
        err = np.abs(got - ref.bf16_round(want))
        ulp = bf16_ulp(want)
        print(f"[qk_norm_rope] {what}: max err / ulp = {(err / ulp).max():.2f}", flush=True)
        assert (err <= ulp).all(), f"{what}: an element is off by more than one bf16 ulp"


def test_mmdit_call_order_errors():
    torch = torch_cuda()
    shape = dataclasses.replace(SHAPES["c4s"], num_layers=1)
    inputs = synth.stage_inputs(shape)
    mm = synth.mmdit_inputs(shape, inputs)
    x = dev(torch, inputs.x)
    c = dev(torch, inputs.c)
    with Stage(shape, dual_stream=True, rope=True) as st:
        st.load(mm.layers)                                  # text stream missing
        with pytest.raises(B.PFError) as e:
            st.run_step(x, c, warmup=True)
        assert e.value.status == B.PF_ERR_STATE and "text-stream" in str(e.value)
        st.load([], mm.txt_layers)
        with pytest.raises(B.PFError) as e:                 # angles missing
            st.run_step(x, c, warmup=True)
        assert e.value.status == B.PF_ERR_STATE and "stage_set_rope" in str(e.value)
        st.set_rope(mm.angles)
        st.run_step(x, c, warmup=True)
    with Stage(shape, qk_norm=True) as st:
        no_norm = [{k: a for k, a in lw.items() if k not in ("q_norm", "k_norm")} for lw in mm.layers]
        with pytest.raises(B.PFError) as e:
            st.load(no_norm)
        assert e.value.status == B.PF_ERR_INVALID_ARG
    with Stage(shape) as st:
        with pytest.raises(B.PFError) as e:
            st.load(mm.layers, mm.txt_layers)
        assert e.value.status == B.PF_ERR_INVALID_ARG
        with pytest.raises(B.PFError) as e:
            st.set_rope(mm.angles)
        assert e.value.status == B.PF_ERR_INVALID_ARG


@pytest.mark.parametrize("block", ["mmdit", "flux-single"])
def test_full_size_flux_blocks_sampled_parity(block):
    """The Flux.1 blocks at the full Flux-shaped stage size (16384 image rows + 512 text rows,
    h 3072, 24 x 128), one layer, in the launch configuration the bench times: warm-up and one
    drifted patched step, checked against the oracle on sampled rows of every micro-step and on
    the whole K/V buffer."""
    torch = torch_cuda()
    shape = dataclasses.replace(C4, num_layers=1, name=C4.name + "-L1")
    inputs = synth.stage_inputs(shape)
    if block == "mmdit":
        mm = synth.mmdit_inputs(shape, inputs)
        opts = dict(qk_norm=True, dual_stream=True, rope=True)
        okw = dict(txt_layers=mm.txt_layers, qk_norm=True, rope_angles=mm.angles)
    else:
        mm = synth.parallel_inputs(shape)
        opts = dict(qk_norm=True, rope=True, parallel=True)
        okw = dict(qk_norm=True, rope_angles=mm.angles, parallel=True)
    kw = dict(heads=shape.heads, head_dim=shape.head_dim, seq_txt=shape.seq_txt, seq_img=shape.seq_img,
              num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio, **okw)
    orc = ref.StageOracle(mm.layers, mode="bf16p", **kw)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(shape.seq_kv, 96, replace=False),
                                     [0, shape.seq_txt - 1, shape.seq_kv - 1] + list(shape.patch_offsets())]))
    with Stage(shape, **opts) as st:
        st.load(mm.layers, mm.txt_layers or None)
        st.set_rope(mm.angles)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        out = torch.empty_like(x)
        for s in range(2):
            if s == 1:
                noise = inputs.next_noise()
                st.add_noise(noise)
                orc.add_noise(noise)
            print(f"[mmdit] {block} full size sampled step {s}", flush=True)
            st.run_step(x, c, warmup=(s == 0), out=out)
            got = host(out)[rows]
            want = orc.step_sampled(inputs.x, inputs.c, rows, warmup=(s == 0))
            check_stage_output(got, want, f"{block} full size step {s} sampled rows", hidden=shape.hidden)
            k, v = st.kv_get(0)
            assert_bf16_close(k, orc.K[0], f"{block} full size step {s} K buffer", **k_bound(orc.K[0], True, True))
            assert_bf16_close(v, orc.V[0], f"{block} full size step {s} V buffer")


@pytest.mark.parametrize("block", ["mmdit", "flux-single"])
def test_flux_blocks_property_b_micro_steps_touch_only_their_rows(block):
    """Property (b) for the Flux.1 blocks: each micro-step of a patched step (the text prefix,
    then every patch) leaves every K and V buffer row outside its own range bit-identical (the
    QK step rewrites K in place), and its own rows hold the fresh values the oracle computes."""
    torch = torch_cuda()
    shape = SHAPES["c4s"]
    inputs = synth.stage_inputs(shape)
    if block == "mmdit":
        mm = synth.mmdit_inputs(shape, inputs)
        opts, okw, txt = dict(qk_norm=True, dual_stream=True, rope=True), dict(txt_layers=mm.txt_layers), mm.txt_layers
    else:
        mm = synth.parallel_inputs(shape)
        opts, okw, txt = dict(qk_norm=True, rope=True, parallel=True), dict(parallel=True), None
    kw = dict(heads=shape.heads, head_dim=shape.head_dim, seq_txt=shape.seq_txt, seq_img=shape.seq_img,
              num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio, qk_norm=True, rope_angles=mm.angles, **okw)
    orc = ref.StageOracle(mm.layers, mode="bf16p", **kw)
    with Stage(shape, **opts) as st:
        st.load(mm.layers, txt)
        st.set_rope(mm.angles)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        st.run_step(x, c, warmup=True, out=torch.empty_like(x))
        orc.step(inputs.x, inputs.c, warmup=True)
        noise = inputs.next_noise()
        st.add_noise(noise)
        orc.add_noise(noise)
        st.set_cond(c)
        orc.set_cond(inputs.c)
        xo = x.clone()
        for off, n in orc.micro_steps(False):
            print(f"[mmdit] {block} property b rows [{off}, {off + n})", flush=True)
            before = [st.kv_get(l) for l in range(shape.num_layers)]
            st.run_patch(off, n, x[off:off + n], xo[off:off + n])
            orc.run_rows(off, n, inputs.x[off:off + n])
            rs = slice(off, off + n)
            outside = np.ones(shape.seq_kv, bool)
            outside[rs] = False
            for l in range(shape.num_layers):
                k, v = st.kv_get(l)
                np.testing.assert_array_equal(k[outside], before[l][0][outside])
                np.testing.assert_array_equal(v[outside], before[l][1][outside])
                ew = chain_elementwise(l, shape.hidden)
                assert_bf16_close(k[rs], orc.K[l][rs], f"{block} fresh K rows [{off},{off + n}) layer {l}",
                                  elementwise=ew, **k_bound(orc.K[l][rs], True, True))
                assert_bf16_close(v[rs], orc.V[l][rs], f"{block} fresh V rows [{off},{off + n}) layer {l}",
                                  elementwise=ew)


@pytest.mark.parametrize("block", ["mmdit", "flux-single"])
def test_flux_blocks_property_a_fresh_equals_stale(block):
    """Property (a) for the Flux.1 blocks: with no drift between steps the stale context equals
    the fresh one, so a patched step reproduces the unpartitioned (warm-up) step.  Layer-0 V
    agrees within one bf16 ulp and K within three ulps of its pair norm (a patch-sized QKV
    projection may split its k range, so its fp32 sums round differently, and K is normalised
    and rotated after that rounding); outputs agree up to fp32 summation order, within the
    contract's tolerances."""
    torch = torch_cuda()
    shape = SHAPES["c4s"]
    inputs = synth.stage_inputs(shape)
    if block == "mmdit":
        mm = synth.mmdit_inputs(shape, inputs)
        opts, txt = dict(qk_norm=True, dual_stream=True, rope=True), mm.txt_layers
    else:
        mm = synth.parallel_inputs(shape)
        opts, txt = dict(qk_norm=True, rope=True, parallel=True), None
    with Stage(shape, **opts) as st:
        st.load(mm.layers, txt)
        st.set_rope(mm.angles)
        x, c = dev(torch, inputs.x), dev(torch, inputs.c)
        warm = torch.empty_like(x)
        st.run_step(x, c, warmup=True, out=warm)
        k0, v0 = (t.clone() for t in st.kv_raw(0))
        patched = torch.empty_like(x)
        st.run_step(x, c, warmup=False, out=patched)
        k1, v1 = st.kv_raw(0)
        ka, kb = host(k0), host(k1)
        va, vb = host(v0), host(v1)
        k_tol = 3.0 * bf16_ulp(pair_norms(np.maximum(np.abs(ka), np.abs(kb)))) + 2.0 ** -19
        v_tol = bf16_ulp(np.maximum(np.abs(va), np.abs(vb))) + 2.0 ** -19
        print(f"[mmdit] {block} property a: K max diff / bound {(np.abs(ka - kb) / k_tol).max():.2f}, "
              f"V {(np.abs(va - vb) / v_tol).max():.2f}", flush=True)
        assert (np.abs(ka - kb) <= k_tol).all(), "layer-0 K beyond three ulps of the pair norm"
        assert (np.abs(va - vb) <= v_tol).all(), "layer-0 V beyond one ulp"
        assert_close(host(patched), host(warm), f"{block} patched step vs warm-up step (fresh == stale)",
                     max_abs_tol=chain_max_abs_tol(shape.hidden))
