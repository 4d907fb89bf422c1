"""The denoising loop around a stage on the GPU (denoiser_step / denoiser_run) against the
fp64 loop oracle (oracle/sampler.py over oracle.ref.StageOracle in bf16-in mode), one
sample and a guided pair; plus argument checks that need no GPU."""
import ctypes
import dataclasses
import math

import numpy as np
import pytest

from oracle import ref, sampler
from patch_pipelined_attention_amd import binding as B
from patch_pipelined_attention_amd import synth
from patch_pipelined_attention_amd.configs import C2, C4
from patch_pipelined_attention_amd.stage import Stage

from _util import MAX_ABS, REL_L2, assert_close, chain_max_abs_tol, dev, host, torch_cuda

C_IN, PATCH, FREQ, T_TRAIN = 4, 2, 256, 1000
TIMESTEPS = [999, 799, 599, 399, 199]


def _cfg(grid):
    return B.DenoiserConfig(in_channels=C_IN, patch=PATCH, grid_h=grid, grid_w=grid, freq_dim=FREQ,
                            train_steps=T_TRAIN, beta_start=1e-4, beta_end=0.02)


def _block(shape, inputs, block):
    """(layers, text layers, angles, Stage options, oracle options) of a block variant."""
    if block == "mmdit":
        mm = synth.mmdit_inputs(shape, inputs)
        return (mm.layers, mm.txt_layers, mm.angles, dict(qk_norm=True, dual_stream=True, rope=True),
                dict(txt_layers=mm.txt_layers, qk_norm=True, rope_angles=mm.angles))
    if block == "flux-single":
        par = synth.parallel_inputs(shape)
        return (par.layers, None, par.angles, dict(qk_norm=True, rope=True, parallel=True),
                dict(qk_norm=True, rope_angles=par.angles, parallel=True))
    return inputs.layers, None, None, {}, {}


def _loop_oracle(shape, inputs, din, batch, layers=None, opts=None, mode="bf16"):
    stages = [ref.StageOracle(inputs.layers if layers is None else layers, heads=shape.heads,
                              head_dim=shape.head_dim, seq_txt=shape.seq_txt, seq_img=shape.seq_img,
                              num_patches=shape.num_patches, mlp_ratio=shape.mlp_ratio, mode=mode, **(opts or {}))
              for _ in range(batch)]
    return sampler.DenoiserOracle(stages, din.weights, C_IN, PATCH, din.grid_h, din.grid_w, FREQ,
                                  sampler.alphas_cumprod(T_TRAIN, 1e-4, 0.02), seq_txt=shape.seq_txt)


@pytest.mark.gpu
@pytest.mark.parametrize("name,batch,guidance,block", [("c2s", 1, 1.0, "dit"), ("c2s", 2, 4.0, "dit"),
                                                      ("c4s", 1, 1.0, "dit"), ("c4s", 2, 3.5, "mmdit"),
                                                      ("c4s", 1, 1.0, "flux-single")])
def test_denoiser_steps_match_loop_oracle(name, batch, guidance, block):
    """Each step starts both sides from the GPU's latent (teacher forcing; each side keeps its own
    stale K/V buffers) and compares the noise prediction the step applied, recovered from the
    DDIM update as eps = (z' - a z) / e, against the oracle's.  The first two steps are
    warm-up steps, the rest reuse stale buffers.  The Flux-shaped cases also run the Flux.1
    blocks (a guided pair over the double-stream block, one sample over the single-stream one).

    Gates: the contract's max-abs 2e-2 and rel-L2 5e-3 against the loop oracle over bf16p stages
    (bf16 probabilities, the precision the kernels compute in; at the Flux-shaped width max-abs is
    reported, see _util.chain_max_abs_tol); the loop over bf16-in stages without rounded
    probabilities is reported."""
    torch = torch_cuda()
    shape = {"c2s": C2.small(seq_img=256, num_layers=2, num_patches=4),
             "c4s": C4.small(seq_img=256, num_layers=1, num_patches=4, seq_txt=32)}[name]
    inputs = synth.stage_inputs(shape)
    din = synth.denoiser_inputs(shape, batch=batch)
    x_txt = synth.randn((batch, shape.seq_txt, shape.hidden), shape.seed + 6000) if shape.seq_txt else None
    layers, txt_layers, angles, st_opts, orc_opts = _block(shape, inputs, block)
    orc = _loop_oracle(shape, inputs, din, batch, layers, orc_opts)
    orc_p = _loop_oracle(shape, inputs, din, batch, layers, orc_opts, mode="bf16p")
    abar = sampler.alphas_cumprod(T_TRAIN, 1e-4, 0.02)
    with Stage(shape, batch=batch, **st_opts) as st:
        st.load(layers, txt_layers)
        if angles is not None:
            st.set_rope(angles)
        d = B.denoiser_create(st.handle, _cfg(din.grid_h))
        try:
            B.denoiser_load_weights(d, {k: dev(torch, v) for k, v in din.weights.items()})
            z = dev(torch, din.z)
            y = dev(torch, din.y)
            xt = dev(torch, x_txt) if x_txt is not None else None
            for i, t in enumerate(TIMESTEPS):
                tn = TIMESTEPS[i + 1] if i + 1 < len(TIMESTEPS) else -1
                warm = i < 2
                z_before = host(z)
                print(f"[denoiser] {name} {block} batch={batch} step {i} t={t} warmup={warm}", flush=True)
                B.denoiser_step(d, z, y, t, tn, warmup=warm, guidance=guidance, x_txt=xt)
                z_after = host(z)
                _, eps_b = orc.step(z_before, din.y, t, tn, warm, guidance, x_txt=x_txt)
                _, eps_p = orc_p.step(z_before, din.y, t, tn, warm, guidance, x_txt=x_txt)
                ab_n = abar[tn] if tn >= 0 else 1.0
                a = math.sqrt(ab_n / abar[t])
                e = math.sqrt(1.0 - ab_n) - a * math.sqrt(1.0 - abar[t])
                eps_got = (z_after - a * z_before) / e
                assert_close(eps_got, eps_p, f"{name} {block} batch {batch} step {i}: eps vs loop oracle (bf16p)",
                             max_abs_tol=chain_max_abs_tol(shape.hidden))
                assert_close(eps_got, eps_b, f"{name} {block} batch {batch} step {i}: eps vs loop oracle (bf16-in, "
                             "reported)", max_abs_tol=None, rel_tol=None)
                if batch == 2:
                    assert np.array_equal(z_after[0], z_after[1]), "a guided pair must keep one shared latent"
        finally:
            torch.cuda.synchronize()
            B.denoiser_destroy(d)


@pytest.mark.gpu
def test_denoiser_run_equals_steps():
    """denoiser_run over a schedule gives the same latent, bit for bit, as the same steps one by one."""
    torch = torch_cuda()
    shape = C2.small(seq_img=256, num_layers=1, num_patches=4)
    inputs = synth.stage_inputs(shape)
    din = synth.denoiser_inputs(shape)
    outs = []
    for mode in ("run", "steps"):
        with Stage(shape) as st:
            st.load(inputs.layers)
            d = B.denoiser_create(st.handle, _cfg(din.grid_h))
            B.denoiser_load_weights(d, {k: dev(torch, v) for k, v in din.weights.items()})
            z, y = dev(torch, din.z), dev(torch, din.y)
            if mode == "run":
                B.denoiser_run(d, z, y, TIMESTEPS, warmup_steps=2)
            else:
                for i, t in enumerate(TIMESTEPS):
                    B.denoiser_step(d, z, y, t, TIMESTEPS[i + 1] if i + 1 < len(TIMESTEPS) else -1, warmup=i < 2)
            outs.append(host(z))
            torch.cuda.synchronize()
            B.denoiser_destroy(d)
    assert np.array_equal(outs[0], outs[1])


def test_denoiser_argument_checks():
    lib = B.lib()
    h = ctypes.c_void_p(7)
    assert lib.denoiser_create(None, None, ctypes.byref(h)) == B.PF_ERR_INVALID_ARG and h.value is None
    assert lib.denoiser_destroy(None) == B.PF_OK
    assert lib.denoiser_step(None, None, None, None, 10, 5, 0, 1.0, None) == B.PF_ERR_INVALID_ARG
    ts = (ctypes.c_int32 * 2)(10, 5)
    assert lib.denoiser_run(None, None, None, None, ts, 2, 0, 1.0, None) == B.PF_ERR_INVALID_ARG   # warmup_steps 0
