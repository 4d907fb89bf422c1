"""CPU pins for the fp64 denoising-loop oracle (oracle/sampler.py): closed forms,
a library special case (torch's conv2d), brute force and limits.  No GPU."""
import math

import numpy as np
import pytest

from oracle import ref, sampler


def test_timestep_features_closed_forms():
    f0 = sampler.timestep_features(0.0, 256)
    assert np.array_equal(f0[:128], np.ones(128)) and np.array_equal(f0[128:], np.zeros(128))
    t = 37.0
    f = sampler.timestep_features(t, 256)
    assert f[0] == pytest.approx(math.cos(t)) and f[128] == pytest.approx(math.sin(t))   # frequency 1
    k = 64                                                                                # frequency 10000^-0.5
    assert f[k] == pytest.approx(math.cos(t * 0.01)) and f[128 + k] == pytest.approx(math.sin(t * 0.01))
    assert np.allclose(f[:128] ** 2 + f[128:] ** 2, 1.0)


def test_pos_embed_closed_forms():
    pe = sampler.pos_embed_2d(3, 5, 16)
    q = 4
    assert np.array_equal(pe[0], np.concatenate([np.zeros(q), np.ones(q), np.zeros(q), np.ones(q)]))
    s = 2 * 5 + 3                                   # row 2, column 3
    assert pe[s, 0] == pytest.approx(math.sin(2.0)) and pe[s, q] == pytest.approx(math.cos(2.0))
    assert pe[s, 2 * q] == pytest.approx(math.sin(3.0)) and pe[s, 3 * q] == pytest.approx(math.cos(3.0))
    assert pe[s, 1] == pytest.approx(math.sin(2.0 * 10000 ** -0.25))


def test_patchify_matches_conv2d():
    """Patch embedding as a linear map on patchify() equals torch's stride-p convolution."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    C, p, H, W, h = 4, 2, 6, 10, 8
    z = rng.standard_normal((C, H, W))
    wconv = rng.standard_normal((h, C, p, p))
    b = rng.standard_normal(h)
    want = torch.nn.functional.conv2d(torch.from_numpy(z)[None], torch.from_numpy(wconv), torch.from_numpy(b),
                                      stride=p)[0].numpy()            # [h, H/p, W/p]
    got = ref.linear(sampler.patchify(z, p), wconv.reshape(h, -1), b)     # [(H/p)(W/p), h]
    assert np.allclose(got, want.reshape(h, -1).T, atol=1e-12)


def test_unpatchify_round_trip_brute_force():
    C, p, gh, gw = 3, 2, 4, 5
    z = np.arange(C * gh * p * gw * p, dtype=np.float64).reshape(C, gh * p, gw * p)
    v = sampler.patchify(z, p)
    for s in range(gh * gw):
        gy, gx = divmod(s, gw)
        for c in range(C):
            for dy in range(p):
                for dx in range(p):
                    assert v[s, (c * p + dy) * p + dx] == z[c, gy * p + dy, gx * p + dx]
    assert np.array_equal(sampler.unpatchify(v, C, p, gh, gw), z)


def test_schedule_first_value_and_monotone():
    ab = sampler.alphas_cumprod(1000, 1e-4, 0.02)
    assert ab[0] == pytest.approx(1.0 - 1e-4)
    assert ab[1] == pytest.approx((1.0 - 1e-4) * (1.0 - (1e-4 + (0.02 - 1e-4) / 999)))
    assert np.all(np.diff(ab) < 0) and 0.0 < ab[-1] < 1e-4


def test_ddim_step_with_exact_noise_recovers_the_trajectory():
    """z_t = sqrt(abar_t) x0 + sqrt(1 - abar_t) e and eps = e give z_s = sqrt(abar_s) x0 + sqrt(1 - abar_s) e."""
    rng = np.random.default_rng(9)
    x0, e = rng.standard_normal((4, 8, 8)), rng.standard_normal((4, 8, 8))
    ab = sampler.alphas_cumprod(1000, 1e-4, 0.02)
    t, s = 801, 601
    zt = math.sqrt(ab[t]) * x0 + math.sqrt(1 - ab[t]) * e
    zs = sampler.ddim_step(zt, e, ab[t], ab[s])
    assert np.allclose(zs, math.sqrt(ab[s]) * x0 + math.sqrt(1 - ab[s]) * e, atol=1e-12)
    assert np.allclose(sampler.ddim_step(zt, e, ab[t], 1.0), x0, atol=1e-12)   # last step returns x0


def test_guidance_limits():
    rng = np.random.default_rng(2)
    ec, eu = rng.standard_normal(10), rng.standard_normal(10)
    assert np.array_equal(sampler.guide(ec, eu, 0.0), eu)
    assert np.allclose(sampler.guide(ec, eu, 1.0), ec)
    assert np.allclose(sampler.guide(ec, eu, 3.0), eu + 3.0 * (ec - eu))


# ---------------------------------------------------------------- the loop as a whole

from oracle import brute_sampler  # noqa: E402

_H, _D, _L, _R, _C, _P, _GH, _GW, _F = 2, 4, 2, 2, 2, 2, 2, 3, 6
_HID = _H * _D


def _loop_weights(seed, zero_fada=False):
    rng = np.random.default_rng(seed)
    h, cpp = _HID, _C * _P * _P
    w = {"w_patch": rng.standard_normal((h, cpp)) * 0.5, "b_patch": rng.standard_normal(h) * 0.1,
         "w_t1": rng.standard_normal((h, _F)) * 0.5, "b_t1": rng.standard_normal(h) * 0.1,
         "w_t2": rng.standard_normal((h, h)) * 0.3, "b_t2": rng.standard_normal(h) * 0.1,
         "w_fada": rng.standard_normal((2 * h, h)) * 0.4, "b_fada": rng.standard_normal(2 * h) * 0.2,
         "w_out": rng.standard_normal((cpp, h)) * 0.5, "b_out": rng.standard_normal(cpp) * 0.1}
    if zero_fada:
        w["w_fada"][:] = 0.0
        w["b_fada"][:] = 0.0
    layers = []
    for _ in range(_L):
        layers.append({"w_qkv": rng.standard_normal((3 * h, h)) * 0.4, "b_qkv": rng.standard_normal(3 * h) * 0.1,
                       "w_o": rng.standard_normal((h, h)) * 0.4, "b_o": rng.standard_normal(h) * 0.1,
                       "w1": rng.standard_normal((_R * h, h)) * 0.4, "b1": rng.standard_normal(_R * h) * 0.1,
                       "w2": rng.standard_normal((h, _R * h)) * 0.4, "b2": rng.standard_normal(h) * 0.1,
                       "w_ada": rng.standard_normal((6 * h, h)) * 0.3, "b_ada": rng.standard_normal(6 * h) * 0.1})
    return w, layers


def _loop_oracle(w, layers, nb, seq_txt, cls=None):
    S_img = _GH * _GW
    stages = [ref.StageOracle(layers, heads=_H, head_dim=_D, seq_txt=seq_txt, seq_img=S_img, num_patches=2,
                              mlp_ratio=_R, mode="exact") for _ in range(nb)]
    return (cls or sampler.DenoiserOracle)(stages, w, _C, _P, _GH, _GW, _F, sampler.alphas_cumprod(1000, 1e-4, 0.02),
                                           seq_txt=seq_txt)


def _loop_inputs(nb, seq_txt, seed):
    rng = np.random.default_rng(seed)
    z1 = rng.standard_normal((_C, _GH * _P, _GW * _P))
    z = np.stack([z1] * nb)                      # a pair shares its latent
    y = rng.standard_normal((nb, _HID))
    x_txt = rng.standard_normal((nb, seq_txt, _HID)) if seq_txt else None
    return z, y, x_txt


def _run_brute(w, layers, nb, seq_txt, z, y, x_txt, schedule, guidance):
    S = seq_txt + _GH * _GW
    lw = [{k: a.tolist() for k, a in W.items()} for W in layers]
    wl = {k: a.tolist() for k, a in w.items()}
    kb = [[[[0.0] * _HID for _ in range(S)] for _ in range(_L)] for _ in range(nb)]
    vb = [[[[0.0] * _HID for _ in range(S)] for _ in range(_L)] for _ in range(nb)]
    abar = brute_sampler.abar_table(1000, 1e-4, 0.02)
    zl = z.tolist()
    outs = []
    for i, (t, t_next) in enumerate(schedule):
        zl, eps = brute_sampler.denoise_step(wl, lw, kb, vb, zl, y.tolist(), t, t_next, abar, heads=_H, d=_D,
                                             seq_txt=seq_txt, num_patches=2, mlp_ratio=_R, patch=_P, freq_dim=_F,
                                             warmup=i == 0, guidance=guidance,
                                             x_txt=None if x_txt is None else x_txt.tolist())
        outs.append((np.array(zl), np.array(eps)))
    return outs


_SCHEDULE = [(999, 667), (667, 333), (333, -1)]


@pytest.mark.parametrize("nb,seq_txt,guidance", [(1, 0, 1.0), (2, 2, 3.5)], ids=["single", "pair-text"])
def test_denoiser_oracle_vs_loop_restatement(nb, seq_txt, guidance):
    """DenoiserOracle.condition / eps / step against the independent loop restatement over
    three steps (a warm-up, a patched step, the last step to x0), one sample and a guided pair
    with a text prefix."""
    w, layers = _loop_weights(21)
    z, y, x_txt = _loop_inputs(nb, seq_txt, 22)
    want = _run_brute(w, layers, nb, seq_txt, z, y, x_txt, _SCHEDULE, guidance)
    orc = _loop_oracle(w, layers, nb, seq_txt)
    zc = z.copy()
    for i, (t, t_next) in enumerate(_SCHEDULE):
        zc, eps = orc.step(zc, y, t, t_next, warmup=i == 0, guidance=guidance, x_txt=x_txt)
        np.testing.assert_allclose(eps, want[i][1], rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(zc, want[i][0], rtol=1e-10, atol=1e-10)


def _stage_out(w, layers, seq_txt, z1, c1, x_txt1):
    """The stage's image-row outputs for one sample's first (warm-up) step, from the pinned
    pieces: patchify, the linear map and the position table, then the stage oracle."""
    x_img = ref.linear(sampler.patchify(z1, _P), w["w_patch"], w["b_patch"]) + sampler.pos_embed_2d(_GH, _GW, _HID)
    x_all = x_img if not seq_txt else np.concatenate([x_txt1, x_img])
    st = ref.StageOracle(layers, heads=_H, head_dim=_D, seq_txt=seq_txt, seq_img=_GH * _GW, num_patches=2,
                         mlp_ratio=_R, mode="exact")
    return st.step(x_all, c1, warmup=True)[seq_txt:]


def test_final_layer_special_cases():
    """With W_fada = 0 the final modulation is the bias alone: b_fada = 0 makes the final layer
    LN(out) W_out^T + b_out; b_fada = [shift; scale] with distinct constants gives
    (LN(out) (1 + scale) + shift) W_out^T + b_out, which a swap of the two halves would break."""
    w, layers = _loop_weights(31, zero_fada=True)
    z, y, _ = _loop_inputs(1, 0, 32)
    orc = _loop_oracle(w, layers, 1, 0)
    c = orc.condition(999, y)[0]
    out = _stage_out(w, layers, 0, z[0], c, None)
    ln = ref.layer_norm(out)
    want = sampler.unpatchify(ln @ w["w_out"].T + w["b_out"], _C, _P, _GH, _GW)
    got = _loop_oracle(w, layers, 1, 0).eps(z[0], y[0], c, ref.StageOracle(
        layers, heads=_H, head_dim=_D, seq_txt=0, seq_img=_GH * _GW, num_patches=2, mlp_ratio=_R), warmup=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    shift, scale = 0.75, -0.4
    w2 = dict(w, b_fada=np.concatenate([np.full(_HID, shift), np.full(_HID, scale)]))
    want2 = sampler.unpatchify((ln * (1.0 + scale) + shift) @ w["w_out"].T + w["b_out"], _C, _P, _GH, _GW)
    got2 = _loop_oracle(w2, layers, 1, 0).eps(z[0], y[0], c, ref.StageOracle(
        layers, heads=_H, head_dim=_D, seq_txt=0, seq_img=_GH * _GW, num_patches=2, mlp_ratio=_R), warmup=True)
    np.testing.assert_allclose(got2, want2, rtol=1e-12, atol=1e-12)
    assert np.abs(want2 - want).max() > 1e-2


@pytest.mark.parametrize("g,which", [(1.0, 0), (0.0, 1)])
def test_guidance_roles(g, which):
    """Guidance 1 gives both samples of a pair the conditional sample's (0) noise prediction,
    guidance 0 the unconditional one's (1): each equals the prediction of a single-sample loop
    run with that sample's condition embedding."""
    w, layers = _loop_weights(41)
    z, y, _ = _loop_inputs(2, 0, 42)
    pair = _loop_oracle(w, layers, 2, 0)
    zp, eps = pair.step(z, y, 999, 667, warmup=True, guidance=g)
    single = _loop_oracle(w, layers, 1, 0)
    zs, eps_s = single.step(z[:1], y[which:which + 1], 999, 667, warmup=True)
    np.testing.assert_allclose(eps[0], eps_s[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(eps[1], eps_s[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(zp[0], zs[0], rtol=1e-12, atol=1e-12)
    other = _loop_oracle(w, layers, 1, 0).step(z[:1], y[1 - which:2 - which], 999, 667, warmup=True)[1]
    assert np.abs(other[0] - eps_s[0]).max() > 1e-3      # the two conditions really differ


def test_loop_pins_catch_planted_mistakes():
    """A final layer with shift and scale swapped, and a guidance with the roles of the two
    samples swapped, each disagree with the loop restatement."""
    w, layers = _loop_weights(51)

    class SwappedShiftScale(sampler.DenoiserOracle):
        def eps(self, z_b, y_b, c_b, stage, warmup, x_txt=None):
            wf = self.w
            self.w = dict(wf, w_fada=np.concatenate([wf["w_fada"][_HID:], wf["w_fada"][:_HID]]),
                          b_fada=np.concatenate([wf["b_fada"][_HID:], wf["b_fada"][:_HID]]))
            try:
                return super().eps(z_b, y_b, c_b, stage, warmup, x_txt)
            finally:
                self.w = wf

    class SwappedRoles(sampler.DenoiserOracle):
        def step(self, z, y, t, t_next, warmup, guidance=1.0, x_txt=None):
            return super().step(z, y[::-1].copy(), t, t_next, warmup, guidance, x_txt)

    for nb, cls in ((1, SwappedShiftScale), (2, SwappedRoles)):
        z, y, _ = _loop_inputs(nb, 0, 52)
        want = _run_brute(w, layers, nb, 0, z, y, None, _SCHEDULE[:1], 3.5)
        good = _loop_oracle(w, layers, nb, 0).step(z, y, *_SCHEDULE[0], warmup=True, guidance=3.5)[1]
        np.testing.assert_allclose(good, want[0][1], rtol=1e-10, atol=1e-10)
        bad = _loop_oracle(w, layers, nb, 0, cls=cls).step(z, y, *_SCHEDULE[0], warmup=True, guidance=3.5)[1]
        assert np.abs(bad - want[0][1]).max() > 1e-3, cls.__name__
