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
