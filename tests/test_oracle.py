"""CPU pins for the fp64 oracle: closed forms, invariants, library special cases,
brute force on tiny inputs, and the stage properties the PipeFusion summaries fix
(dual partitioning, stale step-(T+1) context, per-layer full-spatial KV buffer,
full attention).  Nothing here touches the GPU."""
import math
import os

import numpy as np
import pytest

from oracle import brute, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_golden():
    for row in _golden_rows("bf16_round.txt"):
        x, want = float(row[0]), float(row[1])
        got = ref.bf16_round(np.array([x]))[0]
        assert got == want or (math.isinf(want) and math.isinf(got) and np.sign(got) == np.sign(want)), (x, got, want)


def test_bf16_round_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = ref.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_idempotent_and_monotone():
    x = np.sort(np.random.default_rng(1).standard_normal(5000))
    r = ref.bf16_round(x)
    np.testing.assert_array_equal(ref.bf16_round(r), r)
    assert np.all(np.diff(r) >= 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8 + 1e-300)


# ---------------------------------------------------------------- elementwise pieces

def test_gelu_golden_phi_table():
    for row in _golden_rows("gelu_phi.txt"):
        x, want = float(row[0]), float(row[1])
        assert abs(ref.gelu_erf(np.array([x]))[0] - want) < 1e-15


def test_gelu_odd_part_identity_and_zero():
    # x*Phi(x) - (-x)*Phi(-x) = x because Phi(x) + Phi(-x) = 1; same for the tanh form (tanh is odd).
    x = np.linspace(-6, 6, 1001)
    for g in (ref.gelu_erf, ref.gelu_tanh):
        np.testing.assert_allclose(g(x) - g(-x), x, rtol=0, atol=1e-12)
        assert g(np.array([0.0]))[0] == 0.0
    # published bound of the tanh approximation to x*Phi(x): below 5e-4 everywhere
    assert np.abs(ref.gelu_tanh(x) - ref.gelu_erf(x)).max() < 5e-4


def test_silu_identity():
    x = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(ref.silu(x) - ref.silu(-x), x, atol=1e-12)
    assert ref.silu(np.array([0.0]))[0] == 0.0
    # large x: silu(x) -> x; large -x: -> 0
    assert abs(ref.silu(np.array([40.0]))[0] - 40.0) < 1e-12


def test_layer_norm_moments():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 33)) * 3 + 5
    eps = 1e-6
    y = ref.layer_norm(x, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)
    # a large eps shrinks the variance as var/(var+eps): catches eps outside the sqrt
    y2 = ref.layer_norm(x, 4.0)
    np.testing.assert_allclose(y2.var(axis=1), var / (var + 4.0), rtol=1e-12)
    # brute-force row
    np.testing.assert_allclose(y[3], brute.layer_norm_row(list(x[3]), eps), rtol=1e-12)


def test_modulate_closed_forms():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((4, 6))
    shift = rng.standard_normal(6)
    np.testing.assert_array_equal(ref.modulate(y, shift, -np.ones(6)), np.broadcast_to(shift, y.shape))
    np.testing.assert_array_equal(ref.modulate(y, np.zeros(6), np.zeros(6)), y)
    np.testing.assert_allclose(ref.modulate(y, 0 * shift, np.ones(6)), 2 * y)


def test_linear_and_adaln_against_loops():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))   # [out, in]
    b = rng.standard_normal(4)
    np.testing.assert_allclose(ref.linear(x, w, b), brute.matvec_rows(x.tolist(), w.tolist(), b.tolist()), rtol=1e-13)
    h = 3
    c = rng.standard_normal(h)
    wa = rng.standard_normal((6 * h, h))
    ba = rng.standard_normal(6 * h)
    mod = ref.adaln(c, wa, ba)
    assert mod.shape == (6, h)
    want = brute.matvec_rows([[brute.silu(a) for a in c]], wa.tolist(), ba.tolist())[0]
    np.testing.assert_allclose(mod.reshape(-1), want, rtol=1e-13)
    # c = 0 -> SiLU(0) = 0 -> the modulation is exactly the bias
    np.testing.assert_array_equal(ref.adaln(np.zeros(h), wa, ba).reshape(-1), ba)


# ---------------------------------------------------------------- attention

def test_attention_golden_two_keys():
    rows = {r[0]: [float(v) for v in r[1:]] for r in _golden_rows("attention_two_keys.txt")}
    q = np.array([rows["q"]])
    k = np.array([rows["k0"], rows["k1"]])
    v = np.array([rows["v0"], rows["v1"]])
    o = ref.attention(q, k, v, 1, 4)
    np.testing.assert_allclose(o[0], rows["o"], rtol=0, atol=1e-15)


def test_attention_vs_brute_force():
    rng = np.random.default_rng(6)
    H, d, S, n = 2, 3, 11, 5
    q = rng.standard_normal((n, H * d)) * 2
    k = rng.standard_normal((S, H * d)) * 2
    v = rng.standard_normal((S, H * d))
    got = ref.attention(q, k, v, H, d, chunk=2)
    want = brute.attention(q.tolist(), k.tolist(), v.tolist(), H, d)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(7)
    H, d, S = 3, 8, 37
    k = rng.standard_normal((S, H * d))
    v = rng.standard_normal((S, H * d))
    # Q = 0 -> uniform weights -> column mean of V
    o = ref.attention(np.zeros((4, H * d)), k, v, H, d)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13, atol=1e-14)
    # one dominant key (logit +50 over the rest) -> that row of V, per head
    q = np.zeros((1, H * d))
    k2 = np.zeros((S, H * d))
    for j in range(H):
        k2[5 + j, j * d] = 50.0 * math.sqrt(d)
        q[0, j * d] = 1.0
    o = ref.attention(q, k2, v, H, d)
    for j in range(H):
        np.testing.assert_allclose(o[0, j * d:(j + 1) * d], v[5 + j, j * d:(j + 1) * d], rtol=1e-15, atol=1e-19)
    # permuting buffer rows together leaves O unchanged
    q = rng.standard_normal((6, H * d))
    perm = rng.permutation(S)
    np.testing.assert_allclose(ref.attention(q, k[perm], v[perm], H, d), ref.attention(q, k, v, H, d), rtol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((9, 300)) * 20
    p = ref.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    # invariant to a per-row shift
    np.testing.assert_allclose(ref.softmax_rows(s + 123.0), p, rtol=1e-12)


# ---------------------------------------------------------------- splice

def test_splice_byte_exact_and_bounds():
    rng = np.random.default_rng(9)
    dst = rng.integers(0, 1 << 16, (20, 7), dtype=np.uint16)
    before = dst.copy()
    src = rng.integers(0, 1 << 16, (5, 7), dtype=np.uint16)
    ref.splice(dst, src, 9)
    np.testing.assert_array_equal(dst[9:14], src)
    np.testing.assert_array_equal(dst[:9], before[:9])
    np.testing.assert_array_equal(dst[14:], before[14:])
    with pytest.raises(ValueError):
        ref.splice(dst, src, 16)
    ref.splice(dst, src[:0], 20)            # empty splice at the end is a no-op
    np.testing.assert_array_equal(dst[14:], before[14:])


# ---------------------------------------------------------------- the stage

def _tiny_layers(L, h, r, seed, std=0.3):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(L):
        out.append({"w_qkv": rng.standard_normal((3 * h, h)) * std, "b_qkv": rng.standard_normal(3 * h) * std,
                    "w_o": rng.standard_normal((h, h)) * std, "b_o": rng.standard_normal(h) * std,
                    "w1": rng.standard_normal((r * h, h)) * std, "b1": rng.standard_normal(r * h) * std,
                    "w2": rng.standard_normal((h, r * h)) * std, "b2": rng.standard_normal(h) * std,
                    "w_ada": rng.standard_normal((6 * h, h)) * std, "b_ada": rng.standard_normal(6 * h) * std})
    return out


def _tiny_stage(mode="exact", M=2, S_txt=2, S_img=8, L=2, r=2, H=2, d=4, seed=10):
    layers = _tiny_layers(L, H * d, r, seed)
    st = ref.StageOracle(layers, heads=H, head_dim=d, seq_txt=S_txt, seq_img=S_img, num_patches=M,
                         mlp_ratio=r, mode=mode)
    return st, layers


def test_stage_vs_brute_force_two_steps():
    st, layers = _tiny_stage()
    H, d, h, S = 2, 4, 8, 10
    rng = np.random.default_rng(11)
    x = rng.standard_normal((S, h))
    c = rng.standard_normal(h)
    noise = [(rng.standard_normal((S, h)) * 0.1, rng.standard_normal((S, h)) * 0.1) for _ in layers]
    kb = [[[0.0] * h for _ in range(S)] for _ in layers]
    vb = [[[0.0] * h for _ in range(S)] for _ in layers]
    lw = [{k: a.tolist() for k, a in W.items()} for W in layers]
    kw = dict(heads=H, d=d, seq_txt=2, num_patches=2, mlp_ratio=2)
    out0 = st.step(x, c, warmup=True)
    want0 = brute.stage_step(lw, kb, vb, x.tolist(), c.tolist(), warmup=True, **kw)
    np.testing.assert_allclose(out0, want0, rtol=1e-11, atol=1e-11)
    st.add_noise(noise)
    for l, (nk, nv) in enumerate(noise):
        kb[l] = (np.array(kb[l]) + nk).tolist()
        vb[l] = (np.array(vb[l]) + nv).tolist()
    out1 = st.step(x, c, warmup=False)
    want1 = brute.stage_step(lw, kb, vb, x.tolist(), c.tolist(), warmup=False, **kw)
    np.testing.assert_allclose(out1, want1, rtol=1e-11, atol=1e-11)
    for l in range(2):
        np.testing.assert_allclose(st.K[l], kb[l], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st.V[l], vb[l], rtol=1e-12, atol=1e-12)


def test_property_a_fresh_equals_stale_gives_full_attention():
    """(a) with no drift, every patched step reproduces the warm-up (unpartitioned) output."""
    st, _ = _tiny_stage(M=4, S_txt=0, S_img=16, L=2)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 8))
    c = rng.standard_normal(8)
    full = st.step(x, c, warmup=True)
    for _ in range(2):
        np.testing.assert_allclose(st.step(x, c, warmup=False), full, rtol=1e-12, atol=1e-12)


def test_property_a_single_patch_ignores_stale_context():
    """(a) with M = 1 the patch splices every row before attending: stale values never matter."""
    st, layers = _tiny_stage(M=1, S_txt=0, S_img=9, L=2)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((9, 8))
    c = rng.standard_normal(8)
    full = st.step(x, c, warmup=True)
    st.add_noise([(rng.standard_normal((9, 8)) * 50, rng.standard_normal((9, 8)) * 50) for _ in layers])
    np.testing.assert_allclose(st.step(x, c, warmup=False), full, rtol=1e-12, atol=1e-12)


def test_property_b_buffer_holds_fresh_slice_and_untouched_rest():
    """(b) a micro-step changes only its own buffer rows, and those hold its fresh K/V."""
    st, layers = _tiny_stage(M=2, S_txt=2, S_img=8, L=2)
    rng = np.random.default_rng(14)
    x = rng.standard_normal((10, 8))
    c = rng.standard_normal(8)
    st.step(x, c, warmup=True)
    st.add_noise([(rng.standard_normal((10, 8)), rng.standard_normal((10, 8))) for _ in layers])
    st.trace = []
    st.set_cond(c)
    for off, n in st.micro_steps(False):
        before = [(k.copy(), v.copy()) for k, v in zip(st.K, st.V)]
        st.trace.clear()
        st.run_rows(off, n, x[off:off + n])
        for l in range(2):
            kb, vb = before[l]
            outside = np.ones(10, bool)
            outside[off:off + n] = False
            np.testing.assert_array_equal(st.K[l][outside], kb[outside])
            np.testing.assert_array_equal(st.V[l][outside], vb[outside])
            qkv = st.trace[l]["qkv"]
            np.testing.assert_array_equal(st.K[l][off:off + n], qkv[:, 8:16])
            np.testing.assert_array_equal(st.V[l][off:off + n], qkv[:, 16:24])


def test_patch_order_and_staleness_by_manual_composition():
    """Two image patches, one layer, attention only: patch 0 attends over [fresh 0 | stale 1],
    patch 1 over [fresh 0 | fresh 1].  Built here from the row pieces, not by the stage loop."""
    H, d, h, S = 2, 4, 8, 12
    st, layers = _tiny_stage(M=2, S_txt=0, S_img=S, L=1, r=0)
    W = layers[0]
    rng = np.random.default_rng(15)
    x = rng.standard_normal((S, h))
    c = rng.standard_normal(h)
    st.step(x, c, warmup=True)
    nk, nv = rng.standard_normal((S, h)), rng.standard_normal((S, h))
    k_stale = st.K[0] + nk
    v_stale = st.V[0] + nv
    st.add_noise([(nk, nv)])
    x2 = x + 0.5 * rng.standard_normal((S, h))       # the next step sees a changed input
    out = st.step(x2, c, warmup=False)

    mod = ref.adaln(c, W["w_ada"], W["b_ada"])
    qkv = ref.linear(ref.modulate(ref.layer_norm(x2), mod[0], mod[1]), W["w_qkv"], W["b_qkv"])
    q, kf, vf = qkv[:, :h], qkv[:, h:2 * h], qkv[:, 2 * h:]
    P = S // 2
    k0 = np.concatenate([kf[:P], k_stale[P:]])
    v0 = np.concatenate([vf[:P], v_stale[P:]])
    o0 = ref.attention(q[:P], k0, v0, H, d)
    o1 = ref.attention(q[P:], kf, vf, H, d)
    o = np.concatenate([o0, o1])
    want = x2 + mod[2] * ref.linear(o, W["w_o"], W["b_o"])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    # the stale context matters: a wrong order (later patch first) would give a different result
    assert np.abs(o0 - ref.attention(q[:P], kf, vf, H, d)).max() > 1e-3


def test_text_prefix_runs_first_each_step():
    st, _ = _tiny_stage(M=2, S_txt=2, S_img=8)
    assert st.micro_steps(False) == [(0, 2), (2, 4), (6, 4)]
    assert st.micro_steps(True) == [(0, 10)]


def test_bf16_mode_rounds_the_stored_tensors():
    st, layers = _tiny_stage(mode="bf16", M=2, S_txt=0, S_img=8, L=1)
    rng = np.random.default_rng(16)
    x = rng.standard_normal((8, 8))
    c = rng.standard_normal(8)
    st.trace = []
    st.step(x, c, warmup=True)
    for key in ("h1", "qkv", "o", "h2", "u"):
        a = st.trace[0][key]
        np.testing.assert_array_equal(ref.bf16_round(a), a)
    np.testing.assert_array_equal(ref.bf16_round(st.K[0]), st.K[0])
    exact, _ = _tiny_stage(mode="exact", M=2, S_txt=0, S_img=8, L=1)
    e = exact.step(x, c, warmup=True)
    b = st.step(x, c, warmup=True)
    rel = np.linalg.norm(e - b) / np.linalg.norm(e)
    assert 0 < rel < 2e-2


# ---------------------------------------------------------------- the pins catch planted mistakes

def test_pins_catch_planted_mistakes():
    """Plant plausible slips in the oracle (on the CPU) and check a pin above fails."""
    rng = np.random.default_rng(17)
    H, d, S = 2, 3, 7
    q = rng.standard_normal((3, H * d))
    k = rng.standard_normal((S, H * d))
    v = rng.standard_normal((S, H * d))
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), H, d))

    def wrong_scale(q, k, v, heads, head_dim, chunk=256):
        return ref.attention(q * math.sqrt(head_dim) / head_dim, k, v, heads, head_dim)
    assert np.abs(wrong_scale(q, k, v, H, d) - want).max() > 1e-3

    def swapped_kv(q, k, v, heads, head_dim, chunk=256):
        return ref.attention(q, v, k, heads, head_dim)
    assert np.abs(swapped_kv(q, k, v, H, d) - want).max() > 1e-3

    # splice after attention instead of before: property (a) with M = 1 and drift must break
    st, layers = _tiny_stage(M=1, S_txt=0, S_img=9, L=1, r=0)
    x = rng.standard_normal((9, 8))
    c = rng.standard_normal(8)
    full = st.step(x, c, warmup=True)
    st.add_noise([(rng.standard_normal((9, 8)) * 50, rng.standard_normal((9, 8)) * 50)])
    W = layers[0]
    mod = ref.adaln(c, W["w_ada"], W["b_ada"])
    qkv = ref.linear(ref.modulate(ref.layer_norm(x), mod[0], mod[1]), W["w_qkv"], W["b_qkv"])
    o_late = ref.attention(qkv[:, :8], st.K[0], st.V[0], 2, 4)   # attends over the drifted buffer
    late = x + mod[2] * ref.linear(o_late, W["w_o"], W["b_o"])
    assert np.abs(late - full).max() > 1e-2


def test_sampled_step_matches_full_step():
    st, layers = _tiny_stage(M=2, S_txt=2, S_img=8, L=2)
    st2, _ = _tiny_stage(M=2, S_txt=2, S_img=8, L=2)
    rng = np.random.default_rng(18)
    x = rng.standard_normal((10, 8))
    c = rng.standard_normal(8)
    noise = [(rng.standard_normal((10, 8)), rng.standard_normal((10, 8))) for _ in layers]
    full = st.step(x, c, warmup=True)
    rows = np.array([0, 3, 4, 9])
    np.testing.assert_allclose(st2.step_sampled(x, c, rows, warmup=True), full[rows], rtol=1e-13, atol=1e-13)
    st.add_noise(noise)
    st2.add_noise(noise)
    full = st.step(x, c)
    np.testing.assert_allclose(st2.step_sampled(x, c, rows), full[rows], rtol=1e-13, atol=1e-13)
    for l in range(2):
        np.testing.assert_array_equal(st.K[l], st2.K[l])


def test_round_p_closed_forms():
    """bf16 probabilities: exact when every weight 2^t is a power of two; with V = 1 every output is
    1 (the rounded weights are normalised by their own sum)."""
    H, d, S = 1, 4, 6
    q = np.zeros((1, 4))
    q[0, 0] = 2.0 * math.log(2.0)               # logits = k0 * ln2 (scale 1/2)
    k = np.zeros((S, 4))
    k[:, 0] = -np.arange(S)                     # weights 2^0, 2^-1, ..., 2^-5 (bf16 exact)
    v = np.random.default_rng(19).standard_normal((S, 4))
    np.testing.assert_allclose(ref.attention(q, k, v, H, d, round_p=True), ref.attention(q, k, v, H, d),
                               rtol=1e-13, atol=1e-15)
    rng = np.random.default_rng(20)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((40, 8))
    o = ref.attention(q, k, np.ones((40, 8)), 2, 4, round_p=True)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)
    v = rng.standard_normal((40, 8))
    assert np.abs(ref.attention(q, k, v, 2, 4, round_p=True) - ref.attention(q, k, v, 2, 4)).max() > 1e-5


def test_round_p_golden_two_keys():
    rows = {r[0]: [float(v) for v in r[1:]] for r in _golden_rows("attention_bf16p_two_keys.txt")}
    q = np.array([rows["q"]])
    k = np.array([rows["k0"], rows["k1"]])
    v = np.array([rows["v0"], rows["v1"]])
    np.testing.assert_allclose(ref.attention(q, k, v, 1, 4, round_p=True)[0], rows["o"], rtol=0, atol=1e-14)


def test_round_p_power_of_two_reference():
    """The bf16 weights do not depend on the power-of-two reference: shifting every score of a row
    by n ln2 (n an integer: the base-2 scores move by n) leaves the output unchanged, while a shift
    by half of that moves the rounding points and changes it.  The shift is a fifth dimension with
    q = a and k = b for every key: scores gain a b / sqrt(d)."""
    rng = np.random.default_rng(23)
    n_q, S, d = 6, 300, 5
    q = np.zeros((n_q, d))
    k = np.zeros((S, d))
    q[:, :4] = rng.standard_normal((n_q, 4)) * 1.5
    k[:, :4] = rng.standard_normal((S, 4))
    v = rng.standard_normal((S, d))
    base = ref.attention(q, k, v, 1, d, round_p=True)
    for n, same in ((3.0, True), (-5.0, True), (0.5, False), (2.25, False)):
        qs, ks = q.copy(), k.copy()
        qs[:, 4] = 1.0
        ks[:, 4] = n * math.log(2.0) * math.sqrt(d)
        got = ref.attention(qs, ks, v, 1, d, round_p=True)
        if same:
            np.testing.assert_allclose(got, base, rtol=1e-13, atol=1e-13)
        else:
            assert np.abs(got - base).max() > 1e-6, n
        np.testing.assert_allclose(ref.attention(qs, ks, v, 1, d), ref.attention(q, k, v, 1, d), rtol=1e-12,
                                   atol=1e-12)


# ---------------------------------------------------------------- MM-DiT block variants

def test_rms_norm_heads_closed_forms():
    H, d = 2, 4
    x = np.array([[3.0, 3.0, 3.0, 3.0, 1.0, -1.0, 1.0, -1.0]])
    g = np.array([1.0, 2.0, 0.5, -1.0])
    y = ref.rms_norm_heads(x, H, d, g, eps=0.0)
    np.testing.assert_allclose(y, [[1.0, 2.0, 0.5, -1.0, 1.0, -2.0, 0.5, 1.0]], rtol=1e-15)
    z = np.random.default_rng(0).standard_normal((5, H * d))
    np.testing.assert_allclose(ref.rms_norm_heads(7.5 * z, H, d, np.ones(d), eps=0.0),
                               ref.rms_norm_heads(z, H, d, np.ones(d), eps=0.0), rtol=1e-13)   # scale invariant
    assert np.allclose((ref.rms_norm_heads(z, H, d, np.ones(d), eps=0.0).reshape(5, H, d) ** 2).mean(-1), 1.0)


def test_rope_closed_forms_and_relative_positions():
    H, d = 2, 4
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, H * d))
    np.testing.assert_array_equal(ref.rope(q, H, d, np.zeros((1, d // 2))), q)                 # angle 0
    e = np.zeros((1, H * d)); e[0, 0] = 1.0
    np.testing.assert_allclose(ref.rope(e, H, d, [[math.pi / 2, 0.0]])[0, :2], [0.0, 1.0], atol=1e-15)
    r = ref.rope(q, H, d, rng.uniform(-5, 5, (1, d // 2)))
    np.testing.assert_allclose(np.linalg.norm(r.reshape(H, d // 2, 2), axis=-1),
                               np.linalg.norm(q.reshape(H, d // 2, 2), axis=-1), rtol=1e-13)   # rotation
    # 1-axis positions theta_i = i * w_k: <rope(q, i), rope(k, j)> depends on i - j only
    w = np.array([1.0, 0.1])
    k = rng.standard_normal((1, H * d))
    def dot(i, j):
        return float((ref.rope(q, H, d, [i * w]) * ref.rope(k, H, d, [j * w])).sum())
    assert dot(5, 2) == pytest.approx(dot(13, 10), rel=1e-12)
    assert dot(5, 2) != pytest.approx(dot(5, 3), rel=1e-6)


def _mmdit_layers(L, h, r, d, seed):
    layers = _tiny_layers(L, h, r, seed)
    rng = np.random.default_rng(seed + 50)
    for W in layers:
        W["q_norm"] = 1.0 + 0.3 * rng.standard_normal(d)
        W["k_norm"] = 1.0 + 0.3 * rng.standard_normal(d)
    return layers


def test_mmdit_options_vs_brute_force_two_steps():
    """Dual-stream weights, QK-RMSNorm and RoPE together: the numpy oracle against the loop
    restatement on a tiny stage with a text prefix, warm-up then a drifted patched step."""
    H, d, r, L, S_txt, S_img, M = 2, 4, 2, 2, 2, 8, 2
    h, S = H * d, S_txt + S_img
    img, txt = _mmdit_layers(L, h, r, d, 30), _mmdit_layers(L, h, r, d, 31)
    rng = np.random.default_rng(12)
    ang = rng.uniform(-3, 3, (S, d // 2))
    st = ref.StageOracle(img, heads=H, head_dim=d, seq_txt=S_txt, seq_img=S_img, num_patches=M, mlp_ratio=r,
                         txt_layers=txt, qk_norm=True, rope_angles=ang)
    x = rng.standard_normal((S, h))
    c = rng.standard_normal(h)
    noise = [(rng.standard_normal((S, h)) * 0.1, rng.standard_normal((S, h)) * 0.1) for _ in range(L)]
    kb = [[[0.0] * h for _ in range(S)] for _ in range(L)]
    vb = [[[0.0] * h for _ in range(S)] for _ in range(L)]
    lw = [{k: a.tolist() for k, a in W.items()} for W in img]
    tw = [{k: a.tolist() for k, a in W.items()} for W in txt]
    kw = dict(heads=H, d=d, seq_txt=S_txt, num_patches=M, mlp_ratio=r, txt_layers=tw, qk_norm=True,
              rope_angles=ang.tolist())
    np.testing.assert_allclose(st.step(x, c, warmup=True),
                               brute.stage_step(lw, kb, vb, x.tolist(), c.tolist(), warmup=True, **kw),
                               rtol=1e-11, atol=1e-11)
    st.add_noise(noise)
    for l, (nk, nv) in enumerate(noise):
        kb[l] = (np.array(kb[l]) + nk).tolist()
        vb[l] = (np.array(vb[l]) + nv).tolist()
    np.testing.assert_allclose(st.step(x, c, warmup=False),
                               brute.stage_step(lw, kb, vb, x.tolist(), c.tolist(), warmup=False, **kw),
                               rtol=1e-11, atol=1e-11)
    for l in range(L):
        np.testing.assert_allclose(st.K[l], kb[l], rtol=1e-12, atol=1e-12)


def test_dual_stream_with_equal_weights_is_the_single_stream_block():
    H, d, r, L, S_txt, S_img, M = 2, 4, 2, 2, 3, 8, 2
    h, S = H * d, S_txt + S_img
    img = _mmdit_layers(L, h, r, d, 40)
    rng = np.random.default_rng(13)
    x, c = rng.standard_normal((S, h)), rng.standard_normal(h)
    kw = dict(heads=H, head_dim=d, seq_txt=S_txt, seq_img=S_img, num_patches=M, mlp_ratio=r, qk_norm=True)
    one = ref.StageOracle(img, **kw)
    two = ref.StageOracle(img, txt_layers=[dict(W) for W in img], **kw)
    for warm in (True, False):
        np.testing.assert_array_equal(one.step(x, c, warmup=warm), two.step(x, c, warmup=warm))


def _parallel_layers(L, h, r, d, seed, std=0.3):
    """Weights of the parallel (Flux.1 single-stream) block: w_qkv [3h,h], w1 [rh,h],
    w2 [h, h + rh], w_ada [3h,h], plus q_norm / k_norm [d]."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(L):
        out.append({"w_qkv": rng.standard_normal((3 * h, h)) * std, "b_qkv": rng.standard_normal(3 * h) * std,
                    "w1": rng.standard_normal((r * h, h)) * std, "b1": rng.standard_normal(r * h) * std,
                    "w2": rng.standard_normal((h, h + r * h)) * std, "b2": rng.standard_normal(h) * std,
                    "w_ada": rng.standard_normal((3 * h, h)) * std, "b_ada": rng.standard_normal(3 * h) * std,
                    "q_norm": 1.0 + 0.3 * rng.standard_normal(d), "k_norm": 1.0 + 0.3 * rng.standard_normal(d)})
    return out


def test_parallel_block_vs_brute_force_two_steps():
    """The parallel block with QK-RMSNorm and RoPE: numpy oracle against the loop restatement,
    warm-up then a drifted patched step, with a text prefix."""
    H, d, r, L, S_txt, S_img, M = 2, 4, 2, 2, 2, 8, 2
    h, S = H * d, S_txt + S_img
    lw = _parallel_layers(L, h, r, d, 60)
    rng = np.random.default_rng(14)
    ang = rng.uniform(-3, 3, (S, d // 2))
    st = ref.StageOracle(lw, heads=H, head_dim=d, seq_txt=S_txt, seq_img=S_img, num_patches=M, mlp_ratio=r,
                         qk_norm=True, rope_angles=ang, parallel=True)
    x, c = rng.standard_normal((S, h)), rng.standard_normal(h)
    noise = [(rng.standard_normal((S, h)) * 0.1, rng.standard_normal((S, h)) * 0.1) for _ in range(L)]
    kb = [[[0.0] * h for _ in range(S)] for _ in range(L)]
    vb = [[[0.0] * h for _ in range(S)] for _ in range(L)]
    bw = [{k: a.tolist() for k, a in W.items()} for W in lw]
    kw = dict(heads=H, d=d, seq_txt=S_txt, num_patches=M, mlp_ratio=r, qk_norm=True, rope_angles=ang.tolist(),
              parallel=True)
    np.testing.assert_allclose(st.step(x, c, warmup=True),
                               brute.stage_step(bw, kb, vb, x.tolist(), c.tolist(), warmup=True, **kw),
                               rtol=1e-11, atol=1e-11)
    st.add_noise(noise)
    for l, (nk, nv) in enumerate(noise):
        kb[l] = (np.array(kb[l]) + nk).tolist()
        vb[l] = (np.array(vb[l]) + nv).tolist()
    np.testing.assert_allclose(st.step(x, c, warmup=False),
                               brute.stage_step(bw, kb, vb, x.tolist(), c.tolist(), warmup=False, **kw),
                               rtol=1e-11, atol=1e-11)
    for l in range(L):
        np.testing.assert_allclose(st.K[l], kb[l], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st.V[l], vb[l], rtol=1e-12, atol=1e-12)


def _standard_from_parallel(pw, h, *, attn_only):
    """DiT-block weights that compute what a parallel block computes in one of two special
    cases: attn_only (its W2 has zero MLP columns) -> the attention-only block (r = 0) with
    W_o = W2[:, :h]; otherwise (its V projection is zero, so o = 0) -> a block whose attention
    sublayer adds nothing (W_o = 0, b_o = 0) and whose MLP sublayer uses the same shift, scale
    and gate, W1, b1, W2[:, h:], b2."""
    sw = {"w_qkv": pw["w_qkv"], "b_qkv": pw["b_qkv"], "q_norm": pw["q_norm"], "k_norm": pw["k_norm"]}
    if attn_only:
        sw.update(w_o=pw["w2"][:, :h], b_o=pw["b2"], w1=np.zeros((0, h)), b1=np.zeros(0), w2=np.zeros((h, 0)),
                  b2=np.zeros(h), w_ada=np.concatenate([pw["w_ada"], np.zeros((3 * h, h))]),
                  b_ada=np.concatenate([pw["b_ada"], np.zeros(3 * h)]))
    else:
        sw.update(w_o=np.zeros((h, h)), b_o=np.zeros(h), w1=pw["w1"], b1=pw["b1"], w2=pw["w2"][:, h:], b2=pw["b2"],
                  w_ada=np.concatenate([pw["w_ada"], pw["w_ada"]]), b_ada=np.concatenate([pw["b_ada"], pw["b_ada"]]))
    return sw


@pytest.mark.parametrize("attn_only", [True, False], ids=["zero-mlp-columns", "zero-values"])
def test_parallel_block_special_cases_reduce_to_the_dit_block(attn_only):
    """Two special cases of the parallel block equal the (separately pinned) DiT block: with
    W2's MLP columns zero it is the attention-only block with W_o = W2[:, :h]; with a zero V
    projection it is the MLP sublayer alone (same modulation) with W2's MLP columns.  A swapped
    [u, o] order, a wrong modulation chunk or a second LayerNorm fails one of them."""
    H, d, r, L, S_txt, S_img, M = 2, 4, 2, 2, 2, 8, 2
    h, S = H * d, S_txt + S_img
    lw = _parallel_layers(L, h, r, d, 70)
    for W in lw:
        if attn_only:
            W["w2"][:, h:] = 0.0
        else:
            W["w_qkv"][2 * h:] = 0.0
            W["b_qkv"][2 * h:] = 0.0
    rng = np.random.default_rng(15)
    ang = rng.uniform(-3, 3, (S, d // 2))
    x, c = rng.standard_normal((S, h)), rng.standard_normal(h)
    kw = dict(heads=H, head_dim=d, seq_txt=S_txt, seq_img=S_img, num_patches=M, qk_norm=True, rope_angles=ang)
    par = ref.StageOracle(lw, mlp_ratio=r, parallel=True, **kw)
    std = ref.StageOracle([_standard_from_parallel(W, h, attn_only=attn_only) for W in lw],
                          mlp_ratio=0 if attn_only else r, **kw)
    for warm in (True, False):
        np.testing.assert_allclose(par.step(x, c, warmup=warm), std.step(x, c, warmup=warm), rtol=1e-12, atol=1e-12)


def test_round_p_pins_catch_planted_mistakes():
    """Two plausible slips in the bf16-probability definition fail the pins above: rounding the
    weights relative to the exact row maximum (a non-power-of-two reference) misses the golden
    value, and normalising by the sum of the unrounded weights breaks the V = 1 identity."""
    rows = {r[0]: [float(v) for v in r[1:]] for r in _golden_rows("attention_bf16p_two_keys.txt")}
    q = np.array([rows["q"]])
    k = np.array([rows["k0"], rows["k1"]])
    v = np.array([rows["v0"], rows["v1"]])
    s = q @ k.T / 2.0
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    w = ref.bf16_round(e)
    exact_max_ref = (w @ v) / w.sum(axis=-1, keepdims=True)
    assert np.abs(exact_max_ref[0] - rows["o"]).max() > 1e-5
    rng = np.random.default_rng(20)
    q = rng.standard_normal((5, 4))
    k = rng.standard_normal((40, 4))
    t = (q @ k.T / 2.0) / math.log(2.0)
    w = np.exp2(t - np.ceil(t.max(axis=-1, keepdims=True)))
    unrounded_sum = (ref.bf16_round(w) @ np.ones((40, 4))) / w.sum(axis=-1, keepdims=True)
    assert np.abs(unrounded_sum - 1.0).max() > 1e-6
