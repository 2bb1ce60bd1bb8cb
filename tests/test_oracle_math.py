"""Pins of the oracle's arithmetic against closed forms, invariances, brute
force on tiny inputs and independent library routines (torch, CPU, float64).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a swapped chunk) fails it.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic
from oracle import ModelConfig, manifest
from oracle import model as om
from oracle import sampler as osm

TINY = ModelConfig(hidden=256, n_heads=2, ffn=384, n_layers=1, n_noise_refiner=1,
                   n_context_refiner=1, cap_feat_dim=64, t_mid=64)


def _weights(cfg, seed=0):
    return synthetic.SyntheticWeights(manifest(cfg), seed=seed).materialize(workers=2)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------- norms

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 33))
    w = rng.uniform(0.5, 1.5, 33)
    ref = torch.nn.functional.rms_norm(_t(x), (33,), _t(w), eps=1e-5).numpy()
    np.testing.assert_allclose(om.rms_norm(x, w, 1e-5), ref, rtol=1e-13, atol=0)


def test_rms_norm_scale_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    w = np.ones(64)
    # exact for powers of two, eps = 0
    for k in (-6, 3, 11):
        assert np.array_equal(om.rms_norm(x * 2.0 ** k, w, 0.0), om.rms_norm(x, w, 0.0))
    # any positive factor, eps = 0, to rounding
    np.testing.assert_allclose(om.rms_norm(3.7 * x, w, 0.0), om.rms_norm(x, w, 0.0), rtol=1e-14)
    # with eps > 0 the output moves by at most ~eps / (2 mean x^2) relative
    eps, a = 1e-5, 1e-2
    ms = np.mean((a * x) ** 2, axis=-1, keepdims=True)
    dev = np.abs(om.rms_norm(a * x, w, eps) / om.rms_norm(x, w, 0.0) - 1.0)
    assert np.all(dev <= eps / (2 * ms) * 1.01 + 1e-14)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 50)) * 3 + 1.5
    ref = torch.nn.functional.layer_norm(_t(x), (50,), eps=1e-6).numpy()
    np.testing.assert_allclose(om.layer_norm(x, 1e-6), ref, rtol=1e-12, atol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(om.silu(x), torch.nn.functional.silu(_t(x)).numpy(), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- timestep embedding

def test_timestep_embedding_closed_form():
    cfg = ModelConfig()
    t = np.array([0.0, 0.25, 0.5, 0.9])
    e = om.timestep_embedding(cfg, t)
    assert e.shape == (4, 256)
    assert np.array_equal(e[0, :128], np.ones(128)) and np.array_equal(e[0, 128:], np.zeros(128))
    # f_0 = 1 -> cos(1000 t), sin(1000 t); f_64 = 10000^(-1/2) = 1/100 -> cos(10 t)
    np.testing.assert_allclose(e[:, 0], np.cos(1000 * t), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(e[:, 128], np.sin(1000 * t), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(e[:, 64], np.cos(10 * t), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(e[:, 128 + 64], np.sin(10 * t), rtol=1e-14, atol=1e-14)
    # f_1 = 10000^(-1/128): e[1] = cos(1000 t f_1) written with a power instead of exp/log
    np.testing.assert_allclose(e[:, 1], np.cos(1000 * t * 10000.0 ** (-1 / 128)), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_position_ids_reading():
    cap, img = om.position_ids(3, 2, 4)
    assert cap.tolist() == [[1, 0, 0], [2, 0, 0], [3, 0, 0]]
    assert img.shape == (8, 3)
    assert img[:, 0].tolist() == [4] * 8
    assert img[5].tolist() == [4, 1, 1]  # token n = i*Wp + j, i=1, j=1
    assert len({tuple(r) for r in np.concatenate([cap, img]).tolist()}) == 11


def test_rope_table_closed_form_entries():
    cfg = ModelConfig()
    ids = np.array([[0, 0, 0], [5, 7, 11], [100, 3, 250]], dtype=np.int32)
    cos, sin = om.rope_tables(cfg, ids)
    assert cos.dtype == np.float32 and cos.shape == (3, 64)
    # position 0 is the identity rotation
    assert np.array_equal(cos[0], np.ones(64, np.float32))
    assert np.array_equal(sin[0], np.zeros(64, np.float32))
    # pair 0 of each axis turns at omega = 1; pair d/4 at 256^(-1/2) = 1/16
    # axis 0 pairs are 0..15, axis 1 pairs 16..39, axis 2 pairs 40..63
    for row in (1, 2):
        p0, p1, p2 = (float(v) for v in ids[row])
        assert cos[row, 0] == np.float32(math.cos(p0)) and sin[row, 0] == np.float32(math.sin(p0))
        assert cos[row, 8] == np.float32(math.cos(p0 / 16))
        assert cos[row, 16] == np.float32(math.cos(p1)) and sin[row, 16] == np.float32(math.sin(p1))
        assert cos[row, 16 + 12] == np.float32(math.cos(p1 / 16))
        assert cos[row, 40] == np.float32(math.cos(p2))
        assert sin[row, 40 + 12] == np.float32(math.sin(p2 / 16))
        # last pair of axis 1 (r = 23): omega = 256^(-46/48)
        assert cos[row, 39] == np.float32(math.cos(p1 * 256.0 ** (-46.0 / 48)))


def test_rope_axis_sections_are_independent():
    cfg = ModelConfig()
    base = np.array([[9, 4, 6]], dtype=np.int32)
    c0, s0 = om.rope_tables(cfg, base)
    for axis, sl in ((0, slice(0, 16)), (1, slice(16, 40)), (2, slice(40, 64))):
        moved = base.copy()
        moved[0, axis] += 3
        c1, s1 = om.rope_tables(cfg, moved)
        changed = np.zeros(64, bool)
        changed[sl] = True
        assert np.all(c1[0, ~changed] == c0[0, ~changed])
        assert np.all(s1[0, ~changed] == s0[0, ~changed])
        assert np.all((c1[0, changed] != c0[0, changed]) | (s1[0, changed] != s0[0, changed]))


def test_apply_rope_is_complex_multiplication():
    cfg = ModelConfig()
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 64, size=(6, 3)).astype(np.int32)
    cos, sin = om.rope_tables(cfg, ids)
    x = rng.standard_normal((6, 2, 128))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (cos.astype(np.float64) + 1j * sin.astype(np.float64))[:, None, :]
    y = om.apply_rope(x, cos, sin)
    np.testing.assert_allclose(y[..., 0::2], z.real, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y[..., 1::2], z.imag, rtol=1e-13, atol=1e-14)


def test_rope_preserves_norm_and_is_relative():
    cfg = ModelConfig()
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    p, pk = np.array([[3, 10, 2]]), np.array([[7, 1, 30]])
    cq, sq = om.rope_tables(cfg, p)
    ck, sk = om.rope_tables(cfg, pk)
    rq, rk = om.apply_rope(q, cq, sq), om.apply_rope(k, ck, sk)
    np.testing.assert_allclose(np.linalg.norm(rq), np.linalg.norm(q), rtol=1e-6)
    dot = float(np.sum(rq * rk))
    for delta in ([5, 0, 0], [0, 9, 0], [0, 0, 13], [2, 3, 4]):
        d = np.array([delta])
        cq2, sq2 = om.rope_tables(cfg, p + d)
        ck2, sk2 = om.rope_tables(cfg, pk + d)
        dot2 = float(np.sum(om.apply_rope(q, cq2, sq2) * om.apply_rope(k, ck2, sk2)))
        assert abs(dot2 - dot) <= 1e-5 * (1 + abs(dot))


# ---------------------------------------------------------------- attention

def test_attention_brute_force():
    rng = np.random.default_rng(6)
    S, H, hd = 9, 2, 8
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    ref = np.zeros((S, H, hd))
    for h in range(H):
        for i in range(S):
            scores = [sum(q[i, h, d] * k[j, h, d] for d in range(hd)) / math.sqrt(hd) for j in range(S)]
            m = max(scores)
            ex = [math.exp(s - m) for s in scores]
            z = sum(ex)
            for d in range(hd):
                ref[i, h, d] = sum(ex[j] * v[j, h, d] for j in range(S)) / z
    np.testing.assert_allclose(om.attention(q, k, v), ref, rtol=1e-12, atol=1e-14)


def test_attention_matches_torch_sdpa_and_key_order():
    rng = np.random.default_rng(7)
    Sq, Sk, H, hd = 12, 20, 3, 128
    q = rng.standard_normal((Sq, H, hd))
    k = rng.standard_normal((Sk, H, hd))
    v = rng.standard_normal((Sk, H, hd))
    ref = torch.nn.functional.scaled_dot_product_attention(
        _t(q).transpose(0, 1), _t(k).transpose(0, 1), _t(v).transpose(0, 1)).transpose(0, 1).numpy()
    out = om.attention(q, k, v, q_chunk=5)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)
    perm = rng.permutation(Sk)
    np.testing.assert_allclose(om.attention(q, k[perm], v[perm]), out, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- FFN and block

def test_swiglu_single_token_by_hand():
    rng = np.random.default_rng(8)
    D, F = 5, 3
    W = {"b.feed_forward.w1.weight": rng.standard_normal((F, D)),
         "b.feed_forward.w3.weight": rng.standard_normal((F, D)),
         "b.feed_forward.w2.weight": rng.standard_normal((D, F))}
    h = rng.standard_normal((1, D))
    ref = np.zeros(D)
    for o in range(D):
        for j in range(F):
            a = sum(W["b.feed_forward.w1.weight"][j, i] * h[0, i] for i in range(D))
            b = sum(W["b.feed_forward.w3.weight"][j, i] * h[0, i] for i in range(D))
            ref[o] += W["b.feed_forward.w2.weight"][o, j] * (a / (1 + math.exp(-a))) * b
    np.testing.assert_allclose(om.swiglu_ffn(W, "b", h)[0], ref, rtol=1e-12)


def _block_inputs(cfg, seed=0, S=24):
    W = _weights(cfg, seed)
    x = synthetic.residual((S, cfg.hidden), seed=seed).astype(np.float64)
    rng = np.random.default_rng(seed + 100)
    ids = rng.integers(0, 40, size=(S, 3)).astype(np.int32)
    cos, sin = om.rope_tables(cfg, ids)
    c = synthetic.modulation_input(1, cfg.adaln_dim, seed=seed)[0].astype(np.float64)
    return W, x, cos, sin, c


def test_fp16_safe_rescale_is_exact():
    """w3 / 64 with w2 * 64 leaves the block bit-identical; to_out and w2 by
    1/64 in front of their RMSNorm is exact with eps = 0 ([MNN] "Conversion
    details")."""
    cfg = TINY
    W, x, cos, sin, c = _block_inputs(cfg)
    p = "layers.0"
    mod = om.block_modulation(W, p, c)
    ref = om.block(cfg, W, p, x, cos, sin, mod)
    W2 = dict(W)
    W2[f"{p}.feed_forward.w3.weight"] = W[f"{p}.feed_forward.w3.weight"] / 64
    W2[f"{p}.feed_forward.w2.weight"] = W[f"{p}.feed_forward.w2.weight"] * 64
    assert np.array_equal(om.block(cfg, W2, p, x, cos, sin, mod), ref)

    cfg0 = ModelConfig(**{**cfg.__dict__, "norm_eps": 0.0})
    ref0 = om.block(cfg0, W, p, x, cos, sin, mod)
    W3 = dict(W)
    W3[f"{p}.attention.to_out.0.weight"] = W[f"{p}.attention.to_out.0.weight"] / 64
    W3[f"{p}.feed_forward.w2.weight"] = W[f"{p}.feed_forward.w2.weight"] / 64
    assert np.array_equal(om.block(cfg0, W3, p, x, cos, sin, mod), ref0)


def test_block_gate_chunks_and_identity():
    cfg = TINY
    W, x, cos, sin, c = _block_inputs(cfg)
    p, D = "layers.0", cfg.hidden
    Wz = dict(W)
    aw = W[f"{p}.adaLN_modulation.0.weight"].copy()
    ab = W[f"{p}.adaLN_modulation.0.bias"].copy()
    # zero the gate chunks (1 and 3 in the order s1, g1, s2, g2): identity
    aw[D:2 * D] = 0
    ab[D:2 * D] = 0
    aw[3 * D:] = 0
    ab[3 * D:] = 0
    Wz[f"{p}.adaLN_modulation.0.weight"], Wz[f"{p}.adaLN_modulation.0.bias"] = aw, ab
    assert np.array_equal(om.block(cfg, Wz, p, x, cos, sin, om.block_modulation(Wz, p, c)), x)

    # zero only g1: the attention weights no longer matter
    Wg = dict(W)
    aw = W[f"{p}.adaLN_modulation.0.weight"].copy()
    ab = W[f"{p}.adaLN_modulation.0.bias"].copy()
    aw[D:2 * D] = 0
    ab[D:2 * D] = 0
    Wg[f"{p}.adaLN_modulation.0.weight"], Wg[f"{p}.adaLN_modulation.0.bias"] = aw, ab
    mod = om.block_modulation(Wg, p, c)
    y = om.block(cfg, Wg, p, x, cos, sin, mod)
    Wg2 = dict(Wg)
    Wg2[f"{p}.attention.to_q.weight"] = W[f"{p}.attention.to_q.weight"] * -3.0
    Wg2[f"{p}.attention.to_out.0.weight"] = W[f"{p}.attention.to_out.0.weight"] + 1.0
    assert np.array_equal(om.block(cfg, Wg2, p, x, cos, sin, mod), y)
    assert not np.array_equal(y, x)

    # scale chunk 0 at exactly -1 zeroes the attention input: the attention
    # branch contributes RMSNorm(0) = 0
    Ws = dict(Wg)
    aw = W[f"{p}.adaLN_modulation.0.weight"].copy()
    ab = W[f"{p}.adaLN_modulation.0.bias"].copy()
    aw[:D] = 0
    ab[:D] = -1.0
    Ws[f"{p}.adaLN_modulation.0.weight"], Ws[f"{p}.adaLN_modulation.0.bias"] = aw, ab
    s1, g1, s2, g2 = om.block_modulation(Ws, p, c)
    assert np.all(s1 == 0)
    cap_only_ffn = om.block(cfg, Ws, p, x, cos, sin, (s1, np.ones(D), s2, g2))
    no_attn = dict(Ws)
    no_attn[f"{p}.attention.to_v.weight"] = np.zeros_like(W[f"{p}.attention.to_v.weight"])
    assert np.array_equal(om.block(cfg, no_attn, p, x, cos, sin, (s1, np.ones(D), s2, g2)), cap_only_ffn)


def test_unmodulated_equals_unit_modulation():
    cfg = TINY
    W, x, cos, sin, _ = _block_inputs(cfg)
    p, D = "context_refiner.0", cfg.hidden
    one = np.ones(D)
    assert np.array_equal(om.block(cfg, W, p, x, cos, sin, None),
                          om.block(cfg, W, p, x, cos, sin, (one, one, one, one)))


def test_block_rows_subset_and_sequence_order():
    cfg = TINY
    W, x, cos, sin, c = _block_inputs(cfg, S=20)
    p = "layers.0"
    mod = om.block_modulation(W, p, c)
    full = om.block(cfg, W, p, x, cos, sin, mod)
    rows = np.array([0, 7, 19])
    np.testing.assert_allclose(om.block(cfg, W, p, x, cos, sin, mod, rows=rows), full[rows], rtol=1e-12, atol=1e-12)
    # the token order inside the sequence does not matter (positions travel with tokens)
    perm = np.random.default_rng(9).permutation(20)
    np.testing.assert_allclose(om.block(cfg, W, p, x[perm], cos[perm], sin[perm], mod), full[perm],
                               rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- patches, final layer, forward

def test_patchify_by_loops_and_inverse():
    rng = np.random.default_rng(10)
    C, Hl, Wl = 16, 6, 8
    lat = rng.standard_normal((C, Hl, Wl))
    tok = om.patchify(lat, 2)
    Wp = Wl // 2
    for i in range(Hl // 2):
        for j in range(Wp):
            for a in range(2):
                for b in range(2):
                    for ch in range(C):
                        assert tok[i * Wp + j, (a * 2 + b) * C + ch] == lat[ch, 2 * i + a, 2 * j + b]
    assert np.array_equal(om.unpatchify(tok, C, Hl, Wl, 2), lat)


def test_forward_small_batch_and_finiteness():
    cfg = TINY
    W = _weights(cfg, 1)
    lat = synthetic.latent((2, 16, 8, 6), seed=1)
    caps = synthetic.captions((5, 3), dim=cfg.cap_feat_dim, seed=1)
    t = np.array([0.5, 0.25])
    caps_b = [{}, {}]
    out = om.forward(cfg, W, lat, caps, t, captures=caps_b)
    assert out.shape == lat.shape and np.all(np.isfinite(out))
    one = om.forward(cfg, W, lat[1:], caps[1:], t[1:])
    assert np.array_equal(out[1:], one)
    assert set(caps_b[0]) >= {"x_embed", "cap_embed", "noise_refiner.0", "context_refiner.0", "layers.0", "final"}
    assert caps_b[0]["layers.0"].shape == (12 + 5, cfg.hidden)


def test_final_layer_by_hand():
    cfg = ModelConfig(hidden=4, n_heads=1, adaln_dim=2)
    rng = np.random.default_rng(11)
    W = {"all_final_layer.2-1.adaLN_modulation.1.weight": rng.standard_normal((4, 2)),
         "all_final_layer.2-1.adaLN_modulation.1.bias": rng.standard_normal(4),
         "all_final_layer.2-1.linear.weight": rng.standard_normal((3, 4)),
         "all_final_layer.2-1.linear.bias": rng.standard_normal(3)}
    x = rng.standard_normal((1, 4))
    c = rng.standard_normal(2)
    sc = W["all_final_layer.2-1.adaLN_modulation.1.weight"] @ (c / (1 + np.exp(-c))) + W["all_final_layer.2-1.adaLN_modulation.1.bias"]
    mu = x[0].sum() / 4
    var = ((x[0] - mu) ** 2).sum() / 4
    z = (x[0] - mu) / math.sqrt(var + 1e-6) * (1 + sc)
    ref = W["all_final_layer.2-1.linear.weight"] @ z + W["all_final_layer.2-1.linear.bias"]
    np.testing.assert_allclose(om.final_layer(cfg, W, x, c)[0], ref, rtol=1e-12)


# ---------------------------------------------------------------- sampler

def test_sampler_schedule_exact(golden):
    g = golden["sampler_schedule"]
    sig, t = osm.schedule(g["n_steps"], g["shift"])
    for got, want in zip(osm.base_sigmas(8), g["sigma"]):
        assert got == float(Fraction(want))
    for got, want in zip(sig, g["sigma_shifted"]):
        assert abs(got - float(Fraction(want))) <= 2e-16
    for got, want in zip(t, g["t"]):
        assert abs(got - float(Fraction(want))) <= 2e-16
    for k, want in enumerate(g["dt"]):
        assert abs((sig[k + 1] - sig[k]) - float(Fraction(want))) <= 4e-16


def test_sampler_endpoints_and_euler_sign():
    assert osm.shift_sigma(0.0, 3.0) == 0.0 and osm.shift_sigma(1.0, 3.0) == 1.0
    s = osm.shift_sigma(np.linspace(0, 1, 50), 3.0)
    assert np.all(np.diff(s) > 0)
    # shift 1 is the identity
    np.testing.assert_allclose(osm.shift_sigma(np.linspace(0, 1, 9), 1.0), np.linspace(0, 1, 9), rtol=0, atol=0)
    # a model that returns noise - x0 (the flow target) carries x from noise to x0
    x0 = np.array([[0.3, -1.2]])
    noise = np.array([[1.0, 2.0]])
    sig, _ = osm.schedule(8, 3.0)
    x = noise.copy()
    for k in range(8):
        # the model's raw output is the negated flow target (output negated before the step)
        x = osm.euler_step(x, -(noise - x0), sig[k], sig[k + 1])
    np.testing.assert_allclose(x, x0, rtol=1e-12, atol=1e-12)


def test_cfg_guidance_algebra():
    """The pipeline's scale g is the UI scale minus one: c + g (c - u) equals
    the textbook u + s (c - u) with s = g + 1; g = 0 and c = u give c."""
    rng = np.random.default_rng(3)
    c, u = rng.standard_normal((2, 5, 7))
    for s_ui in (1.0, 4.0, 5.0):
        np.testing.assert_allclose(osm.guided_output(c, u, s_ui - 1.0), u + s_ui * (c - u), rtol=1e-12, atol=1e-12)
    assert np.array_equal(osm.guided_output(c, u, 0.0), c)
    assert np.array_equal(osm.guided_output(c, c, 3.0), c)


def test_cfg_loop_reduces_to_plain_loop_and_closed_form():
    rng = np.random.default_rng(4)
    x0 = rng.standard_normal((1, 3))
    a, b = rng.standard_normal((2, 1, 3))
    calls = []

    def model(x, t, cond):  # raw output x - target: a velocity field pulling towards the target
        calls.append(cond)
        return x - (a if cond else b)

    # g = 0: the conditional forward only, identical to the plain loop
    plain = osm.run(lambda x, t: model(x, t, True), x0, n_steps=6, shift=3.0)
    calls.clear()
    np.testing.assert_array_equal(osm.run_cfg(model, x0, n_steps=6, shift=3.0, guidance=0.0), plain)
    assert calls == [True] * 6
    # guided output x - a', a' = a + g (a - b); Euler: x_{k+1} - a' = (x_k - a') (1 + sig_k - sig_{k+1})
    g = 2.5
    ap = a + g * (a - b)
    sig, _ = osm.schedule(6, 3.0)
    want = ap + (x0 - ap) * np.prod(1.0 + sig[:-1] - sig[1:])
    calls.clear()
    got = osm.run_cfg(model, x0, n_steps=6, shift=3.0, guidance=g)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert calls.count(False) == 6


def test_cfg_truncation_switches_guidance_off_late():
    _, t = osm.schedule(8, 3.0)
    assert all(osm.guidance_active(tk, 1.0) for tk in t)  # default: every step
    on = [osm.guidance_active(tk, 0.5) for tk in t]
    assert on == [tk <= 0.5 for tk in t] and any(on) and not all(on)
    assert on == sorted(on, reverse=True)  # a prefix of the steps (t grows towards clean)
    calls = []

    def model(x, tt, cond):
        calls.append(cond)
        return 0.1 * x

    osm.run_cfg(model, np.ones((1, 2)), n_steps=8, shift=3.0, guidance=3.0, cfg_truncation=0.5)
    assert calls.count(False) == sum(on) and calls.count(True) == 8
