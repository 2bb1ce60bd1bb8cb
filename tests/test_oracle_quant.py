"""Pins of the oracle's int8-projection variant (oracle/quant.py) against
facts fixed outside it: hand-worked codes, exact power-of-two invariance,
the round-to-nearest error bound, brute-force integer sums, a lossless
special case equal to the float product, a library bf16 rounding, and the
variant's distance from the float forward at the tiny workload."""

import numpy as np
import pytest

import synthetic
from oracle import model as om
from oracle import quant as qz
from tests import helpers


def test_codes_worked_example():
    """amax 127 gives scale = inv = 1, so codes are rint of the values: ties
    go to the even integer, signs are kept."""
    x = np.array([[127.0, -63.5, 0.5, 1.5, 2.5, -2.5, 0.0, 126.5, -0.49]], np.float32)
    q, s = qz.quantize_rows(x)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, -64, 0, 2, 2, -2, 0, 126, 0]]


def test_max_maps_to_127_and_zero_row():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    x[3] = 0.0
    q, s = qz.quantize_rows(x)
    assert s[3] == 0 and not q[3].any()
    for r in (0, 1, 2, 4):
        k = np.argmax(np.abs(x[r]))
        assert abs(int(q[r, k])) == 127 and np.sign(q[r, k]) == np.sign(x[r, k])
        assert s[r] == np.float32(np.float32(np.abs(x[r]).max()) / np.float32(127))


@pytest.mark.parametrize("k", [-7, -1, 3, 12])
def test_power_of_two_invariance(k):
    """Scaling a row by 2^k scales amax, scale and 127/amax exactly, so the
    codes are unchanged and the scale moves by 2^k."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 1000)).astype(np.float32)
    q0, s0 = qz.quantize_rows(x)
    q1, s1 = qz.quantize_rows(x * np.float32(2.0 ** k))
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


def test_round_to_nearest_error_bound():
    """|x - q s| is at most half a step (plus the fp32 rounding of x * inv)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 3840)) * rng.uniform(0.01, 100, (16, 1))).astype(np.float32)
    q, s = qz.quantize_rows(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None])
    bound = s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -22)
    assert np.all(err <= bound)


def test_int_matmul_brute_force():
    rng = np.random.default_rng(4)
    qa = rng.integers(-127, 128, (5, 37)).astype(np.int8)
    qw = rng.integers(-127, 128, (7, 37)).astype(np.int8)
    got = qz.int_matmul(qa, qw)
    for i in range(5):
        for j in range(7):
            assert got[i, j] == sum(int(qa[i, k]) * int(qw[j, k]) for k in range(37))
    # extreme magnitude: every term 127 * 127 over a long K stays exact
    big = np.full((1, 10240), 127, np.int8)
    assert qz.int_matmul(big, -big)[0, 0] == -10240 * 127 * 127


def test_lossless_case_equals_float_product():
    """Rows whose values are integers with max |v| = 127 quantize with scale
    1 and codes equal to the values, so the int8 product is the exact float
    product."""
    rng = np.random.default_rng(5)
    x = rng.integers(-127, 128, (6, 256)).astype(np.float32)
    w = rng.integers(-127, 128, (9, 256)).astype(np.float32)
    x[:, 0] = 127
    w[:, 1] = -127
    assert np.array_equal(qz.int8_linear(x, w), x.astype(np.float64) @ w.astype(np.float64).T)


def test_int8_linear_error_bound():
    """Per output: |int8(x, w) - x w^T| <= sum_k |x_k| dw + |w_k| dx + dx dw
    with dx, dw the half-steps (+ the fp32 rounding slack of the codes)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    w = synthetic.bf16_round(rng.standard_normal((16, 512)).astype(np.float32) * 0.02)
    got = qz.int8_linear(x, w)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    _, sx = qz.quantize_rows(x)
    _, sw = qz.quantize_rows(w)
    dx = sx.astype(np.float64)[:, None] * (0.5 + 1e-5)
    dw = sw.astype(np.float64)[:, None] * (0.5 + 1e-5)
    bound = (np.abs(x) @ np.ones((512, 16))) * dw.T + dx * (np.ones((8, 512)) @ np.abs(w).T) + 512 * dx * dw.T
    assert np.all(np.abs(got - ref) <= bound)
    assert helpers.rel_l2(got, ref) < 0.02  # and far inside it in aggregate


def test_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]  # exact ties, both directions
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(qz.to_bf16(x), ref)


def test_int8_forward_near_float_forward_tiny():
    """The int8 variant of the tiny single-block workload stays within 2 %
    (rel-L2) of the float forward, and is not identical to it (the
    projections really are quantized)."""
    wl = synthetic.WORKLOADS["tiny_block"]
    cfg = helpers.oracle_config(wl["model"])
    W = helpers.oracle_weights(wl["model"]).materialize(workers=4)
    lat = synthetic.latent(wl["latent"])
    caps = synthetic.captions(wl["caption_lens"])
    ref = om.forward(cfg, W, lat, caps, wl["t"])
    got = om.forward(cfg, W, lat, caps, wl["t"], quant="int8")
    r = helpers.rel_l2(got, ref)
    assert 1e-5 < r < 2e-2, r
    assert helpers.cosine(got, ref) > 0.9996


def test_sylvester_hadamard_closed_form():
    """H_n[i, j] = (-1)^popcount(i & j); H H^T = n I."""
    for n in (1, 2, 8, 128):
        H = qz.sylvester_hadamard(n)
        want = np.array([[(-1) ** bin(i & j).count("1") for j in range(n)] for i in range(n)], np.float64)
        assert np.array_equal(H, want)
        assert np.array_equal(H @ H.T, n * np.eye(n))


def test_fwht_equals_matrix_product():
    """On small integers every butterfly is exact in fp32, so the fast
    transform equals the block-wise product with H_128 exactly; on random
    values, to fp32 rounding."""
    rng = np.random.default_rng(8)
    H = qz.sylvester_hadamard(128)
    xi = rng.integers(-1000, 1001, (3, 384)).astype(np.float32)
    want = (xi.astype(np.float64).reshape(3, 3, 128) @ H).reshape(3, 384)
    assert np.array_equal(qz.fwht_rows(xi).astype(np.float64), want)
    xr = rng.standard_normal((4, 256)).astype(np.float32)
    want = (xr.astype(np.float64).reshape(4, 2, 128) @ H).reshape(4, 256)
    assert np.allclose(qz.fwht_rows(xr), want, rtol=0, atol=1e-5 * np.abs(xr).max() * 128)


def test_rotation_cancels_in_the_product():
    """(x H)(w H)^T = 128 x w^T, so the rotated int8 product estimates the
    same x w^T; for a heavy-tailed x (a product of two normals, like the
    SwiGLU product) it does so with a smaller error than without rotation."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 1024)) * rng.standard_normal((16, 1024))).astype(np.float32)
    w = synthetic.bf16_round(rng.standard_normal((32, 1024)).astype(np.float32) * 0.02)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rot = qz.fwht_rows(x).astype(np.float64) @ qz.fwht_rows(w).astype(np.float64).T / 128
    assert np.allclose(rot, ref, rtol=0, atol=1e-4 * np.abs(ref).max())
    e_rot = helpers.rel_l2(qz.int8_linear(x, w, rotate=True), ref)
    e_plain = helpers.rel_l2(qz.int8_linear(x, w), ref)
    assert e_rot < 0.75 * e_plain, (e_rot, e_plain)
    # the weight scales carry the exact 1/128
    _, s = qz.quantize_rows(qz.fwht_rows(w))
    _, sr = qz.quantize_rotated_rows(w, weight=True)
    assert np.array_equal(sr * np.float32(128), s)
