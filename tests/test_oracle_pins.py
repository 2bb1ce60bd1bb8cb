"""By-hand pins of the oracle parts whose wiring no invariance fixes: the
timestep MLP, the caption embedder and one modulated block with non-zero
gates and non-uniform QK-norm weights.

Each reference below is written out in scalar Python loops (``math`` only),
and where a library routine computes the same thing (torch's Linear, SiLU,
rms_norm, SDPA, in float64 on the CPU) it is compared too.  Every test also
shows that the mutation it is meant to catch moves the result far outside
its tolerance, so the pin discriminates.

Structure followed ("Z-Image", ostris AI Toolkit docs, Architecture and
Components): adaLN modulation from a 256-d timestep embedding through a
two-layer MLP, caption features RMS-normalised then projected to the hidden
width, QK-RMSNorm followed by the 3-axis RoPE, tanh-gated residual branches.
"""

import math

import numpy as np
import torch

from oracle import ModelConfig
from oracle import model as om

TOL = 1e-10


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _matvec(Wm, v, b=None):
    out = []
    for r in range(len(Wm)):
        s = 0.0
        for c in range(len(v)):
            s += Wm[r][c] * v[c]
        out.append(s + (b[r] if b is not None else 0.0))
    return out


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


# ---------------------------------------------------------------- timestep MLP

def test_timestep_mlp_by_hand():
    """c = W2 SiLU(W1 e + b1) + b2, e = [cos(1000 t f), sin(1000 t f)].

    Catches: a dropped or misplaced SiLU (after the second linear, or on e),
    the two layers applied in the other order, a dropped bias, and the sine
    half placed first."""
    cfg = ModelConfig(adaln_dim=6, t_mid=5)
    rng = np.random.default_rng(21)
    W = {"t_embedder.mlp.0.weight": rng.standard_normal((5, 6)),
         "t_embedder.mlp.0.bias": rng.standard_normal(5),
         "t_embedder.mlp.2.weight": rng.standard_normal((6, 5)),
         "t_embedder.mlp.2.bias": rng.standard_normal(6)}
    ts = [0.0, 0.3, 0.875]
    got = om.timestep_mlp(cfg, W, np.array(ts))

    W1, b1 = W["t_embedder.mlp.0.weight"].tolist(), W["t_embedder.mlp.0.bias"].tolist()
    W2, b2 = W["t_embedder.mlp.2.weight"].tolist(), W["t_embedder.mlp.2.bias"].tolist()

    def by_hand(t, silu_mid=True, sin_first=False):
        freqs = [10000.0 ** (-i / 3.0) for i in range(3)]
        cos_h = [math.cos(1000.0 * t * f) for f in freqs]
        sin_h = [math.sin(1000.0 * t * f) for f in freqs]
        e = sin_h + cos_h if sin_first else cos_h + sin_h
        mid = _matvec(W1, e, b1)
        if silu_mid:
            mid = [_silu(v) for v in mid]
        return _matvec(W2, mid, b2)

    ref = np.array([by_hand(t) for t in ts])
    np.testing.assert_allclose(got, ref, rtol=TOL, atol=1e-12)

    # the same MLP as torch modules
    mlp = torch.nn.Sequential(torch.nn.Linear(6, 5), torch.nn.SiLU(), torch.nn.Linear(5, 6)).double()
    with torch.no_grad():
        mlp[0].weight.copy_(_t(W1))
        mlp[0].bias.copy_(_t(b1))
        mlp[2].weight.copy_(_t(W2))
        mlp[2].bias.copy_(_t(b2))
        emb = _t(om.timestep_embedding(cfg, np.array(ts)))
        np.testing.assert_allclose(got, mlp(emb).numpy(), rtol=TOL, atol=1e-12)

    # the pin discriminates
    assert _rel([by_hand(t, silu_mid=False) for t in ts], ref) > 1e-2
    assert _rel([by_hand(t, sin_first=True) for t in ts], ref) > 1e-2


# ---------------------------------------------------------------- caption embedder

def test_cap_embed_by_hand():
    """y = W_c RMSNorm(e; w, eps) + b_c with eps = norm_eps (1e-5).

    Features are scaled so that mean(e^2) is comparable to eps, so a
    missing RMSNorm, a missing norm weight, a wrong eps (1e-6), the norm
    applied after the linear, or a dropped bias all fail."""
    cfg = ModelConfig(hidden=4, n_heads=1, cap_feat_dim=7)
    rng = np.random.default_rng(22)
    W = {"cap_embedder.0.weight": rng.uniform(0.5, 1.5, 7),
         "cap_embedder.1.weight": rng.standard_normal((4, 7)),
         "cap_embedder.1.bias": rng.standard_normal(4)}
    feats = rng.standard_normal((3, 7)) * 3e-3
    got = om.cap_embed(cfg, W, feats)

    wn, Wc, bc = W["cap_embedder.0.weight"].tolist(), W["cap_embedder.1.weight"].tolist(), W["cap_embedder.1.bias"].tolist()

    def by_hand(e, eps=1e-5, norm=True):
        if norm:
            ms = sum(v * v for v in e) / len(e)
            e = [v / math.sqrt(ms + eps) * wn[i] for i, v in enumerate(e)]
        return _matvec(Wc, e, bc)

    ref = np.array([by_hand(r) for r in feats.tolist()])
    np.testing.assert_allclose(got, ref, rtol=TOL, atol=1e-12)
    lib = torch.nn.functional.linear(
        torch.nn.functional.rms_norm(_t(feats), (7,), _t(wn), eps=1e-5), _t(Wc), _t(bc)).numpy()
    np.testing.assert_allclose(got, lib, rtol=TOL, atol=1e-12)

    assert _rel([by_hand(r, eps=1e-6) for r in feats.tolist()], ref) > 1e-2
    assert _rel([by_hand(r, norm=False) for r in feats.tolist()], ref) > 1e-1


# ---------------------------------------------------------------- one modulated block

HD = 128  # head_dim; the RoPE axes [32, 48, 48] fill it


def _rope_angles(pos):
    """(axis, omega) per pair: axis a owns d_a channels, pair r turns at
    256^(-2r/d_a) ("Z-Image", Architecture: 3-axis RoPE [32, 48, 48], theta 256)."""
    out = []
    for axis, d in enumerate((32, 48, 48)):
        for r in range(d // 2):
            out.append(pos[axis] * 256.0 ** (-(2.0 * r) / d))
    return out


def _block_by_hand(Wl, x, cos, sin, c, tanh_gate=True, norm_then_rope=True):
    """One modulated S3-DiT block over the rows of x (lists), scalar loops.

    h = RMSNorm(x; n1)(1 + s1); q, k, v = h W^T; per head q, k get RMSNorm
    (norm_q / norm_k) then RoPE; softmax(q k^T / sqrt(128)) v; x += G(g1)
    RMSNorm(o Wo^T; n2); h2 = RMSNorm(x; f1)(1 + s2); x += G(g2)
    RMSNorm(w2(SiLU(w1 h2) * w3 h2); f2), with G = tanh (or identity for the
    mutation)."""
    eps = 1e-5
    D = len(x[0])
    H = D // HD
    m = _matvec(Wl["ada_w"], c, Wl["ada_b"])
    s1, g1, s2, g2 = m[:D], m[D:2 * D], m[2 * D:3 * D], m[3 * D:]
    G = math.tanh if tanh_gate else (lambda v: v)

    def rms(v, w):
        r = 1.0 / math.sqrt(sum(a * a for a in v) / len(v) + eps)
        return [a * r * w[i] for i, a in enumerate(v)]

    def rope(v, cs, sn):
        out = list(v)
        for p in range(len(cs)):
            a, b = v[2 * p], v[2 * p + 1]
            out[2 * p] = a * cs[p] - b * sn[p]
            out[2 * p + 1] = a * sn[p] + b * cs[p]
        return out

    S = len(x)
    hs = [[v * (1.0 + s1[i]) for i, v in enumerate(rms(row, Wl["n1"]))] for row in x]
    qs = [_matvec(Wl["q"], h) for h in hs]
    ks = [_matvec(Wl["k"], h) for h in hs]
    vs = [_matvec(Wl["v"], h) for h in hs]
    o = [[0.0] * D for _ in range(S)]
    for hh in range(H):
        sl = slice(hh * HD, (hh + 1) * HD)
        if norm_then_rope:
            qh = [rope(rms(qs[s][sl], Wl["nq"]), cos[s], sin[s]) for s in range(S)]
            kh = [rope(rms(ks[s][sl], Wl["nk"]), cos[s], sin[s]) for s in range(S)]
        else:
            qh = [rms(rope(qs[s][sl], cos[s], sin[s]), Wl["nq"]) for s in range(S)]
            kh = [rms(rope(ks[s][sl], cos[s], sin[s]), Wl["nk"]) for s in range(S)]
        for i in range(S):
            sc = [sum(qh[i][d] * kh[j][d] for d in range(HD)) / math.sqrt(HD) for j in range(S)]
            mx = max(sc)
            p = [math.exp(v - mx) for v in sc]
            z = sum(p)
            for d in range(HD):
                o[i][hh * HD + d] = sum(p[j] / z * vs[j][hh * HD + d] for j in range(S))
    x1 = []
    for i in range(S):
        a = rms(_matvec(Wl["out"], o[i]), Wl["n2"])
        x1.append([x[i][d] + G(g1[d]) * a[d] for d in range(D)])
    out = []
    for i in range(S):
        h2 = [v * (1.0 + s2[d]) for d, v in enumerate(rms(x1[i], Wl["f1"]))]
        a1 = _matvec(Wl["w1"], h2)
        a3 = _matvec(Wl["w3"], h2)
        f = rms(_matvec(Wl["w2"], [_silu(u) * w for u, w in zip(a1, a3)]), Wl["f2"])
        out.append([x1[i][d] + G(g2[d]) * f[d] for d in range(D)])
    return out


def test_modulated_block_by_hand():
    """Three tokens at distinct 3-axis positions, one head of 128, non-zero
    gates (tanh(g) differs from g by tens of percent) and non-uniform
    norm_q / norm_k weights (so QK-RMSNorm and RoPE do not commute).

    Catches: tanh(g) replaced by g; RoPE applied before QK-RMSNorm; a
    modulation chunk order other than (s1, g1, s2, g2); scale applied as s
    instead of 1 + s; a dropped post-norm weight."""
    D, F, A = HD, 24, 4
    cfg = ModelConfig(hidden=D, n_heads=1, ffn=F, adaln_dim=A)
    rng = np.random.default_rng(23)
    p = "layers.0"
    lin = lambda o, i, s: rng.standard_normal((o, i)) * s  # noqa: E731
    ada_b = np.concatenate([rng.uniform(-0.5, 0.5, D), rng.uniform(0.6, 1.4, D) * rng.choice([-1, 1], D),
                            rng.uniform(-0.5, 0.5, D), rng.uniform(0.6, 1.4, D) * rng.choice([-1, 1], D)])
    W = {f"{p}.adaLN_modulation.0.weight": lin(4 * D, A, 0.05),
         f"{p}.adaLN_modulation.0.bias": ada_b,
         f"{p}.attention.to_q.weight": lin(D, D, 0.3),
         f"{p}.attention.to_k.weight": lin(D, D, 0.3),
         f"{p}.attention.to_v.weight": lin(D, D, 0.1),
         f"{p}.attention.to_out.0.weight": lin(D, D, 0.1),
         f"{p}.attention.norm_q.weight": rng.uniform(0.2, 2.0, HD),
         f"{p}.attention.norm_k.weight": rng.uniform(0.2, 2.0, HD),
         f"{p}.feed_forward.w1.weight": lin(F, D, 0.1),
         f"{p}.feed_forward.w3.weight": lin(F, D, 0.1),
         f"{p}.feed_forward.w2.weight": lin(D, F, 0.2),
         f"{p}.attention_norm1.weight": rng.uniform(0.5, 1.5, D),
         f"{p}.attention_norm2.weight": rng.uniform(0.5, 1.5, D),
         f"{p}.ffn_norm1.weight": rng.uniform(0.5, 1.5, D),
         f"{p}.ffn_norm2.weight": rng.uniform(0.5, 1.5, D)}
    x = rng.standard_normal((3, D))
    ids = [(1, 0, 0), (9, 2, 5), (9, 7, 1)]
    c = rng.standard_normal(A)

    # the tables the block receives, from the angles written out above
    ang = np.array([_rope_angles(i) for i in ids])
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    got = om.block(cfg, W, p, x, cos, sin, om.block_modulation(W, p, c))

    Wl = {"ada_w": W[f"{p}.adaLN_modulation.0.weight"].tolist(), "ada_b": ada_b.tolist(),
          "q": W[f"{p}.attention.to_q.weight"].tolist(), "k": W[f"{p}.attention.to_k.weight"].tolist(),
          "v": W[f"{p}.attention.to_v.weight"].tolist(), "out": W[f"{p}.attention.to_out.0.weight"].tolist(),
          "nq": W[f"{p}.attention.norm_q.weight"].tolist(), "nk": W[f"{p}.attention.norm_k.weight"].tolist(),
          "w1": W[f"{p}.feed_forward.w1.weight"].tolist(), "w3": W[f"{p}.feed_forward.w3.weight"].tolist(),
          "w2": W[f"{p}.feed_forward.w2.weight"].tolist(),
          "n1": W[f"{p}.attention_norm1.weight"].tolist(), "n2": W[f"{p}.attention_norm2.weight"].tolist(),
          "f1": W[f"{p}.ffn_norm1.weight"].tolist(), "f2": W[f"{p}.ffn_norm2.weight"].tolist()}
    # both sides rotate by the same fp32-rounded table entries
    cs, sn = cos.astype(np.float64).tolist(), sin.astype(np.float64).tolist()
    ref = np.array(_block_by_hand(Wl, x.tolist(), cs, sn, c.tolist()))
    np.testing.assert_allclose(got, ref, rtol=TOL, atol=1e-12)

    # branches: the residual dominates the output, so compare what the block adds
    br_got, br_ref = got - x, ref - x
    assert _rel(br_got, br_ref) < TOL

    # each mutation moves the branch far beyond that tolerance
    wrong_gate = np.array(_block_by_hand(Wl, x.tolist(), cs, sn, c.tolist(), tanh_gate=False)) - x
    wrong_order = np.array(_block_by_hand(Wl, x.tolist(), cs, sn, c.tolist(), norm_then_rope=False)) - x
    assert _rel(wrong_gate, br_ref) > 1e-1
    assert _rel(wrong_order, br_ref) > 5e-2

    # attention part against torch's SDPA on the oracle's own normalised,
    # rotated q and k (library routine for the softmax-attention step)
    h = om.rms_norm(x, W[f"{p}.attention_norm1.weight"], 1e-5) * (1 + om.block_modulation(W, p, c)[0])
    q = om.apply_rope(om.rms_norm((h @ W[f"{p}.attention.to_q.weight"].T).reshape(3, 1, HD),
                                  W[f"{p}.attention.norm_q.weight"], 1e-5), cos, sin)
    k = om.apply_rope(om.rms_norm((h @ W[f"{p}.attention.to_k.weight"].T).reshape(3, 1, HD),
                                  W[f"{p}.attention.norm_k.weight"], 1e-5), cos, sin)
    v = (h @ W[f"{p}.attention.to_v.weight"].T).reshape(3, 1, HD)
    sd = torch.nn.functional.scaled_dot_product_attention(_t(q).permute(1, 0, 2), _t(k).permute(1, 0, 2),
                                                          _t(v).permute(1, 0, 2)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(om.attention(q, k, v), sd, rtol=1e-12, atol=1e-14)


def _mutant(func, old, new):
    """``func`` of oracle.model rebuilt from its source with ``old`` replaced
    by ``new`` (a mistake planted in the oracle, on the CPU only)."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(func))
    assert old in src, f"mutation site not found in {func.__name__}"
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), f"<mutant {func.__name__}>", "exec"), ns)
    return ns[func.__name__]


def test_modulated_block_by_hand_rejects_mutants(monkeypatch):
    """The block pin fails when the oracle itself is mutated: tanh(g) -> g
    on both gates, and RoPE moved in front of QK-RMSNorm."""
    def passes():
        try:
            test_modulated_block_by_hand()
        except AssertionError:
            return False
        return True

    assert passes()
    with monkeypatch.context() as mp:
        mp.setattr(om, "block_modulation",
                   _mutant(om.block_modulation, "np.tanh(g1), 1.0 + s2, np.tanh(g2)", "g1, 1.0 + s2, g2"))
        assert not passes()
    norm_first = (
        '    q = rms_norm(q.reshape(-1, H, hd), W[f"{prefix}.attention.norm_q.weight"], eps)\n'
        '    k = rms_norm(k.reshape(-1, H, hd), W[f"{prefix}.attention.norm_k.weight"], eps)\n'
        '    q = apply_rope(q, _f64(cos)[qrows], _f64(sin)[qrows])\n'
        '    k = apply_rope(k, cos, sin)\n')
    rope_first = (
        '    q = apply_rope(q.reshape(-1, H, hd), _f64(cos)[qrows], _f64(sin)[qrows])\n'
        '    k = apply_rope(k.reshape(-1, H, hd), cos, sin)\n'
        '    q = rms_norm(q, W[f"{prefix}.attention.norm_q.weight"], eps)\n'
        '    k = rms_norm(k, W[f"{prefix}.attention.norm_k.weight"], eps)\n')
    with monkeypatch.context() as mp:
        mp.setattr(om, "block", _mutant(om.block, norm_first, rope_first))
        assert not passes()


# ---------------------------------------------------------------- pad tokens

def test_padded_sequence_by_hand():
    """token_pad 32: an image run of 5 and a caption run of 3 tokens become
    32 + 32 rows; the added rows are copies of x_pad_token / cap_pad_token;
    caption positions run 1..32, real image tokens sit at (33, i, j), image
    pads at (0, 0, 0).  token_pad 0 leaves the runs and positions alone."""
    D = 8
    rng = np.random.default_rng(30)
    W = {"x_pad_token": rng.standard_normal((1, D)), "cap_pad_token": rng.standard_normal((1, D))}
    x_img, y = rng.standard_normal((5, D)), rng.standard_normal((3, D))
    cfg = ModelConfig(hidden=D, n_heads=1, token_pad=32)
    xi, yy, ids_cap, ids_img = om.padded_sequence(cfg, W, x_img, y, 1, 5)
    assert xi.shape == (32, D) and yy.shape == (32, D)
    assert np.array_equal(xi[:5], x_img) and np.array_equal(yy[:3], y)
    for r in range(5, 32):
        assert np.array_equal(xi[r], W["x_pad_token"][0])
    for r in range(3, 32):
        assert np.array_equal(yy[r], W["cap_pad_token"][0])
    assert ids_cap.tolist() == [[k + 1, 0, 0] for k in range(32)]
    assert ids_img.tolist() == [[33, 0, j] for j in range(5)] + [[0, 0, 0]] * 27
    cfg0 = ModelConfig(hidden=D, n_heads=1)
    xi0, yy0, c0, i0 = om.padded_sequence(cfg0, W, x_img, y, 1, 5)
    assert xi0 is x_img and yy0 is y
    assert c0.tolist() == [[1, 0, 0], [2, 0, 0], [3, 0, 0]] and i0.tolist() == [[4, 0, j] for j in range(5)]


def _tiny_forward(token_pad, lat_shape, L, W=None, seed=3):
    import synthetic
    from oracle import manifest
    cfg = ModelConfig(hidden=256, n_heads=2, ffn=384, n_layers=1, n_noise_refiner=1, n_context_refiner=1,
                      cap_feat_dim=64, t_mid=64, token_pad=token_pad)
    if W is None:
        W = synthetic.SyntheticWeights(manifest(cfg), seed=seed).materialize(workers=2)
    lat = synthetic.latent(lat_shape, seed=seed)
    caps = synthetic.captions((L,), dim=64, seed=seed)
    return om.forward(cfg, W, lat, caps, np.array([0.4])), W


def test_padding_is_a_no_op_on_whole_runs():
    """Runs that already hold a multiple of 32 tokens get no pad tokens:
    the padded forward is the plain one, bit for bit."""
    a, W = _tiny_forward(32, (1, 16, 8, 16), 32)    # 4 x 8 = 32 image tokens, 32 caption tokens
    b, _ = _tiny_forward(0, (1, 16, 8, 16), 32, W)
    assert np.array_equal(a, b)


def test_pad_tokens_take_part_in_attention():
    """With ragged runs the pad embeddings reach the real tokens' outputs
    (they are keys of the sample): changing either pad token changes the
    output, and the padded forward differs from the plain one."""
    a, W = _tiny_forward(32, (1, 16, 6, 10), 7)     # 15 image tokens -> 32, 7 caption tokens -> 32
    plain, _ = _tiny_forward(0, (1, 16, 6, 10), 7, W)
    assert not np.allclose(a, plain, rtol=1e-3)
    for key in ("x_pad_token", "cap_pad_token"):
        W2 = dict(W)
        W2[key] = W[key] + 0.5
        b, _ = _tiny_forward(32, (1, 16, 6, 10), 7, W2)
        assert np.all(np.isfinite(b)) and not np.allclose(a, b, rtol=1e-6), key
