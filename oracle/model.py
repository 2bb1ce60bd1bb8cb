"""Plain float64 CPU oracle of the S3-DiT denoiser forward.

Test infrastructure only (see oracle/__init__.py).

One sample at a time: its image tokens and caption tokens form one sequence
[image; caption] ([AIT] "Architecture": text and image tokens share one
sequence; [GD] "Overview": tokens are concatenated into one sequence before
the transformer).  A batch is a loop over samples, so samples never interact.

Weights are read from any mapping ``W[name] -> array`` (names from
``oracle.manifest``); every array is converted to float64 on use.
"""

import math

import numpy as np

from .config import ModelConfig
from .manifest import block_prefixes
from . import quant as qz


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------

def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def rms_norm(x, w, eps):
    """RMSNorm over the last axis: w * x / sqrt(mean(x^2) + eps).

    [AIT] "Architecture" (RMSNorm, QK RMSNorm); [MNN] "Conversion details"
    relies on its scale invariance.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(w)


def layer_norm(x, eps):
    """LayerNorm over the last axis without affine parameters.

    Reading: the final layer normalises with a LayerNorm that has no weight
    or bias -- the 1.2M-parameter count of the final layer's two linears
    ([H3D] "What was changed, and why") leaves no room for one.
    """
    x = _f64(x)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


# ---------------------------------------------------------------------------
# timestep conditioning
# ---------------------------------------------------------------------------

def timestep_embedding(cfg: ModelConfig, t):
    """Sinusoidal embedding of the model time t (shape [B]) -> [B, adaln_dim].

    [AIT] "Architecture": adaLN modulation from a 256-d timestep embedding.
    [AIT] "Specifics" / [MNN] "Scheduler": the model takes t in [0, 1]
    (1 = clean).  Reading: tau = t_scale * t; frequencies
    f_i = exp(-ln(max_period) * i / half), i < half = dim/2; the embedding
    is [cos(tau f), sin(tau f)] (cosine half first).
    """
    t = _f64(t).reshape(-1)
    half = cfg.adaln_dim // 2
    i = np.arange(half, dtype=np.float64)
    freqs = np.exp(-math.log(cfg.max_period) * i / half)
    args = (cfg.t_scale * t)[:, None] * freqs[None, :]
    return np.concatenate([np.cos(args), np.sin(args)], axis=1)


def timestep_mlp(cfg: ModelConfig, W, t):
    """c = W2 SiLU(W1 e + b1) + b2 with e the sinusoid of t -> [B, adaln_dim]."""
    e = timestep_embedding(cfg, t)
    hmid = e @ _f64(W["t_embedder.mlp.0.weight"]).T + _f64(W["t_embedder.mlp.0.bias"])
    return silu(hmid) @ _f64(W["t_embedder.mlp.2.weight"]).T + _f64(W["t_embedder.mlp.2.bias"])


def block_modulation(W, prefix, c):
    """(scale_attn, gate_attn, scale_ffn, gate_ffn) for one sample's c [adaln_dim].

    [AIT] "Architecture": adaLN modulation from the timestep embedding.
    Readings: one linear (no SiLU in front) to 4*hidden, split in the order
    (s1, g1, s2, g2); no shift.  Scale is applied as (1 + s), gate as tanh(g).
    """
    m = _f64(W[f"{prefix}.adaLN_modulation.0.weight"]) @ _f64(c) + _f64(
        W[f"{prefix}.adaLN_modulation.0.bias"])
    s1, g1, s2, g2 = np.split(m, 4)
    return 1.0 + s1, np.tanh(g1), 1.0 + s2, np.tanh(g2)


# ---------------------------------------------------------------------------
# tokens and positions
# ---------------------------------------------------------------------------

def patchify(latent, patch=2):
    """[C, Hl, Wl] latent -> [(Hl/p)*(Wl/p), p*p*C] tokens.

    [AIT] "Latent space": the transformer patchifies 2x2 internally, one
    token per 16x16 pixels.  Reading: token n = i*(Wl/p) + j; feature
    (a*p + b)*C + ch holds latent[ch, p*i + a, p*j + b] (channel fastest).
    """
    lat = _f64(latent)
    C, Hl, Wl = lat.shape
    Hp, Wp = Hl // patch, Wl // patch
    x = lat.reshape(C, Hp, patch, Wp, patch)          # ch, i, a, j, b
    x = x.transpose(1, 3, 2, 4, 0)                     # i, j, a, b, ch
    return x.reshape(Hp * Wp, patch * patch * C)


def unpatchify(tokens, C, Hl, Wl, patch=2):
    """Inverse of ``patchify``: [(Hl/p)*(Wl/p), p*p*C] -> [C, Hl, Wl]."""
    Hp, Wp = Hl // patch, Wl // patch
    x = _f64(tokens).reshape(Hp, Wp, patch, patch, C)   # i, j, a, b, ch
    x = x.transpose(4, 0, 2, 1, 3)                      # ch, i, a, j, b
    return x.reshape(C, Hl, Wl)


def position_ids(n_caption, Hp, Wp):
    """3-axis integer positions: caption [L, 3] and image [Hp*Wp, 3].

    [AIT] "Architecture": 3-axis RoPE over one shared sequence.  Reading:
    caption token k -> (k + 1, 0, 0); image token (i, j) -> (L + 1, i, j),
    so the caption runs along axis 0 and the image sits one step after it,
    spread over axes 1 and 2.
    """
    cap = np.zeros((n_caption, 3), dtype=np.int32)
    cap[:, 0] = np.arange(1, n_caption + 1, dtype=np.int32)
    ii, jj = np.meshgrid(np.arange(Hp), np.arange(Wp), indexing="ij")
    img = np.zeros((Hp * Wp, 3), dtype=np.int32)
    img[:, 0] = n_caption + 1
    img[:, 1] = ii.reshape(-1)
    img[:, 2] = jj.reshape(-1)
    return cap, img


def rope_frequencies(cfg: ModelConfig):
    """(axis, omega) for each of the head_dim/2 rotation pairs.

    [AIT] "Architecture": 3-axis RoPE [32, 48, 48], theta 256.  Axis a owns
    d_a consecutive channels; its pair r (r < d_a/2) turns at
    omega = theta ** (-(2 r) / d_a), computed in float64.
    """
    out = []
    for axis, d in enumerate(cfg.rope_axes):
        for r in range(d // 2):
            out.append((axis, float(cfg.rope_theta) ** (-(2.0 * r) / d)))
    return out


def rope_tables(cfg: ModelConfig, ids):
    """cos and sin tables [S, head_dim/2] as float32 for position ids [S, 3].

    The angle of pair p at a row is pos[axis_p] * omega_p in float64; its
    cosine and sine are taken in float64 (C libm through Python's math
    module) and rounded to nearest float32.
    """
    ids = np.asarray(ids)
    freqs = rope_frequencies(cfg)
    S, P = ids.shape[0], len(freqs)
    cos = np.empty((S, P), dtype=np.float32)
    sin = np.empty((S, P), dtype=np.float32)
    for s in range(S):
        pos = [float(ids[s, 0]), float(ids[s, 1]), float(ids[s, 2])]
        for p, (axis, omega) in enumerate(freqs):
            phi = pos[axis] * omega
            cos[s, p] = math.cos(phi)
            sin[s, p] = math.sin(phi)
    return cos, sin


def apply_rope(x, cos, sin):
    """Rotate interleaved channel pairs (2p, 2p+1) of x [S, H, hd] by the
    per-row table angle of pair p: (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).

    Reading: pairs are adjacent channels inside each axis section, sections
    in axis order ([AIT] "Architecture" gives only the axis split).
    """
    x = _f64(x)
    c = _f64(cos)[:, None, :]
    s = _f64(sin)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ---------------------------------------------------------------------------
# attention and the block
# ---------------------------------------------------------------------------

def attention(q, k, v, q_chunk=2048):
    """Full bidirectional softmax attention per head.

    q [Sq, H, hd], k and v [Sk, H, hd] -> [Sq, H, hd];
    o = softmax(q k^T / sqrt(hd)) v, no mask ([MNN] "Performance":
    non-causal attention; [FV] "Transformer": torch SDPA, whose default scale
    is 1/sqrt(hd)).  Query rows are processed ``q_chunk`` at a time to bound
    memory; that changes no row's arithmetic.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Sq, H, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    out = np.empty((Sq, H, v.shape[2]), dtype=np.float64)
    for h in range(H):
        kh, vh = k[:, h, :], v[:, h, :]
        for r0 in range(0, Sq, q_chunk):
            s = (q[r0:r0 + q_chunk, h, :] @ kh.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[r0:r0 + q_chunk, h, :] = p @ vh
    return out


def linear(x, w, quant=None, held="f32", rotate=False):
    """x W^T without bias.  quant None: float64.  quant "int8": the W8A8
    product of oracle.quant, with x quantized from the precision it is held
    in when it reaches the projection (``held``: "f32" or "bf16"), rotated
    first when ``rotate`` (w2's input)."""
    if quant is None:
        return _f64(x) @ _f64(w).T
    if quant != "int8":
        raise ValueError(f"unknown quantization {quant!r}")
    xh = qz.to_bf16(x) if held == "bf16" else qz.to_f32(x)
    return qz.int8_linear(xh, w, rotate=rotate)


def swiglu_ffn(W, prefix, h, quant=None):
    """w2( SiLU(w1 h) * (w3 h) ), no biases ([AIT] "Architecture": SwiGLU
    FFN; [MNN] "Conversion details": weights w1, w2, w3).  With int8
    projections, the SwiGLU product reaches w2 as bf16 values and is rotated
    before it is quantized (oracle.quant)."""
    a = linear(h, W[f"{prefix}.feed_forward.w1.weight"], quant)
    b = linear(h, W[f"{prefix}.feed_forward.w3.weight"], quant)
    return linear(silu(a) * b, W[f"{prefix}.feed_forward.w2.weight"], quant, held="bf16", rotate=True)


def block(cfg: ModelConfig, W, prefix, x, cos, sin, mod=None, rows=None, taps=None, quant=None):
    """One S3-DiT transformer block over a single sample's sequence x [S, D].

    Sandwich-norm block ([AIT] "Architecture"; [MNN] "Conversion details":
    the to_out and w2 outputs feed directly into an RMSNorm):
      h  = RMSNorm(x; attention_norm1) * (1 + s1)
      q, k, v = h Wq^T, h Wk^T, h Wv^T               (heads of 128)
      q, k = RoPE(RMSNorm_hd(q; norm_q)), RoPE(RMSNorm_hd(k; norm_k))
      o  = softmax(q k^T / sqrt(hd)) v
      x  = x + tanh(g1) * RMSNorm(o Wout^T; attention_norm2)
      h2 = RMSNorm(x; ffn_norm1) * (1 + s2)
      x  = x + tanh(g2) * RMSNorm(w2(SiLU(w1 h2) * w3 h2); ffn_norm2)
    ``mod`` is the tuple from ``block_modulation``; None means unmodulated
    (context refiner, [AIT] "Architecture"): scales 1 and gates 1.
    ``rows`` restricts the output (and the queries) to those rows; keys and
    values still come from every row.  ``taps`` (a dict), if given, receives
    the w2 output under "ffn_out" (observation only).  ``quant`` "int8"
    runs the seven projections as oracle.quant defines (the attention output
    reaches to_out as bf16 values).
    """
    D, H, hd, eps = cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.norm_eps
    x = _f64(x)
    if mod is None:
        scale_a = gate_a = scale_f = gate_f = 1.0
    else:
        scale_a, gate_a, scale_f, gate_f = mod
    qrows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)

    h = rms_norm(x, W[f"{prefix}.attention_norm1.weight"], eps) * scale_a
    q = linear(h[qrows], W[f"{prefix}.attention.to_q.weight"], quant)
    k = linear(h, W[f"{prefix}.attention.to_k.weight"], quant)
    v = linear(h, W[f"{prefix}.attention.to_v.weight"], quant)
    q = rms_norm(q.reshape(-1, H, hd), W[f"{prefix}.attention.norm_q.weight"], eps)
    k = rms_norm(k.reshape(-1, H, hd), W[f"{prefix}.attention.norm_k.weight"], eps)
    q = apply_rope(q, _f64(cos)[qrows], _f64(sin)[qrows])
    k = apply_rope(k, cos, sin)
    o = attention(q, k, v.reshape(-1, H, hd)).reshape(-1, D)
    a = linear(o, W[f"{prefix}.attention.to_out.0.weight"], quant, held="bf16")
    x1 = x[qrows] + gate_a * rms_norm(a, W[f"{prefix}.attention_norm2.weight"], eps)

    h2 = rms_norm(x1, W[f"{prefix}.ffn_norm1.weight"], eps) * scale_f
    f = swiglu_ffn(W, prefix, h2, quant)
    if taps is not None:
        taps["ffn_out"] = f
    return x1 + gate_f * rms_norm(f, W[f"{prefix}.ffn_norm2.weight"], eps)


# ---------------------------------------------------------------------------
# embedders, final layer, whole forward
# ---------------------------------------------------------------------------

def x_embed(cfg: ModelConfig, W, latent):
    """Patch embed: patchify 2x2 then linear patch_dim -> hidden with bias."""
    v = patchify(latent, cfg.patch)
    return v @ _f64(W["all_x_embedder.2-1.weight"]).T + _f64(W["all_x_embedder.2-1.bias"])


def cap_embed(cfg: ModelConfig, W, feats):
    """Caption embed: RMSNorm over the 2560-d features, then linear -> hidden
    ([AIT] "Architecture": 2560-d Qwen3-4B hidden states; "Components")."""
    y = rms_norm(feats, W["cap_embedder.0.weight"], cfg.norm_eps)
    return y @ _f64(W["cap_embedder.1.weight"]).T + _f64(W["cap_embedder.1.bias"])


def final_layer(cfg: ModelConfig, W, x_img, c):
    """z = LayerNorm(x) * (1 + scale), scale = W SiLU(c) + b; out = z Wf^T + bf.

    [H3D] "What was changed, and why": the final layer is two small linears,
    final_layer.linear is [64, 3840].  Reading: SiLU in front of its
    modulation linear, a scale only, and LayerNorm without affine.
    """
    scale = _f64(W["all_final_layer.2-1.adaLN_modulation.1.weight"]) @ silu(c) + _f64(
        W["all_final_layer.2-1.adaLN_modulation.1.bias"])
    z = layer_norm(x_img, cfg.final_eps) * (1.0 + scale)
    return z @ _f64(W["all_final_layer.2-1.linear.weight"]).T + _f64(W["all_final_layer.2-1.linear.bias"])


def padded_sequence(cfg: ModelConfig, W, x_img, y, Hp, Wp):
    """The sample's image and caption runs as the blocks see them, with
    their 3-axis position ids: (x_img, y, ids_cap, ids_img).

    cfg.token_pad = 0: the embedded tokens as they are ([AIT]
    "Architecture": padding dropped), positions from ``position_ids``.
    cfg.token_pad = p (32): the released model's padding ([H3D] "Measured
    performance versus the regular layout": a 4,128 = 4,096 + 32 token
    forward; [AIT] "Components": the parameter total includes the two
    3840-d pad embeddings; [FV] "Component contracts", Transformer: the
    padded variable-length stream needs a key mask).  Reading, parity
    unpinned beyond that: each run is padded to a multiple of p, the image
    run with copies of x_pad_token and the caption run with copies of
    cap_pad_token; pad tokens are ordinary members of their sample's
    sequence (queries and keys; only other samples are masked); the caption
    positions continue through its pads (k + 1 for k < L_p), the image
    positions start after the padded caption ((L_p + 1, i, j)), and image
    pad tokens sit at position (0, 0, 0).
    """
    N, L = x_img.shape[0], y.shape[0]
    p = cfg.token_pad
    if not p:
        ids_cap, ids_img = position_ids(L, Hp, Wp)
        return x_img, y, ids_cap, ids_img
    Np, Lp = -(-N // p) * p, -(-L // p) * p
    x_img = np.concatenate([x_img, np.repeat(_f64(W["x_pad_token"]).reshape(1, -1), Np - N, axis=0)])
    y = np.concatenate([y, np.repeat(_f64(W["cap_pad_token"]).reshape(1, -1), Lp - L, axis=0)])
    ids_cap, ids_img = position_ids(Lp, Hp, Wp)
    ids_img = np.concatenate([ids_img, np.zeros((Np - N, 3), dtype=np.int32)])
    return x_img, y, ids_cap, ids_img


def forward_sample(cfg: ModelConfig, W, latent, feats, t, capture=None, ffn_peak=None, quant=None):
    """Forward of one sample: latent [C, Hl, Wl], caption features [L, 2560],
    scalar model time t -> raw model output [C, Hl, Wl].

    Order ([AIT] "Architecture"): noise refiner over the image tokens,
    context refiner (unmodulated) over the caption tokens, then the joint
    blocks over [image; caption], then the final layer on the image tokens.
    ``capture`` (a dict) receives the residual after each stage; ``ffn_peak``
    (a list) receives max |w2 output| of each block (observation only).
    ``quant`` selects the block projections' arithmetic (see ``block``);
    embedders, conditioning and the final layer stay in float64.
    """
    C, Hl, Wl = np.shape(latent)
    Hp, Wp = Hl // cfg.patch, Wl // cfg.patch
    L = np.shape(feats)[0]
    c = timestep_mlp(cfg, W, np.array([t]))[0]

    x_img = x_embed(cfg, W, latent)
    y = cap_embed(cfg, W, feats)
    x_img, y, ids_cap, ids_img = padded_sequence(cfg, W, x_img, y, Hp, Wp)
    if capture is not None:
        capture["x_embed"] = x_img.copy()
        capture["cap_embed"] = y.copy()

    cos_img, sin_img = rope_tables(cfg, ids_img)
    cos_cap, sin_cap = rope_tables(cfg, ids_cap)
    cos_all = np.concatenate([cos_img, cos_cap])
    sin_all = np.concatenate([sin_img, sin_cap])

    x = None
    for prefix, modulated in block_prefixes(cfg):
        mod = block_modulation(W, prefix, c) if modulated else None
        taps = {} if ffn_peak is not None else None
        if prefix.startswith("noise_refiner"):
            x_img = block(cfg, W, prefix, x_img, cos_img, sin_img, mod, taps=taps, quant=quant)
            out = x_img
        elif prefix.startswith("context_refiner"):
            y = block(cfg, W, prefix, y, cos_cap, sin_cap, None, taps=taps, quant=quant)
            out = y
        else:
            if x is None:
                x = np.concatenate([x_img, y])
            x = block(cfg, W, prefix, x, cos_all, sin_all, mod, taps=taps, quant=quant)
            out = x
        if ffn_peak is not None:
            ffn_peak.append(float(np.max(np.abs(taps["ffn_out"]))))
        if capture is not None:
            capture[prefix] = out.copy()
    if x is None:
        x = np.concatenate([x_img, y])

    o = final_layer(cfg, W, x[: Hp * Wp], c)
    if capture is not None:
        capture["final"] = o.copy()
    return unpatchify(o, C, Hl, Wl, cfg.patch)


def forward(cfg: ModelConfig, W, latent, caption_feats, t, captures=None, ffn_peak=None, quant=None):
    """Batched forward: latent [B, C, Hl, Wl], caption_feats a list of B
    arrays [L_b, 2560] (exact lengths, no padding: [AIT] "Architecture",
    "padding dropped"), t [B] -> [B, C, Hl, Wl].  Samples are independent.
    ``captures`` (a list of B dicts) receives per-stage residuals.
    """
    latent = _f64(latent)
    t = _f64(t).reshape(-1)
    outs = []
    for b in range(latent.shape[0]):
        cap = captures[b] if captures is not None else None
        outs.append(forward_sample(cfg, W, latent[b], caption_feats[b], t[b], cap, ffn_peak, quant))
    return np.stack(outs)
