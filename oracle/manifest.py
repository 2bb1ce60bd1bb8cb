"""Named weight tensors of the S3-DiT and their shapes.

Test infrastructure only (see oracle/__init__.py).

Module names follow the ones the pages print: ``t_embedder``,
``cap_embedder``, ``all_x_embedder`` and ``all_final_layer`` ([AIT]
"Specifics", quantization note; the patch-size key ``2-1`` of both),
``final_layer.linear`` at [64, 3840] ([H3D] "What was changed, and why"),
``to_out`` and the FFN's ``w1/w2/w3`` ([MNN] "Conversion details").  The
whole key set is pinned: its sorted-key SHA-256 equals the digest [FV]
"Component contracts" (Transformer) prints for the released checkpoint's
safetensors index, which also fixes the module order inside the small
sequentials -- ``t_embedder.mlp.0`` / ``.2`` (an activation at index 1),
``cap_embedder.0`` (the RMSNorm) before ``.1`` (the linear), a block's
``adaLN_modulation.0`` (the linear first: no activation in front of it) and
the final layer's ``adaLN_modulation.1`` (an activation at index 0).

Block structure (the reading that reproduces the printed counts):
  * separate q, k, v, out projections without bias, QK-RMSNorm weights of
    head_dim ([AIT] "Architecture": "QK RMSNorm");
  * SwiGLU w1, w2, w3 without bias ([AIT] "Architecture");
  * four RMSNorm weights: pre/post around attention and around the FFN
    ([MNN] "Conversion details": to_out and w2 outputs feed an RMSNorm);
  * adaLN: one linear adaln_dim -> 4*hidden with bias (scale and gate for
    attention and FFN; no shift) -- modulated blocks only; the context
    refiner is unmodulated ([AIT] "Architecture").
Global tensors: timestep MLP 256 -> t_mid -> 256, caption RMSNorm + linear
2560 -> hidden, patch linear 64 -> hidden, final layer (SiLU + linear
adaln_dim -> hidden for the scale; linear hidden -> 64), two pad tokens.

With the full configuration this gives 521 tensors ([FV] "Reference assets and
scope": "the same 521 checkpoint keys/shapes") holding 6,154,908,736
parameters ([AIT] "Components": transformer 6,154,908,736), and a final layer
of 1,232,704 parameters ([H3D]: "1.2M of 6.15B parameters").
"""

from .config import ModelConfig


BLOCK_GROUPS = (
    # (prefix, count attribute, modulated)
    ("noise_refiner", "n_noise_refiner", True),
    ("context_refiner", "n_context_refiner", False),
    ("layers", "n_layers", True),
)


def block_keys(cfg: ModelConfig, prefix: str, modulated: bool):
    D, F, hd = cfg.hidden, cfg.ffn, cfg.head_dim
    keys = [
        (f"{prefix}.attention.to_q.weight", (D, D)),
        (f"{prefix}.attention.to_k.weight", (D, D)),
        (f"{prefix}.attention.to_v.weight", (D, D)),
        (f"{prefix}.attention.to_out.0.weight", (D, D)),
        (f"{prefix}.attention.norm_q.weight", (hd,)),
        (f"{prefix}.attention.norm_k.weight", (hd,)),
        (f"{prefix}.feed_forward.w1.weight", (F, D)),
        (f"{prefix}.feed_forward.w2.weight", (D, F)),
        (f"{prefix}.feed_forward.w3.weight", (F, D)),
        (f"{prefix}.attention_norm1.weight", (D,)),
        (f"{prefix}.attention_norm2.weight", (D,)),
        (f"{prefix}.ffn_norm1.weight", (D,)),
        (f"{prefix}.ffn_norm2.weight", (D,)),
    ]
    if modulated:
        keys += [
            (f"{prefix}.adaLN_modulation.0.weight", (4 * D, cfg.adaln_dim)),
            (f"{prefix}.adaLN_modulation.0.bias", (4 * D,)),
        ]
    return keys


def block_prefixes(cfg: ModelConfig):
    """(prefix, modulated) for every block, in execution order."""
    out = []
    for name, attr, modulated in BLOCK_GROUPS:
        for i in range(getattr(cfg, attr)):
            out.append((f"{name}.{i}", modulated))
    return out


def manifest(cfg: ModelConfig):
    """List of (name, shape) for every weight tensor, in canonical order."""
    D = cfg.hidden
    keys = [
        ("t_embedder.mlp.0.weight", (cfg.t_mid, cfg.adaln_dim)),
        ("t_embedder.mlp.0.bias", (cfg.t_mid,)),
        ("t_embedder.mlp.2.weight", (cfg.adaln_dim, cfg.t_mid)),
        ("t_embedder.mlp.2.bias", (cfg.adaln_dim,)),
        ("cap_embedder.0.weight", (cfg.cap_feat_dim,)),
        ("cap_embedder.1.weight", (D, cfg.cap_feat_dim)),
        ("cap_embedder.1.bias", (D,)),
        ("all_x_embedder.2-1.weight", (D, cfg.patch_dim)),
        ("all_x_embedder.2-1.bias", (D,)),
        ("all_final_layer.2-1.adaLN_modulation.1.weight", (D, cfg.adaln_dim)),
        ("all_final_layer.2-1.adaLN_modulation.1.bias", (D,)),
        ("all_final_layer.2-1.linear.weight", (cfg.patch_dim, D)),
        ("all_final_layer.2-1.linear.bias", (cfg.patch_dim,)),
        ("x_pad_token", (1, D)),
        ("cap_pad_token", (1, D)),
    ]
    for prefix, modulated in block_prefixes(cfg):
        keys += block_keys(cfg, prefix, modulated)
    return keys


def param_count(cfg: ModelConfig) -> int:
    total = 0
    for _, shape in manifest(cfg):
        n = 1
        for s in shape:
            n *= s
        total += n
    return total
