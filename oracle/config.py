"""Model hyperparameters of the S3-DiT, as the oracle sees them.

Test infrastructure only (see oracle/__init__.py).

Defaults are the full model of [AIT] "Architecture": hidden 3840 (30 heads of
128), SwiGLU FFN 10240, 30 joint blocks plus 2 noise-refiner and 2
context-refiner blocks, 3-axis RoPE [32, 48, 48] with theta 256, adaLN from a
256-d timestep embedding, 2560-d Qwen3-4B caption features ([AIT]
"Components"), 16-channel latent patchified 2x2 ([AIT] "Latent space").

Readings where the pages are silent (each is pinned only by the parameter
count of [AIT] "Components", or not at all):
  t_mid = 1024       hidden width of the timestep MLP (pinned by the count)
  t_scale = 1000     the model time t in [0, 1] is multiplied by 1000 before
                     the sinusoid ([AIT] "Specifics" divides the 0..1000
                     timestep by 1000; parity unpinned)
  max_period = 1e4   sinusoid period (parity unpinned)
  norm_eps = 1e-5    RMSNorm epsilon (parity unpinned)
  final_eps = 1e-6   final LayerNorm epsilon (parity unpinned)
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelConfig:
    hidden: int = 3840
    n_heads: int = 30
    ffn: int = 10240
    n_layers: int = 30
    n_noise_refiner: int = 2
    n_context_refiner: int = 2
    in_channels: int = 16
    patch: int = 2
    cap_feat_dim: int = 2560
    adaln_dim: int = 256
    t_mid: int = 1024
    rope_axes: tuple = (32, 48, 48)
    rope_theta: float = 256.0
    t_scale: float = 1000.0
    max_period: float = 10000.0
    norm_eps: float = 1e-5
    final_eps: float = 1e-6
    # 0: each sample's sequence holds exactly its caption and image tokens
    # ("padding dropped"); 32: each of the two runs is padded to a multiple
    # of 32 with the learned x_pad_token / cap_pad_token (see model.py)
    token_pad: int = 0

    @property
    def head_dim(self) -> int:
        return self.hidden // self.n_heads

    @property
    def patch_dim(self) -> int:
        return self.patch * self.patch * self.in_channels

    @classmethod
    def from_dict(cls, d: dict) -> "ModelConfig":
        kw = {k: v for k, v in d.items() if k in cls.__dataclass_fields__}
        if "rope_axes" in kw:
            kw["rope_axes"] = tuple(kw["rope_axes"])
        return cls(**kw)
