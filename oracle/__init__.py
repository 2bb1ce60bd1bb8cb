"""Plain, slow, obviously-correct CPU oracle of the Z-Image S3-DiT denoiser
forward and of the FlowMatch Euler sampler around it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP engine (``diffusion_transformer_image_amd``) and never imports it.

Every function computes in float64 (numpy), step by step, in the order the
pages give, with no blocking, fusion or reordering beyond what the definition
states.  Each function names the passage it follows.  Where the pages leave a
step open, the reading taken is stated in the docstring.

Pages cited (by title and section):
  [AIT]  "Z-Image" -- ostris AI Toolkit model documentation
         (sections: Components, Latent space, Architecture, Specifics).
  [MNN]  "Z-Image-Turbo MNN (int8, fp16-safe)" model card
         (sections: Model files, Conversion details, Performance, Scheduler).
  [H3D]  "Z-Image-Turbo, repackaged for H3ddle" model card
         (sections: Measured performance..., What was changed, and why).
  [FV]   "Local component coverage and quality handoff for the zimage
         FastVideo port" (sections: Reference assets and scope, Pinned
         official pipeline context, Component contracts).
  [GD]   "tongyi-mai/z-image architecture" (GitDiagram overview).

Parity status per function (what pins it; see tests/test_oracle_*.py):
  manifest                 pinned: param total, key count, final-layer size
  rms_norm / layer_norm    pinned: invariances, torch library routines
  rope tables / apply_rope pinned: closed-form entries, norm, relativity
  attention                pinned: brute-force loops, torch SDPA
  swiglu ffn               pinned: exact 1/64 compensation, hand formula
  block wiring             pinned: zero-gate identity, unmodulated reduction,
                           one modulated block written out by hand (non-zero
                           tanh gates, QK-RMSNorm before RoPE), with planted
                           mutants that the pin rejects
  timestep MLP             pinned: by-hand loops and torch Linear/SiLU
  caption embedder         pinned: by-hand loops and torch rms_norm/linear
  patchify / unpatchify    pinned: brute-force index loops, token counts
  sampler schedule         pinned: exact rational values of the closed form
  timestep embedding       pinned: closed-form entries (constants themselves
                           are a reading: parity unpinned vs the released
                           model, as are SiLU placement and position-id
                           offsets -- no released weights or activations
                           exist to compare against)
"""

from .config import ModelConfig
from .manifest import manifest, param_count
from . import model, sampler

__all__ = ["ModelConfig", "manifest", "param_count", "model", "sampler"]
