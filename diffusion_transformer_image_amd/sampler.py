"""FlowMatch Euler sampling loop around the engine's forward.

Schedule ("Z-Image-Turbo MNN (int8, fp16-safe)", Scheduler; "Z-Image" (AI
Toolkit docs), Specifics; "Local component coverage and quality handoff for
the zimage FastVideo port", Pinned official pipeline context): base sigmas
linspace(1, 1/N, N), shifted sigma' = s sigma / (1 + (s - 1) sigma), a final
sigma' = 0 appended (no model call there); model time t = (1000 - 1000
sigma')/1000; each step x += (sigma'_{k+1} - sigma'_k) * (-model_out).  The
schedule is computed on the host in float64; the update runs on the GPU.
"""

import numpy as np

from . import binding


def schedule(n_steps, shift):
    """(shifted sigmas [N+1] ending at 0, model times [N]) in float64."""
    base = np.linspace(1.0, 1.0 / n_steps, n_steps, dtype=np.float64)
    shifted = shift * base / (1.0 + (shift - 1.0) * base)
    sig = np.append(shifted, 0.0)
    t = (1000.0 - 1000.0 * shifted) / 1000.0
    return sig, t


def euler_loop(dit, latent, caption_feats, caption_lens, n_steps=8, shift=3.0, out=None, on_step=None,
               stream=None):
    """Run the N-step loop in place on ``latent`` (torch CUDA fp32 [B, C, Hl, Wl]).

    ``out`` is a scratch tensor of the latent's shape for the model output.
    Returns ``latent``.
    """
    import torch
    sig, t = schedule(n_steps, shift)
    B = latent.shape[0]
    if out is None:
        out = torch.empty_like(latent)
    for k in range(n_steps):
        tk = np.full(B, t[k], dtype=np.float32)
        dit.forward(latent, caption_feats, caption_lens, tk, out, stream=stream)
        if on_step is not None:
            on_step(k, latent, out)
        binding.euler_step(latent, out, float(sig[k + 1] - sig[k]), stream=stream)
    return latent
