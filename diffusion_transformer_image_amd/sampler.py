"""FlowMatch Euler sampling loop around the engine's forward.

Schedule ("Z-Image-Turbo MNN (int8, fp16-safe)", Scheduler; "Z-Image" (AI
Toolkit docs), Specifics; "Local component coverage and quality handoff for
the zimage FastVideo port", Pinned official pipeline context): base sigmas
linspace(1, 1/N, N), shifted sigma' = s sigma / (1 + (s - 1) sigma), a final
sigma' = 0 appended (no model call there); model time t = (1000 - 1000
sigma')/1000; each step x += (sigma'_{k+1} - sigma'_k) * (-model_out).  The
schedule comes from the library (zimg_flowmatch_schedule, host float64); the
update runs on the GPU.
"""

import numpy as np

from . import binding


def schedule(n_steps, shift):
    """(shifted sigmas [N+1] ending at 0, model times [N]) in float64."""
    return binding.flowmatch_schedule(n_steps, shift)


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


def guidance_active(t, cfg_truncation):
    """Guidance is applied at model times t <= cfg_truncation (compared in
    float32); the default 1.0 applies it on every step."""
    return bool(np.float32(t) <= np.float32(cfg_truncation))


def cfg_euler_loop(dit, latent, caps_cond, lens_cond, caps_uncond, lens_uncond, n_steps=28, shift=3.0,
                   guidance=3.0, cfg_truncation=1.0, on_step=None):
    """Euler loop with classifier-free guidance, in place on ``latent``
    (torch CUDA fp32 [B, C, Hl, Wl]).  Each guided step runs one forward of
    the batch [latent; latent] with captions [cond; uncond] (``caps_*``:
    packed CUDA rows, ``lens_*``: B lengths each) and one fused update
    (zimg_cfg_euler_step); a step without guidance (guidance 0 or model time
    past ``cfg_truncation``) runs the conditional half alone.  The engine
    needs max_batch >= 2 B.  ``guidance`` is the pipeline's scale (the
    user-facing scale minus one).  Everything runs on torch's current
    stream.  Returns ``latent``."""
    import torch
    sig, t = schedule(n_steps, shift)
    B = latent.shape[0]
    pair = torch.empty((2 * B,) + tuple(latent.shape[1:]), dtype=latent.dtype, device=latent.device)
    out = torch.empty_like(pair)
    caps_pair = torch.cat([caps_cond, caps_uncond])
    lens_pair = list(lens_cond) + list(lens_uncond)
    for k in range(n_steps):
        dt = float(sig[k + 1] - sig[k])
        if guidance != 0.0 and guidance_active(t[k], cfg_truncation):
            pair[:B].copy_(latent)
            pair[B:].copy_(latent)
            dit.forward(pair, caps_pair, lens_pair, np.full(2 * B, t[k], dtype=np.float32), out)
            if on_step is not None:
                on_step(k, latent, out)
            binding.cfg_euler_step(latent, out[:B], out[B:], guidance, dt)
        else:
            dit.forward(latent, caps_cond, list(lens_cond), np.full(B, t[k], dtype=np.float32), out[:B])
            if on_step is not None:
                on_step(k, latent, out[:B])
            binding.euler_step(latent, out[:B], dt)
    return latent
