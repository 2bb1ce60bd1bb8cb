"""FlowMatch Euler sampler around the DiT forward, in float64.

Test infrastructure only (see oracle/__init__.py).

[MNN] "Scheduler": FlowMatch Euler with shift s = 3.0; sigmas are
linspace(1, 1/N, N), shifted by sigma' = s*sigma / (1 + (s-1)*sigma); the
model is given t = (1000 - 1000*sigma') / 1000; its output is negated before
the Euler step.  [AIT] "Specifics": t = (1000 - timestep)/1000, 1 = clean;
the output is negated to match the noise - latents flow target; the fixed
shift is 3.0.  [FV] "Pinned official pipeline context" / "Scheduler": the
schedule has num_steps + 1 points ending at sigma = 0, and no DiT call is
made at that final zero point.

Classifier-free guidance: [FV] "Pinned official pipeline context" lists a
negative prompt, ``guidance_scale`` (default 0.0) and ``cfg_truncation``
(default 1.0); [AIT] "Specifics" says the UI's guidance scale reaches the
pipeline reduced by one; the base model runs 28-50 steps at CFG 3-5 ([AIT],
the model summary above "Components").
"""

import numpy as np


def base_sigmas(n_steps):
    """linspace(1, 1/N, N) in float64."""
    return np.linspace(1.0, 1.0 / n_steps, n_steps, dtype=np.float64)


def shift_sigma(sigma, shift):
    """sigma' = shift*sigma / (1 + (shift - 1)*sigma)."""
    sigma = np.asarray(sigma, dtype=np.float64)
    return shift * sigma / (1.0 + (shift - 1.0) * sigma)


def model_time(sigma_shifted):
    """t = (1000 - 1000*sigma') / 1000 (1 = clean)."""
    s = np.asarray(sigma_shifted, dtype=np.float64)
    return (1000.0 - 1000.0 * s) / 1000.0


def schedule(n_steps, shift):
    """(sigma' with the final 0 appended [N+1], t for the N model calls [N])."""
    sp = shift_sigma(base_sigmas(n_steps), shift)
    return np.concatenate([sp, [0.0]]), model_time(sp)


def euler_step(x, model_out, sigma_now, sigma_next):
    """x + (sigma_next - sigma_now) * (-model_out)."""
    return np.asarray(x, np.float64) + (sigma_next - sigma_now) * (-np.asarray(model_out, np.float64))


def run(model_fn, latent0, n_steps=8, shift=3.0, on_step=None):
    """Euler loop: for k < N, out_k = model_fn(x_k, t_k) and
    x_{k+1} = x_k + (sigma'_{k+1} - sigma'_k) * (-out_k).

    ``model_fn(x, t_vector)`` is the oracle forward with the caption fixed;
    t is cast to float32 before the call (the model time is a float32
    input).  Returns the final latent.
    """
    sig, t = schedule(n_steps, shift)
    x = np.asarray(latent0, dtype=np.float64)
    B = x.shape[0]
    for k in range(n_steps):
        tk = np.full(B, np.float32(t[k]), dtype=np.float64)
        out = model_fn(x, tk)
        x = euler_step(x, out, sig[k], sig[k + 1])
        if on_step is not None:
            on_step(k, x, out)
    return x


def guided_output(out_cond, out_uncond, guidance):
    """Classifier-free guidance as the pipeline receives it.  The pipeline's
    guidance scale g is the user-facing scale minus one ([AIT] "Specifics":
    a UI scale of 4 reaches the pipeline as 3), so the guided prediction is
    the conditional output pushed away from the unconditional one by g times
    their difference; g = 0 (the Turbo default, [FV] "Pinned official
    pipeline context" / "Official defaults") is the conditional output."""
    c = np.asarray(out_cond, np.float64)
    u = np.asarray(out_uncond, np.float64)
    return c + guidance * (c - u)


def guidance_active(t, cfg_truncation):
    """Reading of ``cfg_truncation`` (the pages give only its default, 1.0):
    guidance is applied at steps whose model time t (0 = noise, 1 = clean)
    is at most cfg_truncation, so 1.0 keeps it on every step and smaller
    values switch it off for the last, nearly clean steps.  Both values are
    compared as float32, as the engine's sampler does."""
    return bool(np.float32(t) <= np.float32(cfg_truncation))


def run_cfg(model_fn, latent0, n_steps=28, shift=3.0, guidance=3.0, cfg_truncation=1.0, on_step=None):
    """Euler loop with classifier-free guidance.  ``model_fn(x, t_vector,
    cond)`` is the oracle forward with the conditional (cond=True) or the
    unconditional (negative) caption.  A step where guidance is off (g = 0 or
    truncated) calls only the conditional forward."""
    sig, t = schedule(n_steps, shift)
    x = np.asarray(latent0, dtype=np.float64)
    B = x.shape[0]
    for k in range(n_steps):
        tk = np.full(B, np.float32(t[k]), dtype=np.float64)
        out = model_fn(x, tk, True)
        if guidance != 0.0 and guidance_active(t[k], cfg_truncation):
            out = guided_output(out, model_fn(x, tk, False), guidance)
        x = euler_step(x, out, sig[k], sig[k + 1])
        if on_step is not None:
            on_step(k, x, out)
    return x
