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
