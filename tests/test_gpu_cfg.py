"""Classifier-free guidance through the C ABI: the fused guided Euler update
against its float64 definition, and the guided sampling loop (a batch of
[latent; latent] with captions [cond; negative], guidance on the early
steps only) against the oracle's guided loop at reduced width."""

import numpy as np
import pytest

import synthetic
from oracle import model as om
from oracle import sampler as osm
from tests import helpers

pytestmark = pytest.mark.gpu

REDUCED = dict(hidden=512, n_heads=4, ffn=1536, n_layers=2, n_noise_refiner=1, n_context_refiner=1)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("n,offset", [(16 * 48 * 40, 0), (1001, 0), (4096, 1)])
@pytest.mark.parametrize("guidance", [0.0, 3.0, -0.5])
def test_cfg_euler_step_kernel(n, offset, guidance):
    """Vector path (n % 4 == 0, aligned) and scalar path (odd n, or a view
    one element in); g = 0 equals the plain Euler update bit for bit."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    rng = np.random.default_rng(n + offset)
    x0, c, u = (rng.standard_normal(n + offset).astype(np.float32) * s for s in (1.0, 2.0, 2.0))
    dt = -0.0625
    xd = torch.from_numpy(x0).cuda()
    cd = torch.from_numpy(c).cuda()
    ud = torch.from_numpy(u).cuda()
    binding.cfg_euler_step(xd[offset:], cd[offset:], ud[offset:], guidance, dt)
    torch.cuda.synchronize()
    got = xd.cpu().numpy()
    x64, c64, u64 = (a.astype(np.float64) for a in (x0, c, u))
    ref = x64 + dt * -(c64 + guidance * (c64 - u64))
    assert np.array_equal(got[:offset], x0[:offset])
    err = np.abs(got[offset:] - ref[offset:])
    scale = np.abs(x64) + abs(dt) * (np.abs(c64) + abs(guidance) * np.abs(c64 - u64))
    assert np.all(err <= 4.0 * 2.0 ** -24 * scale[offset:] + 1e-30)
    if guidance == 0.0:
        xe = torch.from_numpy(x0).cuda()
        binding.euler_step(xe[offset:], cd[offset:], dt)
        torch.cuda.synchronize()
        assert np.array_equal(xe.cpu().numpy(), got)


def test_cfg_euler_step_argument_errors():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    x = torch.zeros(64, device="cuda")
    o = torch.zeros(64, device="cuda")
    for g, dt in ((float("nan"), 0.1), (1.0, float("inf"))):
        with pytest.raises(binding.ZimgError) as ei:
            binding.cfg_euler_step(x, o, o, g, dt)
        assert ei.value.code == binding.ZIMG_EINVAL
    with pytest.raises(binding.ZimgError) as ei:
        binding.cfg_euler_step(x, x, o, 1.0, 0.1)
    assert ei.value.code == binding.ZIMG_EINVAL and "alias" in str(ei.value)


def test_cfg_loop_reduced_width_vs_oracle():
    torch = _torch()
    from diffusion_transformer_image_amd import binding, cfg_euler_loop
    shape, lc, lu = (1, 16, 48, 32), 77, 20
    n_steps, guidance, trunc = 6, 3.0, 0.3  # model times 0, .06, .14, .25 | .4, .625
    ecfg = helpers.engine_config(REDUCED, max_batch=2, max_image_tokens=24 * 16, max_caption_tokens=77)
    dit = binding.DiT(ecfg, helpers.engine_weights(ecfg, seed=2).items_parallel(as_bits=True))
    lat = synthetic.latent(shape, seed=8)
    cond, uncond = synthetic.captions((lc, lu), seed=8)
    x = torch.from_numpy(lat).cuda()
    guided = []
    cfg_euler_loop(dit, x, torch.from_numpy(cond).cuda(), [lc], torch.from_numpy(uncond).cuda(), [lu],
                   n_steps=n_steps, shift=3.0, guidance=guidance, cfg_truncation=trunc,
                   on_step=lambda k, xx, o: guided.append(o.shape[0] == 2))
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    dit.close()

    ocfg = helpers.oracle_config(REDUCED)
    Wo = helpers.oracle_weights(REDUCED, seed=2).materialize(workers=4)
    calls = []

    def model_fn(xx, tt, is_cond):
        calls.append(is_cond)
        return om.forward(ocfg, Wo, xx, [cond if is_cond else uncond], tt)

    ref = osm.run_cfg(model_fn, lat, n_steps=n_steps, shift=3.0, guidance=guidance, cfg_truncation=trunc)
    # the same steps were guided on both sides, and not all of them
    n_guided = calls.count(False)
    assert guided == [True] * n_guided + [False] * (n_steps - n_guided) and 0 < n_guided < n_steps
    r, c = helpers.assert_parity(got, ref, "latent after the guided loop")
    print(f"{n_guided} of {n_steps} steps guided; final latent rel-L2 {r:.2e} cos {c:.7f}")
