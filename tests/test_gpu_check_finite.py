"""The check_finite debug option through the C ABI: a clean forward gives
bitwise the output of the engine without it, and a NaN or infinity planted
in the latent, a caption, or one block's weights is reported as
ZIMG_ENONFINITE naming the first stage where it appeared (the embeddings,
that block).  NaN arithmetic only: no kernel branches on the planted values
in a way that changes its control flow or memory accesses."""

import numpy as np
import pytest

import synthetic
from tests import helpers

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=512, n_heads=4, ffn=1536, n_layers=2, n_noise_refiner=1, n_context_refiner=1)
SHAPE, LENS, T = (2, 16, 16, 24), (40, 17), (0.3, 0.7)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _engine(check, weights=None):
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(SMALL, max_batch=2, max_image_tokens=96, max_caption_tokens=64,
                                 check_finite=check)
    if weights is None:
        weights = helpers.engine_weights(ecfg, seed=3).items_parallel(as_bits=True)
    return binding.DiT(ecfg, weights)


def _inputs():
    torch = _torch()
    lat = torch.from_numpy(synthetic.latent(SHAPE, seed=3)).cuda()
    caps = torch.from_numpy(np.concatenate(synthetic.captions(LENS, seed=3))).cuda()
    return lat, caps


def test_clean_forward_is_unchanged():
    torch = _torch()
    lat, caps = _inputs()
    outs = []
    for check in (0, 1):
        dit = _engine(check)
        o = torch.empty_like(lat)
        dit.forward(lat, caps, LENS, T, o)
        torch.cuda.synchronize()
        outs.append(o.cpu())
        dit.close()
    assert torch.isfinite(outs[0]).all().item()
    assert torch.equal(outs[0], outs[1])


def test_nan_in_latent_and_inf_in_caption_are_caught_at_the_embeddings():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    lat, caps = _inputs()
    dit = _engine(1)
    out = torch.empty_like(lat)
    bad_lat = lat.clone()
    bad_lat[1, 3, 5, 7] = float("nan")
    with pytest.raises(binding.ZimgError) as ei:
        dit.forward(bad_lat, caps, LENS, T, out)
    assert ei.value.code == binding.ZIMG_ENONFINITE and "after the embeddings" in str(ei.value)
    bad_caps = caps.clone()
    bad_caps[LENS[0] + 4, 11] = float("inf")
    with pytest.raises(binding.ZimgError) as ei:
        dit.forward(lat, bad_caps, LENS, T, out)
    assert ei.value.code == binding.ZIMG_ENONFINITE and "after the embeddings" in str(ei.value)
    # the handle stays usable: a clean call afterwards succeeds
    dit.forward(lat, caps, LENS, T, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    dit.close()


@pytest.mark.parametrize("name,block", [("layers.1.feed_forward.w2.weight", "block 3 (layers.1)"),
                                        ("context_refiner.0.attention.to_v.weight", "block 1 (context_refiner.0)")])
def test_nan_in_a_block_weight_names_that_block(name, block):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(SMALL, max_batch=2, max_image_tokens=96, max_caption_tokens=64, check_finite=1)
    W = dict(helpers.engine_weights(ecfg, seed=3).materialize(workers=4))
    w = W[name].copy()
    w.flat[w.size // 3] = np.nan
    W[name] = w
    dit = binding.DiT(ecfg, W)
    lat, caps = _inputs()
    out = torch.empty_like(lat)
    with pytest.raises(binding.ZimgError) as ei:
        dit.forward(lat, caps, LENS, T, out)
    assert ei.value.code == binding.ZIMG_ENONFINITE and block in str(ei.value), str(ei.value)
    dit.close()


def test_a_nan_sample_leaves_the_other_samples_and_later_calls_unchanged():
    """Samples never interact, whatever the other rows hold: a NaN in sample
    1 leaves sample 0's output bitwise as in a clean batch of the same
    geometry (keys past a range's end have weight 0 and their V^T columns
    are loaded as zeros, so 0 * NaN never reaches another sample), and the
    handle is not poisoned: later clean calls, of the same geometry and of a
    smaller one whose alignment rows were that sample's tokens, give bitwise
    what a fresh engine gives."""
    torch = _torch()
    lat, caps = _inputs()

    def run(dit, lat_d, caps_d, lens, t):
        o = torch.empty_like(lat_d)
        dit.forward(lat_d, caps_d, lens, t, o)
        torch.cuda.synchronize()
        return o.cpu()

    small_lat = torch.from_numpy(synthetic.latent((1, 16, 10, 12), seed=5)).cuda()  # 30 tokens, 2 alignment rows
    small_caps = torch.from_numpy(np.concatenate(synthetic.captions((9,), seed=5))).cuda()
    fresh = _engine(0)
    clean = run(fresh, lat, caps, LENS, T)
    clean_small = run(fresh, small_lat, small_caps, (9,), (0.4,))
    fresh.close()

    dit = _engine(0)
    bad = lat.clone()
    bad[1, 0, 2, 2] = float("nan")
    got = run(dit, bad, caps, LENS, T)
    assert torch.isnan(got[1]).any().item()
    assert torch.equal(got[0], clean[0]), "a NaN in sample 1 reached sample 0"
    bad0 = lat.clone()
    bad0[0, 0, 15, 23] = float("nan")  # sample 0, whose rows become alignment rows below
    assert torch.isnan(run(dit, bad0, caps, LENS, T)[0]).any().item()
    assert torch.equal(run(dit, small_lat, small_caps, (9,), (0.4,)), clean_small)
    assert torch.equal(run(dit, lat, caps, LENS, T), clean)
    dit.close()
