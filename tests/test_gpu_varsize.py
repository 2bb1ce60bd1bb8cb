"""Batches whose samples differ in image size as well as caption length
(zimg_dit_forward_varsize): every block of every sample against the oracle
run on that sample alone; a sample in the batch against the same sample run
alone (bitwise with batch_invariant = 1); one-size batches through both entry
points bitwise equal; argument errors."""

import numpy as np
import pytest

import synthetic
from oracle import model as om
from tests import helpers

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=512, n_heads=4, ffn=1536, n_layers=2, n_noise_refiner=1, n_context_refiner=1)
# latent sizes (Hl, Wl), caption lengths, model times: 120, 6 and 17 image
# tokens (two of them not multiples of 16), captions of 77, 1 and 33 tokens
SIZES = [(24, 20), (4, 6), (2, 34)]
LENS = (77, 1, 33)
TIMES = (0.3, 0.6, 0.9)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _engine(batch_invariant=0, max_batch=3, seed=7):
    from diffusion_transformer_image_amd import binding
    n_max = max((h // 2) * (w // 2) for h, w in SIZES)
    ecfg = helpers.engine_config(SMALL, max_batch=max_batch, max_image_tokens=n_max, max_caption_tokens=max(LENS),
                                 batch_invariant=batch_invariant)
    return binding.DiT(ecfg, helpers.engine_weights(ecfg, seed=seed).items_parallel(as_bits=True))


def _inputs(seed=7):
    torch = _torch()
    lats = [synthetic.latent((1, 16, h, w), seed=seed + i)[0] for i, (h, w) in enumerate(SIZES)]
    caps = synthetic.captions(LENS, seed=seed)
    return lats, caps, [torch.from_numpy(x).cuda() for x in lats], torch.from_numpy(np.concatenate(caps)).cuda()


def test_varsize_batch_vs_oracle():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    from oracle.manifest import block_prefixes
    dit = _engine()
    lats, caps, lat_d, caps_d = _inputs()
    n_img = [(h // 2) * (w // 2) for h, w in SIZES]
    img_off, cap_off, S = binding.row_layout_varsize(n_img, LENS)
    D = SMALL["hidden"]
    cap = torch.full(((dit.n_blocks + 1) * S * D,), float("nan"), device="cuda")
    dit.set_capture(cap)
    outs = [torch.empty_like(x) for x in lat_d]
    dit.forward_varsize(lat_d, caps_d, LENS, TIMES, outs)
    torch.cuda.synchronize()
    dit.set_capture(None)
    capt = cap.cpu().numpy().reshape(dit.n_blocks + 1, S, D)
    ocfg = helpers.oracle_config(SMALL)
    Wo = helpers.oracle_weights(SMALL, seed=7).materialize(workers=4)
    prefixes = [p for p, _ in block_prefixes(ocfg)]
    worst, worst_row = 0.0, 0.0
    for b in range(3):
        c = {}
        ref = om.forward_sample(ocfg, Wo, lats[b], caps[b], float(np.float32(TIMES[b])), capture=c)
        ri = img_off[b] + np.arange(n_img[b])
        rc = cap_off[b] + np.arange(LENS[b])
        helpers.assert_parity(capt[0][ri], c["x_embed"], f"sample {b} x_embed")
        helpers.assert_parity(capt[0][rc], c["cap_embed"], f"sample {b} cap_embed")
        # block inputs of each side: the branch check subtracts each side's own input
        g_img, g_cap, o_img, o_cap = capt[0][ri], capt[0][rc], c["x_embed"], c["cap_embed"]
        g_prev = o_prev = None
        for i, p in enumerate(prefixes):
            slot = capt[i + 1]
            if p.startswith("noise_refiner"):
                got, gin, oin = slot[ri], g_img, o_img
                g_img, o_img = got, c[p]
            elif p.startswith("context_refiner"):
                got, gin, oin = slot[rc], g_cap, o_cap
                g_cap, o_cap = got, c[p]
            else:
                got = np.concatenate([slot[ri], slot[rc]])
                if o_prev is None:
                    gin, oin = np.concatenate([g_img, g_cap]), np.concatenate([o_img, o_cap])
                else:
                    gin, oin = g_prev, o_prev
                g_prev, o_prev = got, c[p]
            r, _ = helpers.assert_parity(got, c[p], f"sample {b} {p}")
            _, rw = helpers.assert_branch(got, gin, c[p], oin, f"sample {b} {p}")
            worst, worst_row = max(worst, r), max(worst_row, rw)
        r, _ = helpers.assert_parity(outs[b].cpu().numpy(), ref, f"sample {b} final output")
        worst = max(worst, r)
    print(f"worst rel-L2 {worst:.2e}, worst row branch rel-L2 {worst_row:.2e}")


def test_varsize_sample_alone_equals_in_batch():
    """With batch_invariant = 1 each sample's output is bitwise the one it
    gets alone through the one-size entry point."""
    torch = _torch()
    dit = _engine(batch_invariant=1)
    lats, caps, lat_d, caps_d = _inputs()
    outs = [torch.empty_like(x) for x in lat_d]
    dit.forward_varsize(lat_d, caps_d, LENS, TIMES, outs)
    for b in range(3):
        alone = torch.empty_like(lat_d[b][None])
        dit.forward(lat_d[b][None].contiguous(), torch.from_numpy(caps[b]).cuda(), LENS[b:b + 1], TIMES[b:b + 1], alone)
        torch.cuda.synchronize()
        assert torch.equal(alone[0], outs[b]), f"sample {b}"


@pytest.mark.parametrize("batch_invariant", [0, 1])
def test_one_size_batch_both_entry_points(batch_invariant):
    """B latents of one size: the varsize call on separate buffers equals the
    one-size call on a [B, C, Hl, Wl] array (bitwise with batch_invariant =
    1; to the parity bar otherwise, since the one-size call runs the final
    layer as one GEMM whose last-wave split may differ)."""
    torch = _torch()
    dit = _engine(batch_invariant=batch_invariant, max_batch=2)
    lat = torch.from_numpy(synthetic.latent((2, 16, 24, 20), seed=11)).cuda()
    lens = (40, 64)
    caps = torch.from_numpy(np.concatenate(synthetic.captions(lens, seed=11))).cuda()
    t = (0.25, 0.75)
    o1 = torch.empty_like(lat)
    dit.forward(lat, caps, lens, t, o1)
    parts = [lat[0].clone(), lat[1].clone()]
    outs = [torch.empty_like(p) for p in parts]
    dit.forward_varsize(parts, caps, lens, t, outs)
    # the same buffers seen as one array take the one-launch path
    o3 = torch.empty_like(lat)
    dit.forward_varsize([lat[0], lat[1]], caps, lens, t, [o3[0], o3[1]])
    torch.cuda.synchronize()
    assert torch.equal(o3, o1)
    for b in range(2):
        if batch_invariant:
            assert torch.equal(outs[b], o1[b])
        else:
            helpers.assert_parity(outs[b].cpu().numpy(), o1[b].cpu().numpy(), f"sample {b}")


def test_varsize_argument_errors():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    dit = _engine()
    lats, caps, lat_d, caps_d = _inputs()
    outs = [torch.empty_like(x) for x in lat_d]
    odd = torch.zeros((16, 5, 6), device="cuda")
    big = torch.zeros((16, 26, 20), device="cuda")  # 130 image tokens > 120
    cases = [
        (lambda: dit.forward_varsize([lat_d[0], odd, lat_d[2]], caps_d, LENS, TIMES, [outs[0], torch.empty_like(odd), outs[2]]),
         "multiples"),
        (lambda: dit.forward_varsize([lat_d[0], big, lat_d[2]], caps_d, LENS, TIMES, [outs[0], torch.empty_like(big), outs[2]]),
         "exceed"),
        (lambda: dit.forward_varsize(lat_d, caps_d, (77, 0, 33), TIMES, outs), "length 0"),
    ]
    for fn, msg in cases:
        with pytest.raises(binding.ZimgError) as ei:
            fn()
        assert ei.value.code == binding.ZIMG_EINVAL and msg in str(ei.value), str(ei.value)
    with pytest.raises(ValueError):
        dit.forward_varsize(lat_d, caps_d, LENS, TIMES, outs[:2])


def test_varsize_batch_int8_projections():
    """The mixed batch with int8 block projections: each sample's output
    against the oracle's int8 variant on that sample alone (int8 bar) and
    against the float oracle (the pages' int8 cosine)."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    from tests.test_gpu_int8 import I8_COS_TOL, I8_REL_TOL, INT8_COS_GATE
    n_max = max((h // 2) * (w // 2) for h, w in SIZES)
    ecfg = helpers.engine_config(SMALL, max_batch=3, max_image_tokens=n_max, max_caption_tokens=max(LENS),
                                 linear_int8=1)
    dit = binding.DiT(ecfg, helpers.engine_weights(ecfg, seed=7).items_parallel(as_bits=True))
    lats, caps, lat_d, caps_d = _inputs()
    outs = [torch.empty_like(x) for x in lat_d]
    dit.forward_varsize(lat_d, caps_d, LENS, TIMES, outs)
    torch.cuda.synchronize()
    dit.close()
    ocfg = helpers.oracle_config(SMALL)
    Wo = helpers.oracle_weights(SMALL, seed=7).materialize(workers=4)
    for b in range(3):
        t32 = float(np.float32(TIMES[b]))
        got = outs[b].cpu().numpy()
        ref_q = om.forward_sample(ocfg, Wo, lats[b], caps[b], t32, quant="int8")
        helpers.assert_parity(got, ref_q, f"sample {b} vs the int8 oracle", I8_REL_TOL, I8_COS_TOL)
        cf = helpers.cosine(got, om.forward_sample(ocfg, Wo, lats[b], caps[b], t32))
        assert cf >= INT8_COS_GATE, f"sample {b}: cosine {cf:.6f} against the float oracle"
