"""Full-forward parity through the C ABI against the float64 oracle on the
same seeded inputs: every block output (fp32 residual) and the final output,
at the tiny single-block workload, the full-width single block at 512x512,
and a small varlen batch whose image token count is not a multiple of 16.
Also: bitwise determinism, batch independence (bitwise with the
batch-invariant option), error paths."""

import math

import numpy as np
import pytest

import synthetic
from oracle import model as om
from tests import helpers

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _make_engine(model, max_batch, max_img, max_cap, seed=0, outlier_log2=None, **extra):
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(model, max_batch=max_batch, max_image_tokens=max_img,
                                 max_caption_tokens=max_cap, **extra)
    W = helpers.engine_weights(ecfg, seed=seed, outlier_log2=outlier_log2)
    return binding.DiT(ecfg, W.items_parallel(as_bits=True))


def _inputs(latent_shape, lens, seed=0):
    torch = _torch()
    lat = synthetic.latent(latent_shape, seed=seed)
    caps = synthetic.captions(lens, seed=seed)
    lat_d = torch.from_numpy(lat).cuda()
    caps_d = torch.from_numpy(np.concatenate(caps)).cuda()
    return lat, caps, lat_d, caps_d


def _run_with_capture(dit, lat_d, caps_d, lens, t):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    B, C, Hl, Wl = lat_d.shape
    n_img = (Hl // 2) * (Wl // 2)
    img_off, cap_off, S = binding.row_layout(B, n_img, lens)
    D = dit.cfg.hidden
    cap = torch.full(((dit.n_blocks + 1) * S * D,), float("nan"), device="cuda")
    dit.set_capture(cap)
    out = torch.empty_like(lat_d)
    dit.forward(lat_d, caps_d, lens, t, out)
    torch.cuda.synchronize()
    dit.set_capture(None)
    return out.cpu().numpy(), cap.cpu().numpy().reshape(dit.n_blocks + 1, S, D), img_off, cap_off


def _compare_forward(model, wl_latent, lens, t, max_img, max_cap, seed=0):
    dit = _make_engine(model, len(lens), max_img, max_cap, seed=seed)
    lat, caps, lat_d, caps_d = _inputs(wl_latent, lens, seed=seed)
    out, capt, img_off, cap_off = _run_with_capture(dit, lat_d, caps_d, lens, t)
    ocfg = helpers.oracle_config(model)
    Wo = helpers.oracle_weights(model, seed=seed)
    from oracle.manifest import block_prefixes
    prefixes = [p for p, _ in block_prefixes(ocfg)]
    n_img = (wl_latent[2] // 2) * (wl_latent[3] // 2)
    report = []
    for b in range(len(lens)):
        c = {}
        ref = om.forward_sample(ocfg, Wo, lat[b], caps[b], float(np.float32(t[b])), capture=c)
        ri = img_off[b] + np.arange(n_img)
        rc = cap_off[b] + np.arange(lens[b])
        helpers.assert_parity(capt[0][ri], c["x_embed"], f"sample {b} x_embed")
        helpers.assert_parity(capt[0][rc], c["cap_embed"], f"sample {b} cap_embed")
        # block inputs of each side: the branch check subtracts each side's own input
        o_img, o_cap = c["x_embed"], c["cap_embed"]
        g_img, g_cap = capt[0][ri], capt[0][rc]
        o_prev = g_prev = None
        for i, p in enumerate(prefixes):
            slot = capt[i + 1]
            if p.startswith("noise_refiner"):
                got, want, gin, oin = slot[ri], c[p], g_img, o_img
                g_img, o_img = got, want
            elif p.startswith("context_refiner"):
                got, want, gin, oin = slot[rc], c[p], g_cap, o_cap
                g_cap, o_cap = got, want
            else:
                got, want = np.concatenate([slot[ri], slot[rc]]), c[p]
                if o_prev is None:
                    gin, oin = np.concatenate([g_img, g_cap]), np.concatenate([o_img, o_cap])
                else:
                    gin, oin = g_prev, o_prev
                g_prev, o_prev = got, want
            r, cs = helpers.assert_parity(got, want, f"sample {b} {p}")
            # what the block added, compared on its own (not diluted by the residual)
            rb, rw = helpers.assert_branch(got, gin, want, oin, f"sample {b} {p}")
            report.append((b, p, f"rel-L2 {r:.2e}", f"cos {cs:.7f}", f"branch {rb:.2e}", f"worst row {rw:.2e}"))
        helpers.assert_parity(out[b], ref, f"sample {b} final output")
    return report, dit


def test_forward_tiny_block():
    wl = synthetic.WORKLOADS["tiny_block"]
    rep, _ = _compare_forward(wl["model"], wl["latent"], wl["caption_lens"], wl["t"], 256, 32)
    print(rep)


def test_forward_block_512():
    wl = synthetic.WORKLOADS["block_512"]
    rep, _ = _compare_forward(wl["model"], wl["latent"], wl["caption_lens"], wl["t"], 1024, 128)
    print(rep)


SMALL = dict(hidden=512, n_heads=4, ffn=1536, n_layers=2, n_noise_refiner=1, n_context_refiner=1)


def test_forward_small_varlen_batch():
    """B = 2, captions 77 and 45 tokens, 12x10 = 120 image tokens (padded rows)."""
    rep, _ = _compare_forward(SMALL, (2, 16, 24, 20), (77, 45), (0.3, 0.8), 120, 77)
    print(rep)


def test_forward_batch_past_one_conditioning_launch():
    """B = 10, each sample with its own timestep and caption length: the adaLN
    GEMV takes up to 8 samples per launch, so samples 8 and 9 go through a
    second launch; every sample's blocks and output against the oracle."""
    lens = (3, 17, 1, 40, 8, 25, 64, 2, 33, 11)
    t = tuple(0.05 + 0.09 * i for i in range(10))
    rep, _ = _compare_forward(SMALL, (10, 16, 4, 6), lens, t, 6, 64)
    print(rep[-3:])


@pytest.mark.parametrize("latent,lens", [
    ((1, 16, 2, 2), (1,)),                # one image token, one caption token
    ((3, 16, 4, 6), (1, 77, 33)),         # 6 image tokens; captions of 1, 77 and 33 tokens
    ((2, 16, 2, 34), (64, 65)),           # 1 x 17 image tokens; captions at a tile edge and one past it
])
def test_forward_degenerate_geometries(latent, lens):
    """Smallest images and captions, single-tile and one-past-a-tile key
    ranges, batches mixing them: every block against the oracle."""
    n_img = (latent[2] // 2) * (latent[3] // 2)
    t = tuple(0.2 + 0.3 * i for i in range(len(lens)))
    rep, _ = _compare_forward(SMALL, latent, lens, t, n_img, max(lens))
    print(rep[-1])


# alone vs in batch with the default splits: the batch changes which GEMM
# tiles are split along K and which attention pairs are split along keys
# (here sample 0's joint pairs run in two key chunks alone and whole in the
# batch), i.e. the fp32 summation order, and so some bf16 roundings of the
# activations downstream.  Measured 1.1e-3 after this 4-block model (sample
# 1: bitwise equal); the bar is three times that
SPLIT_ORDER_TOL = 3e-3


@pytest.mark.parametrize("batch_invariant", [0, 1])
def test_determinism_and_batch_independence(batch_invariant):
    """Two identical calls are bitwise equal.  A sample run alone matches its
    row of the batch: bitwise with batch_invariant = 1; by default only to
    the parity bar, since the batch changes which GEMM tiles and attention
    work items are split (the fp32 summation order)."""
    torch = _torch()
    dit = _make_engine(SMALL, 2, 120, 77, seed=3, batch_invariant=batch_invariant)
    lens = (77, 45)
    lat, caps, lat_d, caps_d = _inputs((2, 16, 24, 20), lens, seed=3)
    t = (0.3, 0.8)
    o1 = torch.empty_like(lat_d)
    o2 = torch.empty_like(lat_d)
    dit.forward(lat_d, caps_d, lens, t, o1)
    dit.forward(lat_d, caps_d, lens, t, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for b in range(2):
        ob = torch.empty_like(lat_d[b:b + 1])
        dit.forward(lat_d[b:b + 1].contiguous(), torch.from_numpy(caps[b]).cuda(), lens[b:b + 1], t[b:b + 1], ob)
        torch.cuda.synchronize()
        if batch_invariant:
            assert torch.equal(ob[0], o1[b]), f"sample {b} alone vs in batch differ"
        else:
            r = helpers.rel_l2(ob[0].cpu().numpy(), o1[b].cpu().numpy())
            print(f"sample {b}: alone vs in batch rel-L2 {r:.3e}")
            assert r <= SPLIT_ORDER_TOL, f"sample {b} alone vs in batch: rel-L2 {r:.3e}"


def test_caption_bf16_input_matches_fp32():
    torch = _torch()
    dit = _make_engine(SMALL, 1, 120, 77, seed=4)
    lat, caps, lat_d, caps_d = _inputs((1, 16, 24, 20), (50,), seed=4)
    o1 = torch.empty_like(lat_d)
    o2 = torch.empty_like(lat_d)
    dit.forward(lat_d, caps_d, (50,), (0.5,), o1)
    dit.forward(lat_d, caps_d.to(torch.bfloat16), (50,), (0.5,), o2)  # captions are bf16-exact
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_forward_argument_errors():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    dit = _make_engine(SMALL, 1, 120, 77, seed=5)
    lat_d = torch.zeros((1, 16, 24, 20), device="cuda")
    caps_d = torch.zeros((200, 2560), device="cuda")  # rows for every case's lengths
    out = torch.empty_like(lat_d)
    def run(lat, lens, t):
        return dit.forward(lat, caps_d, lens, t, torch.empty_like(lat))

    bad = [
        (lambda: run(torch.zeros((1, 16, 23, 20), device="cuda"), (50,), (0.5,)), "multiples"),
        (lambda: run(lat_d, (0,), (0.5,)), "length 0"),
        (lambda: run(lat_d, (78,), (0.5,)), "outside 1..77"),
        (lambda: run(lat_d, (50,), (math.nan,)), "not finite"),
        (lambda: run(torch.zeros((1, 16, 24, 22), device="cuda"), (50,), (0.5,)), "exceed"),
        (lambda: run(torch.zeros((2, 16, 24, 20), device="cuda"), (50, 50), (0.5, 0.5)), "batch"),
    ]
    for fn, msg in bad:
        with pytest.raises(binding.ZimgError) as ei:
            fn()
        assert ei.value.code == binding.ZIMG_EINVAL and msg in str(ei.value), str(ei.value)
    # refused by the binding before any native call: an output of another
    # shape (the library sees only a pointer), a half-precision latent
    with pytest.raises(ValueError, match="shape"):
        dit.forward(lat_d, caps_d, (50,), (0.5,), torch.empty((1, 16, 24, 18), device="cuda"))
    with pytest.raises(ValueError, match="dtype"):
        dit.forward(lat_d.half(), caps_d, (50,), (0.5,), out)


def test_weight_table_errors():
    _torch()
    from diffusion_transformer_image_amd import binding
    model = synthetic.WORKLOADS["tiny_block"]["model"]
    ecfg = helpers.engine_config(model, 1, 256, 32)
    W = dict(helpers.engine_weights(ecfg).materialize(workers=4))
    names = list(W)
    # missing
    with pytest.raises(binding.ZimgError) as ei:
        binding.DiT(ecfg, [(n, W[n]) for n in names[:-1]])
    assert ei.value.code == binding.ZIMG_EWEIGHT and names[-1] in str(ei.value)
    # unknown
    with pytest.raises(binding.ZimgError) as ei:
        binding.DiT(ecfg, list(W.items()) + [("layers.0.attention.to_qkv.weight", W[names[0]])])
    assert ei.value.code == binding.ZIMG_EWEIGHT and "unknown" in str(ei.value)
    # duplicate
    with pytest.raises(binding.ZimgError) as ei:
        binding.DiT(ecfg, list(W.items()) + [(names[3], W[names[3]])])
    assert ei.value.code == binding.ZIMG_EWEIGHT and "duplicate" in str(ei.value)
    # mis-shaped
    bad = dict(W)
    bad["all_x_embedder.2-1.weight"] = W["all_x_embedder.2-1.weight"][:, :32].copy()
    with pytest.raises(binding.ZimgError) as ei:
        binding.DiT(ecfg, bad)
    assert ei.value.code == binding.ZIMG_EWEIGHT and "all_x_embedder.2-1.weight" in str(ei.value)
    # fp32 and bf16-bit inputs give the same engine
    binding.DiT(ecfg, W).close()


def test_geometry_switches_reuse_cached_tables():
    """Forwards that alternate between geometries (more of them than the
    engine keeps tables for, so slots are evicted and rebuilt) give bitwise
    the outputs of the first forward at each geometry, and the attention
    plan follows the geometry of the latest call."""
    torch = _torch()
    dit = _make_engine(SMALL, 2, 120, 77, seed=6)
    geos = [((1, 16, 24, 20), (50,)), ((2, 16, 24, 20), (50, 31)), ((1, 16, 16, 16), (20,)),
            ((2, 16, 8, 12), (1, 77)), ((1, 16, 20, 24), (64,)), ((2, 16, 16, 16), (16, 17))]
    inputs = [_inputs(shape, lens, seed=10 + i) for i, (shape, lens) in enumerate(geos)]

    def run(i):
        (shape, lens), (_, _, lat_d, caps_d) = geos[i], inputs[i]
        out = torch.empty_like(lat_d)
        dit.forward(lat_d, caps_d, lens, tuple(0.25 + 0.5 * b for b in range(len(lens))), out)
        return out

    first = {}
    order = [0, 1, 0, 1, 2, 3, 4, 5, 0, 2, 1, 5, 5, 3]
    outs = [run(i) for i in order]  # enqueued back to back, no synchronisation in between
    torch.cuda.synchronize()
    for i, o in zip(order, outs):
        if i not in first:
            first[i] = o
        else:
            assert torch.equal(o, first[i]), f"geometry {geos[i]} changed after switching"
    plan_last = dit.attention_plan(2)
    # a fresh engine at the last geometry makes the same plan
    dit2 = _make_engine(SMALL, 2, 120, 77, seed=6)
    lat_d, caps_d = inputs[order[-1]][2], inputs[order[-1]][3]
    dit2.forward(lat_d, caps_d, geos[order[-1]][1], (0.25, 0.75), torch.empty_like(lat_d))
    torch.cuda.synchronize()
    assert dit2.attention_plan(2) == plan_last
    dit.close()
    dit2.close()

