"""Parity at the full sizes of the 1024x1024 and 2048x2048 workloads, in the
launch configuration the benchmark times (same kernels, tiles, splits).

The float64 oracle cannot run 34 full-width blocks in a test, so each kind
of block (noise refiner on the image rows, context refiner on the caption
rows, joint block on all rows) runs once on a seeded synthetic residual at
the full geometry, and the oracle computes its output for sampled rows (keys
and values still from every row).  The full-depth forward is checked for
properties that hold at any size: finite, bitwise reproducible, embeddings
equal to the oracle's.
"""

import numpy as np
import pytest

import synthetic
from oracle import model as om
from tests import helpers

pytestmark = pytest.mark.gpu

FULL = synthetic.WORKLOADS["dit_1024"]["model"]
THREE_BLOCKS = dict(FULL, n_layers=1, n_noise_refiner=1, n_context_refiner=1)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _engine(model, max_img, max_cap=512, max_batch=1, outlier_log2=None):
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(model, max_batch=max_batch, max_image_tokens=max_img,
                                 max_caption_tokens=max_cap)
    W = helpers.engine_weights(ecfg, outlier_log2=outlier_log2)
    return binding.DiT(ecfg, W.items_parallel(as_bits=True))


def _sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, n // 2, n - 2, n - 1]
    return np.unique(np.concatenate([[r for r in fixed if r < n], rng.choice(n, size=k, replace=False)]))


@pytest.fixture(scope="module")
def three_block_engine():
    _torch()
    dit = _engine(THREE_BLOCKS, 16384)
    yield dit
    dit.close()


@pytest.mark.parametrize("geom", [("dit_1024", 128), ("dit_2048", 256)])
def test_each_block_kind_at_full_size(three_block_engine, geom):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    name, side = geom
    L, t = 512, 0.5
    Hp = Wp = side // 2
    N = Hp * Wp
    img_off, cap_off, S = binding.row_layout(1, N, [L])
    assert S == N + L and cap_off[0] == N
    D = FULL["hidden"]
    x0 = synthetic.residual((S, D), seed=11)
    ocfg = helpers.oracle_config(THREE_BLOCKS)
    Wo = helpers.oracle_weights(THREE_BLOCKS)
    c = om.timestep_mlp(ocfg, Wo, np.array([t]))[0]
    cap_ids, img_ids = om.position_ids(L, Hp, Wp)
    cos_i, sin_i = om.rope_tables(ocfg, img_ids)
    cos_c, sin_c = om.rope_tables(ocfg, cap_ids)
    cases = [
        (0, "noise_refiner.0", slice(0, N), cos_i, sin_i, True),
        (1, "context_refiner.0", slice(N, S), cos_c, sin_c, False),
        (2, "layers.0", slice(0, S), np.concatenate([cos_i, cos_c]), np.concatenate([sin_i, sin_c]), True),
    ]
    for bi, prefix, rows_sl, cos, sin, modulated in cases:
        xd = torch.from_numpy(x0).cuda()
        three_block_engine.run_blocks(xd, 1, 2 * Hp, 2 * Wp, [L], [t], bi, 1)
        torch.cuda.synchronize()
        got_all = xd.cpu().numpy()
        # rows outside the block's stage are untouched
        untouched = np.ones(S, bool)
        untouched[rows_sl] = False
        assert np.array_equal(got_all[untouched], x0[untouched]), prefix
        xin = x0[rows_sl].astype(np.float64)
        rows = _sample_rows(xin.shape[0], 24, bi)
        mod = om.block_modulation(Wo, prefix, c) if modulated else None
        want = om.block(ocfg, Wo, prefix, xin, cos, sin, mod, rows=rows)
        got = got_all[rows_sl][rows]
        r, cs = helpers.assert_parity(got, want, f"{name} {prefix} sampled rows")
        rb, rw = helpers.assert_branch(got, xin[rows], want, xin[rows], f"{name} {prefix}")
        print(f"{name} {prefix}: rel-L2 {r:.2e} cos {cs:.7f} branch {rb:.2e} worst row {rw:.2e}")


def test_each_block_kind_euler_workload_full_width():
    """The 8-step Euler workload's geometry at full width: batch 2 at
    1536x640 (3,840 image tokens each), captions of 77 and 300 tokens, w2
    rows of 4 output channels per block scaled by 2**16.  Each kind of block
    runs once through zimg_dit_run_blocks on the batch; sampled rows of each
    sample are compared with the oracle's block on that sample alone.  The
    oracle's w2 outputs on those rows show the heavy tail the workload is
    meant to exercise ("Z-Image-Turbo MNN (int8, fp16-safe)", Conversion
    details: w2 outputs with outliers up to about 1e6): on these few rows
    their peak is above 2e5 and at most 1e6 (the whole step's peak, over
    every row of every block, is checked against (5e5, 1e6] on the stored
    oracle outputs)."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    wl = synthetic.WORKLOADS["euler_1536x640"]
    B, _, Hl, Wl = wl["latent"]
    lens, log2 = list(wl["caption_lens"]), wl["outlier_log2"]
    Hp, Wp = Hl // 2, Wl // 2
    N = Hp * Wp
    dit = _engine(THREE_BLOCKS, N, max(lens), max_batch=B, outlier_log2=log2)
    img_off, cap_off, S = binding.row_layout(B, N, lens)
    D = FULL["hidden"]
    ts = [0.1, 0.5]
    x0 = synthetic.residual((S, D), seed=17)
    ocfg = helpers.oracle_config(THREE_BLOCKS)
    Wo = helpers.oracle_weights(THREE_BLOCKS, outlier_log2=log2)
    cvec = om.timestep_mlp(ocfg, Wo, np.array(ts, dtype=np.float32).astype(np.float64))
    peak = 0.0
    for bi, prefix, modulated in [(0, "noise_refiner.0", True), (1, "context_refiner.0", False),
                                  (2, "layers.0", True)]:
        xd = torch.from_numpy(x0).cuda()
        dit.run_blocks(xd, B, Hl, Wl, lens, ts, bi, 1)
        torch.cuda.synchronize()
        got_all = xd.cpu().numpy()
        for b in range(B):
            L = lens[b]
            cap_ids, img_ids = om.position_ids(L, Hp, Wp)
            ri = img_off[b] + np.arange(N)
            rc = cap_off[b] + np.arange(L)
            ci, si = om.rope_tables(ocfg, img_ids)
            cc, sc = om.rope_tables(ocfg, cap_ids)
            rows_all, cos, sin = {0: (ri, ci, si), 1: (rc, cc, sc),
                                  2: (np.concatenate([ri, rc]), np.concatenate([ci, cc]),
                                      np.concatenate([si, sc]))}[bi]
            xin = x0[rows_all].astype(np.float64)
            rows = _sample_rows(xin.shape[0], 24, 100 * bi + b)
            mod = om.block_modulation(Wo, prefix, cvec[b]) if modulated else None
            taps = {}
            want = om.block(ocfg, Wo, prefix, xin, cos, sin, mod, rows=rows, taps=taps)
            got = got_all[rows_all][rows]
            what = f"1536x640 sample {b} {prefix}"
            r, cs = helpers.assert_parity(got, want, f"{what} sampled rows")
            rb, rw = helpers.assert_branch(got, xin[rows], want, xin[rows], what)
            p = float(np.max(np.abs(taps["ffn_out"])))
            peak = max(peak, p)
            print(f"{what}: rel-L2 {r:.2e} cos {cs:.7f} branch {rb:.2e} worst row {rw:.2e} w2 peak {p:.3g}")
    dit.close()
    assert 2e5 < peak <= 1e6, f"w2 output peak {peak:.4g} on the sampled rows outside (2e5, 1e6]"


@pytest.fixture(scope="module")
def full_engine():
    _torch()
    dit = _engine(FULL, 16384)
    yield dit
    dit.close()


def test_full_forward_1024_properties(full_engine):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    wl = synthetic.WORKLOADS["dit_1024"]
    lat = synthetic.latent(wl["latent"])
    caps = synthetic.captions(wl["caption_lens"])
    lat_d = torch.from_numpy(lat).cuda()
    caps_d = torch.from_numpy(np.concatenate(caps)).cuda()
    N, L, D = 4096, 512, FULL["hidden"]
    img_off, cap_off, S = binding.row_layout(1, N, [L])
    cap = torch.empty((full_engine.n_blocks + 1) * S * D, device="cuda")
    full_engine.set_capture(cap)
    o1 = torch.empty_like(lat_d)
    full_engine.forward(lat_d, caps_d, wl["caption_lens"], wl["t"], o1)
    full_engine.set_capture(None)
    o2 = torch.empty_like(lat_d)
    full_engine.forward(lat_d, caps_d, wl["caption_lens"], wl["t"], o2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all().item()
    assert torch.equal(o1, o2), "two forwards differ"
    emb = cap[: S * D].view(S, D).cpu().numpy()
    ocfg = helpers.oracle_config(FULL)
    Wo = helpers.oracle_weights(FULL)
    helpers.assert_parity(emb[:N], om.x_embed(ocfg, Wo, lat[0]), "1024 x_embed")
    helpers.assert_parity(emb[N:S], om.cap_embed(ocfg, Wo, caps[0]), "1024 cap_embed")
    # every block moved the residual and kept it finite
    res = cap.view(full_engine.n_blocks + 1, S, D)
    for i in range(1, full_engine.n_blocks + 1):
        assert torch.isfinite(res[i]).all().item()
        assert not torch.equal(res[i], res[i - 1])


def _golden(name):
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"{name}_oracle_outputs.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not written (tests/golden/make_fullsize_outputs.py)")
    z = np.load(path)
    return {k: z[k] for k in z.files if k != "meta"}, json.loads(str(z["meta"]))


def test_full_forward_2048_properties(full_engine):
    """The whole 34-block 2048x2048 forward: finite, bitwise reproducible,
    and equal to the stored float64 oracle output at the parity bar."""
    torch = _torch()
    wl = synthetic.WORKLOADS["dit_2048"]
    lat = synthetic.latent(wl["latent"], seed=wl["seed"])
    caps = synthetic.captions(wl["caption_lens"], seed=wl["seed"])
    lat_d = torch.from_numpy(lat).cuda()
    caps_d = torch.from_numpy(np.concatenate(caps)).cuda()
    o1 = torch.empty_like(lat_d)
    o2 = torch.empty_like(lat_d)
    full_engine.forward(lat_d, caps_d, wl["caption_lens"], wl["t"], o1)
    full_engine.forward(lat_d, caps_d, wl["caption_lens"], wl["t"], o2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all().item()
    assert torch.equal(o1, o2)
    assert o1.abs().max().item() > 0
    gold, meta = _golden("dit_2048")
    assert meta["latent"] == list(wl["latent"]) and meta["caption_lens"] == list(wl["caption_lens"])
    r, c = helpers.assert_parity(o1.cpu().numpy(), gold["float"].astype(np.float64), "2048 forward vs the oracle")
    print(f"2048x2048 forward vs the stored oracle output: rel-L2 {r:.2e}, cosine {c:.7f}")
