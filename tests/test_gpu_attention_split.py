"""Attention with split key ranges, through the C ABI, against the oracle.

When the (query tile, head) pairs of the last round of resident attention
workgroups would fill at most half of the GPU, each of those pairs is split
into chunks of its 64-key tiles and the chunks' partial softmax states are
merged by a second kernel.  These cases are chosen so that the split path
runs with chunks of an odd tile count (padded inside the kernel), chunks of
unequal length, a chunk that crosses from a sample's image keys into its
caption keys, ragged last tiles, and two samples of different caption
lengths in one launch.  Each block kind runs once on a seeded residual and
is compared, per sample, with the oracle's block on that sample's rows.
"""

import numpy as np
import pytest

import synthetic
from oracle import model as om
from tests import helpers

pytestmark = pytest.mark.gpu

NARROW = dict(hidden=256, n_heads=2, ffn=512, n_layers=1, n_noise_refiner=1, n_context_refiner=1)

# (latent shape, caption lengths, stages whose attention must be split)
CASES = [
    ((1, 16, 40, 42), (45,), (0, 2)),            # 420 image keys: 7 tiles -> chunks 2, 2, 3
    ((2, 16, 40, 42), (45, 300), (0, 2)),        # joint chunks of 3 cross the image/caption edge
    ((1, 16, 96, 96), (300,), (0, 1, 2)),        # 41 joint tiles in 12 unequal chunks
]


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def engine():
    _torch()
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(NARROW, max_batch=2, max_image_tokens=48 * 48, max_caption_tokens=300)
    W = helpers.engine_weights(ecfg, seed=7)
    dit = binding.DiT(ecfg, W.items_parallel(as_bits=True))
    yield dit
    dit.close()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_split_attention_blocks_vs_oracle(engine, case):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    shape, lens, split_stages = CASES[case]
    B, _, Hl, Wl = shape
    Hp, Wp = Hl // 2, Wl // 2
    N = Hp * Wp
    img_off, cap_off, S = binding.row_layout(B, N, list(lens))
    D = NARROW["hidden"]
    ts = [0.25, 0.7][:B]
    x0 = synthetic.residual((S, D), seed=20 + case)
    ocfg = helpers.oracle_config(NARROW)
    Wo = helpers.oracle_weights(NARROW, seed=7)
    cvec = om.timestep_mlp(ocfg, Wo, np.array(ts, dtype=np.float32).astype(np.float64))
    kinds = [(0, "noise_refiner.0", True), (1, "context_refiner.0", False), (2, "layers.0", True)]
    for bi, prefix, modulated in kinds:
        xd = torch.from_numpy(x0).cuda()
        engine.run_blocks(xd, B, Hl, Wl, list(lens), ts, bi, 1)
        torch.cuda.synchronize()
        got_all = xd.cpu().numpy()
        pairs, n_full, split = engine.attention_plan(bi)
        print(f"case {case} {prefix}: pairs {pairs}, whole {n_full}, chunks {split}")
        if bi in split_stages:
            assert split >= 2 and n_full < pairs, f"{prefix}: attention was not split"
        for b in range(B):
            L = lens[b]
            cap_ids, img_ids = om.position_ids(L, Hp, Wp)
            ri = img_off[b] + np.arange(N)
            rc = cap_off[b] + np.arange(L)
            if bi == 0:
                rows = ri
                cos, sin = om.rope_tables(ocfg, img_ids)
            elif bi == 1:
                rows = rc
                cos, sin = om.rope_tables(ocfg, cap_ids)
            else:
                rows = np.concatenate([ri, rc])
                ci, si = om.rope_tables(ocfg, img_ids)
                cc, sc = om.rope_tables(ocfg, cap_ids)
                cos, sin = np.concatenate([ci, cc]), np.concatenate([si, sc])
            xin = x0[rows].astype(np.float64)
            mod = om.block_modulation(Wo, prefix, cvec[b]) if modulated else None
            want = om.block(ocfg, Wo, prefix, xin, cos, sin, mod)
            got = got_all[rows]
            r, cs = helpers.assert_parity(got, want, f"case {case} sample {b} {prefix}")
            rb, rw = helpers.assert_branch(got, xin, want, xin, f"case {case} sample {b} {prefix}")
            print(f"  sample {b}: rel-L2 {r:.2e} cos {cs:.7f} branch {rb:.2e} worst row {rw:.2e}")
