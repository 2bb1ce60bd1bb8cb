"""The 8-step FlowMatch Euler workload (shift 3, batch 2, captions of 77 and
300 tokens, FFN w2 outputs with outliers up to ~1e6).

At reduced width the whole loop runs against the oracle's loop; at full
width and the workload's 1536x640 geometry the loop runs against the float64
oracle's outputs stored by tests/golden/make_fullsize_outputs.py (the oracle
needs about 20 minutes of CPU per full-width step of the pair), and is
checked for finiteness, bitwise reproducibility, and batch independence (each sample run alone matches its
row of the batch to the parity bar; not bitwise: the batch size changes the
GEMM tile counts and attention work items, and so which of them are split
along K or keys, i.e. the fp32 summation order, and after 8 x 34 blocks
those last-bit differences have flipped enough bf16 roundings to reach
~2.5e-3.  The engine's batch-invariant option disables those splits).
"""

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


def _engine(model, max_batch, max_img, max_cap, outlier_log2, **extra):
    from diffusion_transformer_image_amd import binding
    ecfg = helpers.engine_config(model, max_batch=max_batch, max_image_tokens=max_img,
                                 max_caption_tokens=max_cap, **extra)
    W = helpers.engine_weights(ecfg, outlier_log2=outlier_log2)
    return binding.DiT(ecfg, W.items_parallel(as_bits=True))


@pytest.mark.parametrize("quant", [None, "int8"])
def test_euler_loop_reduced_width_vs_oracle(quant):
    """bf16: every step's model output and the final latent at the parity
    bar.  int8 block projections: against the oracle's int8 loop at the int8
    bar (tests/test_gpu_int8.py derives it), and the final latent against the
    float oracle's at the pages' int8 quality figure (cosine >= 0.9996)."""
    torch = _torch()
    from diffusion_transformer_image_amd import euler_loop
    from tests.test_gpu_int8 import I8_COS_TOL, I8_REL_TOL, INT8_COS_GATE
    lens, shape, log2 = (77, 300), (2, 16, 48, 32), 20
    dit = _engine(REDUCED, 2, 24 * 16, 300, log2, linear_int8=1 if quant else 0)
    lat = synthetic.latent(shape, seed=5)
    caps = synthetic.captions(lens, seed=5)
    x = torch.from_numpy(lat).cuda()
    caps_d = torch.from_numpy(np.concatenate(caps)).cuda()
    outs_gpu = []
    euler_loop(dit, x, caps_d, lens, n_steps=8, shift=3.0,
               on_step=lambda k, xx, o: outs_gpu.append(o.cpu().numpy()))
    torch.cuda.synchronize()
    got = x.cpu().numpy()

    ocfg = helpers.oracle_config(REDUCED)
    Wo = helpers.oracle_weights(REDUCED, outlier_log2=log2).materialize(workers=4)
    peaks = []
    outs_ref = []

    def model_fn(xx, tt):
        return om.forward(ocfg, Wo, xx, caps, tt, ffn_peak=peaks if not outs_ref else None, quant=quant)

    ref = osm.run(model_fn, lat, n_steps=8, shift=3.0, on_step=lambda k, xx, o: outs_ref.append(o))
    # heavy-tailed FFN outputs were present (the outlier channels dominate)
    assert max(peaks) > 1e5, f"w2 output peak {max(peaks):.3g}"
    tol = (I8_REL_TOL, I8_COS_TOL) if quant else (helpers.REL_L2_TOL, helpers.COS_TOL)
    for k in range(8):
        helpers.assert_parity(outs_gpu[k], outs_ref[k], f"step {k} model output", *tol)
    r, c = helpers.assert_parity(got, ref, "final latent after 8 steps", *tol)
    msg = f"w2 output peak {max(peaks):.3g}; final latent rel-L2 {r:.2e} cos {c:.7f}"
    if quant:
        ref_f = osm.run(lambda xx, tt: om.forward(ocfg, Wo, xx, caps, tt), lat, n_steps=8, shift=3.0)
        cf = helpers.cosine(got, ref_f)
        assert cf >= INT8_COS_GATE, f"final latent cosine {cf:.6f} against the float oracle's loop"
        msg += f"; vs the float loop cos {cf:.7f}"
    print(msg)
    dit.close()


def _golden():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "euler_1536x640_oracle_outputs.npz")
    if not os.path.exists(path):
        return None, None
    z = np.load(path)
    return {k: z[k] for k in z.files if k != "meta"}, json.loads(str(z["meta"]))


def test_euler_loop_full_size_vs_stored_oracle():
    """The full-width loop at 1536x640, batch 2, captions 77 / 300, w2
    outliers: the step-0 model output of the batch against the stored
    float64 oracle output (every sample at the parity bar), and, where the
    oracle's whole 8-step loop is stored, every step's model output and the
    final latent."""
    torch = _torch()
    from diffusion_transformer_image_amd import euler_loop
    wl = synthetic.WORKLOADS["euler_1536x640"]
    gold, meta = _golden()
    if gold is None:
        pytest.skip("tests/golden/euler_1536x640_oracle_outputs.npz not written")
    assert meta["outlier_log2"] == wl["outlier_log2"] and meta["caption_lens"] == list(wl["caption_lens"])
    lens, shape = wl["caption_lens"], wl["latent"]
    dit = _engine(wl["model"], 2, (shape[2] // 2) * (shape[3] // 2), max(lens), wl["outlier_log2"])
    lat = synthetic.latent(shape, seed=wl["seed"])
    caps = synthetic.captions(lens, seed=wl["seed"])
    x = torch.from_numpy(lat).cuda()
    outs = []
    euler_loop(dit, x, torch.from_numpy(np.concatenate(caps)).cuda(), lens, n_steps=wl["steps"], shift=wl["shift"],
               on_step=lambda k, xx, o: outs.append(o.cpu().numpy()))
    torch.cuda.synchronize()
    for b in range(2):
        r, c = helpers.assert_parity(outs[0][b], gold["out0"][b].astype(np.float64), f"step 0 sample {b}")
        print(f"step 0 sample {b}: rel-L2 {r:.2e} cos {c:.7f}")
    if "final" in gold:
        for k in range(wl["steps"]):
            r, c = helpers.assert_parity(outs[k], gold["outs"][k].astype(np.float64), f"step {k} model output")
            print(f"step {k}: rel-L2 {r:.2e} cos {c:.7f}")
        r, c = helpers.assert_parity(x.cpu().numpy(), gold["final"].astype(np.float64), "final latent")
        print(f"final latent after {wl['steps']} steps: rel-L2 {r:.2e} cos {c:.7f}")
    dit.close()


def test_euler_step0_full_size_int8_vs_stored_oracle():
    """Int8 block projections on the full-width Euler workload (1536x640,
    batch 2, captions 77 / 300, w2 outliers): the step-0 model output of the
    batch is as close to the float64 output as the oracle's own int8 variant
    of that step (stored next to the float runs) is, up to a fifth of the
    scheme's own loss.

    Here the int8 scheme itself loses accuracy: after the first block the
    residual carries the w2 outlier channels (about 30x the row rms), so the
    per-token scale of every later block input is set by them and the rest
    of each row keeps only a few quantization levels (input error 4 % after
    two blocks against 1 % without outliers).  With steps that coarse, the
    engine and the oracle (whose fp32 / bf16 values feeding each quantizer
    differ at the 1e-3 level) take many code decisions differently, so the
    two int8 results are compared through their distance to the float output
    rather than element by element at the int8 bar of ordinary rows."""
    torch = _torch()
    wl = synthetic.WORKLOADS["euler_1536x640"]
    gold, meta = _golden()
    if gold is None or "out0_int8" not in gold:
        pytest.skip("the oracle's int8 step-0 output is not stored (make_fullsize_outputs.py euler_int8)")
    lens, shape = wl["caption_lens"], wl["latent"]
    dit = _engine(wl["model"], 2, (shape[2] // 2) * (shape[3] // 2), max(lens), wl["outlier_log2"], linear_int8=1)
    x = torch.from_numpy(synthetic.latent(shape, seed=wl["seed"])).cuda()
    caps = torch.from_numpy(np.concatenate(synthetic.captions(lens, seed=wl["seed"]))).cuda()
    t0 = float(np.float32(meta["t0"]))
    out = torch.empty_like(x)
    dit.forward(x, caps, lens, (t0, t0), out)
    torch.cuda.synchronize()
    dit.close()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    ref_f, ref_q = gold["out0"].astype(np.float64), gold["out0_int8"].astype(np.float64)
    cf, co = helpers.cosine(got, ref_f), meta["int8_step0_vs_float_cosine"]
    print(f"int8 step 0: cosine vs the float oracle: engine {cf:.7f}, oracle's int8 variant {co:.7f}; engine vs the "
          f"int8 oracle: rel-L2 {helpers.rel_l2(got, ref_q):.2e} cos {helpers.cosine(got, ref_q):.6f}")
    assert cf >= co - (1.0 - co) / 5, f"engine int8 cosine {cf:.7f} vs the oracle's int8 variant {co:.7f}"


def test_euler_loop_full_size_reproducible_and_batch_independent():
    torch = _torch()
    from diffusion_transformer_image_amd import euler_loop
    wl = synthetic.WORKLOADS["euler_1536x640"]
    lens, shape = wl["caption_lens"], wl["latent"]
    dit = _engine(wl["model"], 2, (shape[2] // 2) * (shape[3] // 2), max(lens), wl["outlier_log2"])
    lat = synthetic.latent(shape, seed=wl["seed"])
    caps = synthetic.captions(lens, seed=wl["seed"])
    xb = torch.from_numpy(lat).cuda()
    euler_loop(dit, xb, torch.from_numpy(np.concatenate(caps)).cuda(), lens, n_steps=wl["steps"],
               shift=wl["shift"])
    torch.cuda.synchronize()
    assert torch.isfinite(xb).all().item()
    xb2 = torch.from_numpy(lat).cuda()
    euler_loop(dit, xb2, torch.from_numpy(np.concatenate(caps)).cuda(), lens, n_steps=wl["steps"],
               shift=wl["shift"])
    torch.cuda.synchronize()
    assert torch.equal(xb, xb2), "the 8-step loop is not reproducible"
    for b in range(2):
        xs = torch.from_numpy(lat[b:b + 1].copy()).cuda()
        euler_loop(dit, xs, torch.from_numpy(caps[b]).cuda(), lens[b:b + 1], n_steps=wl["steps"],
                   shift=wl["shift"])
        torch.cuda.synchronize()
        r = helpers.rel_l2(xs[0].cpu().numpy(), xb[b].cpu().numpy())
        print(f"sample {b}: alone vs in batch rel-L2 {r:.2e}")
        # measured 2.5e-3 after 8 x 34 blocks; the bar is about three times that
        assert r <= 8e-3, f"sample {b} alone vs in batch: rel-L2 {r:.3e}"
    dit.close()
