"""Shared helpers of the test-suite: configs of both sides from one workload
recipe, seeded weights for both sides, error metrics, row-layout mapping."""

import numpy as np

import synthetic
from oracle import ModelConfig
from oracle import manifest as oracle_manifest

# parity bar on every block output (fp32 residual rows), accumulated in float64
REL_L2_TOL = 1e-2
COS_TOL = 0.9999
# what a block adds to the residual (output - input, each side its own
# input), over all compared rows and for the worst single row: the residual
# dominates a block's output, so a fault confined to one row tile or one
# head would hide in the aggregate residual figure but not here
BRANCH_TOL = 3e-2
ROW_BRANCH_TOL = 5e-2


def oracle_config(model: dict) -> ModelConfig:
    return ModelConfig.from_dict(model)


def engine_config(model: dict, max_batch=1, max_image_tokens=4096, max_caption_tokens=512, **extra):
    from diffusion_transformer_image_amd import binding
    kw = dict(model, **extra)
    return binding.config(max_batch=max_batch, max_image_tokens=max_image_tokens,
                          max_caption_tokens=max_caption_tokens, **kw)


def oracle_weights(model: dict, seed=0, outlier_log2=None):
    return synthetic.SyntheticWeights(oracle_manifest(oracle_config(model)), seed=seed,
                                      outlier_log2=outlier_log2)


def engine_weights(ecfg, seed=0, outlier_log2=None):
    """The engine's own manifest drives the draw; values equal the oracle's by name."""
    from diffusion_transformer_image_amd import binding
    return synthetic.SyntheticWeights(binding.manifest(ecfg), seed=seed, outlier_log2=outlier_log2)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def cosine(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(got @ ref / max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300))


def assert_parity(got, ref, what, rel_tol=REL_L2_TOL, cos_tol=COS_TOL):
    r, c = rel_l2(got, ref), cosine(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert r <= rel_tol and c >= cos_tol, f"{what}: rel-L2 {r:.3e} (<= {rel_tol}), cosine {c:.6f} (>= {cos_tol})"
    return r, c


def row_rel_l2(got, ref):
    """Relative L2 error of each row (last axis), in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def assert_branch(got, got_in, want, want_in, what, tol=BRANCH_TOL, row_tol=ROW_BRANCH_TOL):
    """The block's added branch (output minus input, each side its own
    input) against the oracle's: rel-L2 over all rows <= tol, and every
    single row's rel-L2 <= row_tol.  Returns (aggregate, worst row)."""
    bg = np.asarray(got, np.float64) - np.asarray(got_in, np.float64)
    bw = np.asarray(want, np.float64) - np.asarray(want_in, np.float64)
    rb = rel_l2(bg, bw)
    rows = row_rel_l2(bg.reshape(-1, bg.shape[-1]), bw.reshape(-1, bw.shape[-1]))
    worst, at = float(rows.max()), int(rows.argmax())
    assert rb <= tol, f"{what}: branch rel-L2 {rb:.3e} (<= {tol})"
    assert worst <= row_tol, f"{what}: branch rel-L2 of row {at} is {worst:.3e} (<= {row_tol})"
    return rb, worst


def engine_rows(img_off, cap_off, b, n_img, n_cap):
    """Engine row indices of sample b in the oracle's [image; caption] order."""
    return np.concatenate([img_off[b] + np.arange(n_img), cap_off[b] + np.arange(n_cap)])
