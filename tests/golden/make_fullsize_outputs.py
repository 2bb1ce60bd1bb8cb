"""Write the oracle's outputs of the two large workloads that no test can
recompute in its run time, as float16 arrays next to this file:

  euler_1536x640_oracle_outputs.npz
      the 8-step FlowMatch Euler loop at 1536x640 (latent [2, 16, 192, 80]),
      batch 2 with captions of 77 and 300 tokens, w2 outliers scaled by
      2**16: the step-0 model output of the batch (``out0``), the largest
      |w2 output| of every block of that step for each sample (``ffn_peak``,
      float64), and -- with ``--loop`` -- the model output of every step and
      the final latent after 8 steps (``outs``, ``final``); ``euler_int8``
      adds the oracle's int8 variant of the step-0 model output
      (``out0_int8``) to that file;
  dit_2048_oracle_outputs.npz
      the 2048x2048 forward (16,384 image + 512 caption tokens, t = 0.5).

Calls only oracle/ and the seeded input generators (synthetic/).  The float64
oracle takes about 20 minutes per full-width 1536x640 forward of the pair and
about an hour for the 2048x2048 forward on an 8-core host:

    python tests/golden/make_fullsize_outputs.py euler [--loop]
    python tests/golden/make_fullsize_outputs.py euler_int8
    python tests/golden/make_fullsize_outputs.py dit_2048
"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402
from oracle import ModelConfig, manifest  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import sampler as osm  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def euler(loop):
    name = "euler_1536x640"
    wl = synthetic.WORKLOADS[name]
    cfg = ModelConfig.from_dict(wl["model"])
    W = synthetic.SyntheticWeights(manifest(cfg), seed=wl["seed"], outlier_log2=wl["outlier_log2"])
    lat = synthetic.latent(wl["latent"], seed=wl["seed"])
    caps = synthetic.captions(wl["caption_lens"], seed=wl["seed"])
    sig, t = osm.schedule(wl["steps"], wl["shift"])
    t0 = np.full(lat.shape[0], np.float32(t[0]), dtype=np.float64)
    start = time.time()
    peaks = []
    out0 = om.forward(cfg, W, lat, caps, t0, ffn_peak=peaks)
    secs = {"step0": time.time() - start}
    print(f"step 0: {secs['step0']:.1f} s, w2 output peak {max(peaks):.4g}", flush=True)
    nb = len(peaks) // lat.shape[0]
    meta = {"workload": name, "latent": list(wl["latent"]), "caption_lens": list(wl["caption_lens"]),
            "steps": wl["steps"], "shift": wl["shift"], "outlier_log2": wl["outlier_log2"], "seed": wl["seed"],
            "t0": float(np.float32(t[0])), "stored_as": "float16 (ffn_peak float64)",
            "ffn_peak_max": max(peaks)}
    arrays = {"out0": out0.astype(np.float16), "ffn_peak": np.array(peaks, np.float64).reshape(lat.shape[0], nb)}
    path = os.path.join(HERE, f"{name}_oracle_outputs.npz")
    np.savez(path, meta=np.array(json.dumps(dict(meta, seconds=secs))), **arrays)
    if loop:
        outs = []
        start = time.time()

        def model_fn(x, tt):
            if not outs:  # step 0 is the forward above
                o = out0
            else:
                o = om.forward(cfg, W, x, caps, tt)
            print(f"step {len(outs)}: {time.time() - start:.1f} s", flush=True)
            outs.append(o)
            return o

        final = osm.run(model_fn, lat, n_steps=wl["steps"], shift=wl["shift"])
        secs["loop"] = time.time() - start
        arrays["outs"] = np.stack(outs).astype(np.float16)
        arrays["final"] = final.astype(np.float16)
    meta["seconds"] = secs
    np.savez(path, meta=np.array(json.dumps(meta)), **arrays)
    print(json.dumps(meta, indent=1))


def euler_int8():
    """The int8 variant's step-0 model output of the Euler workload, added
    to the stored file of the float runs (which it leaves as they are)."""
    name = "euler_1536x640"
    path = os.path.join(HERE, f"{name}_oracle_outputs.npz")
    z = np.load(path, allow_pickle=False)
    arrays = {k: z[k] for k in z.files if k != "meta"}
    meta = json.loads(str(z["meta"]))
    wl = synthetic.WORKLOADS[name]
    cfg = ModelConfig.from_dict(wl["model"])
    W = synthetic.SyntheticWeights(manifest(cfg), seed=wl["seed"], outlier_log2=wl["outlier_log2"])
    lat = synthetic.latent(wl["latent"], seed=wl["seed"])
    caps = synthetic.captions(wl["caption_lens"], seed=wl["seed"])
    sig, t = osm.schedule(wl["steps"], wl["shift"])
    t0 = np.full(lat.shape[0], np.float32(t[0]), dtype=np.float64)
    start = time.time()
    out = om.forward(cfg, W, lat, caps, t0, quant="int8")
    secs = time.time() - start
    ref = arrays["out0"].astype(np.float64)
    cos = float(np.sum(out * ref) / np.sqrt(np.sum(out * out) * np.sum(ref * ref)))
    print(f"int8 step 0: {secs:.1f} s, cosine {cos:.7f} against the stored float output", flush=True)
    arrays["out0_int8"] = out.astype(np.float16)
    meta["int8_step0_vs_float_cosine"] = cos
    meta.setdefault("seconds", {})["step0_int8"] = secs
    np.savez(path, meta=np.array(json.dumps(meta)), **arrays)


def dit_2048():
    name = "dit_2048"
    wl = synthetic.WORKLOADS[name]
    cfg = ModelConfig.from_dict(wl["model"])
    W = synthetic.SyntheticWeights(manifest(cfg), seed=wl["seed"])
    lat = synthetic.latent(wl["latent"], seed=wl["seed"])
    caps = synthetic.captions(wl["caption_lens"], seed=wl["seed"])
    t = [float(np.float32(v)) for v in wl["t"]]
    start = time.time()
    out = om.forward(cfg, W, lat, caps, t)
    meta = {"workload": name, "latent": list(wl["latent"]), "caption_lens": list(wl["caption_lens"]), "t": t,
            "seed": wl["seed"], "stored_as": "float16", "seconds": time.time() - start}
    np.savez(os.path.join(HERE, f"{name}_oracle_outputs.npz"), float=out.astype(np.float16),
             meta=np.array(json.dumps(meta)))
    print(json.dumps(meta, indent=1))


if __name__ == "__main__":
    what = sys.argv[1] if len(sys.argv) > 1 else ""
    if what == "euler":
        euler("--loop" in sys.argv[2:])
    elif what == "euler_int8":
        euler_int8()
    elif what == "dit_2048":
        dit_2048()
    else:
        sys.exit(__doc__)
