"""Write the oracle's outputs of the 1024x1024 forward (4,096 image tokens,
512-token caption, t = 0.5, seeded synthetic weights and inputs) for the
float64 forward and for the int8-projection variant, as float16 arrays in
dit_1024_oracle_outputs.npz next to this file.

Calls only oracle/ and the seeded input generators (synthetic/).  Takes a
few minutes per forward on a multi-core host:

    python tests/golden/make_dit_1024_outputs.py
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

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dit_1024_oracle_outputs.npz")


def main():
    wl = synthetic.WORKLOADS["dit_1024"]
    cfg = ModelConfig.from_dict(wl["model"])
    W = synthetic.SyntheticWeights(manifest(cfg), seed=wl["seed"])
    lat = synthetic.latent(wl["latent"], seed=wl["seed"])
    caps = synthetic.captions(wl["caption_lens"], seed=wl["seed"])
    t = [float(np.float32(v)) for v in wl["t"]]
    outs, secs = {}, {}
    for quant in (None, "int8"):
        t0 = time.time()
        outs[quant] = om.forward(cfg, W, lat, caps, t, quant=quant)
        secs[quant] = time.time() - t0
        print(f"quant={quant}: {secs[quant]:.1f} s", flush=True)
    f, q = outs[None].ravel(), outs["int8"].ravel()
    meta = {"workload": "dit_1024", "latent": list(wl["latent"]), "caption_lens": list(wl["caption_lens"]),
            "t": t, "seed": wl["seed"], "stored_as": "float16",
            "int8_vs_float_cosine": float(f @ q / (np.linalg.norm(f) * np.linalg.norm(q))),
            "int8_vs_float_rel_l2": float(np.linalg.norm(q - f) / np.linalg.norm(f)),
            "seconds": {str(k): v for k, v in secs.items()}}
    np.savez(OUT, float=outs[None].astype(np.float16), int8=outs["int8"].astype(np.float16),
             meta=np.array(json.dumps(meta)))
    print(json.dumps(meta, indent=1))


if __name__ == "__main__":
    main()
