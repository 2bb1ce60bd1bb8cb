"""Seeded synthetic inputs: the one module both the HIP path (tests, bench)
and the CPU oracle draw their inputs from.

It holds none of the method's arithmetic: only random draws, rounding to
bfloat16-representable values, and the workload recipes (sizes, seeds,
timesteps).  Tensor names and shapes are passed in by the caller (the oracle
has its own manifest, the engine exports its own), so this module needs
neither.

Recipe (the pages give no weights or data; [AIT] "Latent space" and
"Architecture" give the shapes):
  * every tensor has its own generator, seeded by (seed, stream tag, name
    bytes), so any tensor can be drawn alone, in any order, in parallel;
  * weights of linear layers, biases and pad tokens ~ N(0, 0.02^2);
  * RMSNorm weights (names containing "norm", and the caption-embedder norm
    "cap_embedder.0.weight") ~ U(0.5, 1.5): positive, near 1, and different
    per channel so that a misplaced norm weight changes the result;
  * latents and caption features ~ N(0, 1);
  * every value is rounded to the nearest bfloat16 (ties to even) and kept
    as float32, so the bf16 engine sees exactly the values the oracle sees;
  * outlier injection (heavy-tailed FFN outputs): in every block, the rows
    of feed_forward.w2.weight for 4 seeded output channels are multiplied by
    2**k; powers of two keep the bf16 values exact.
"""

import os
from collections.abc import Mapping
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import WORKLOADS  # noqa: F401  (re-export)

_WEIGHT_STREAM = 1
_LATENT_STREAM = 2
_CAPTION_STREAM = 3
_OUTLIER_STREAM = 4


def _rng(seed, stream, tag=b""):
    return np.random.default_rng(np.random.SeedSequence([int(seed), stream, *tag]))


def bf16_bits(a):
    """float32 array -> uint16 bfloat16 bit patterns (round to nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a):
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bits_to_f32(bf16_bits(a))


def is_norm_weight(name):
    return ("norm" in name and name.endswith(".weight")) or name == "cap_embedder.0.weight"


def draw_tensor(name, shape, seed):
    """One weight tensor as float32 holding bf16-representable values."""
    rng = _rng(seed, _WEIGHT_STREAM, name.encode())
    n = int(np.prod(shape))
    if is_norm_weight(name):
        a = rng.uniform(0.5, 1.5, size=n).astype(np.float32)
    else:
        a = rng.standard_normal(n, dtype=np.float32)
        a *= np.float32(0.02)
    return bf16_round(a).reshape(shape)


def outlier_channels(prefix, n_out, seed, count=4):
    """The seeded output channels of one block's w2 that get scaled."""
    rng = _rng(seed, _OUTLIER_STREAM, prefix.encode())
    return np.sort(rng.choice(n_out, size=count, replace=False))


class SyntheticWeights(Mapping):
    """Lazy mapping name -> float32 tensor, drawn on every access.

    ``outlier_log2`` (int or None): scale exponent of the outlier injection
    applied to every "*.feed_forward.w2.weight".
    """

    def __init__(self, manifest, seed=0, outlier_log2=None):
        self._shapes = {n: tuple(s) for n, s in manifest}
        self._order = [n for n, _ in manifest]
        self.seed = seed
        self.outlier_log2 = outlier_log2

    def __getitem__(self, name):
        a = draw_tensor(name, self._shapes[name], self.seed)
        if self.outlier_log2 is not None and name.endswith(".feed_forward.w2.weight"):
            prefix = name[: -len(".feed_forward.w2.weight")]
            ch = outlier_channels(prefix, a.shape[0], self.seed)
            a[ch, :] *= np.float32(2.0 ** self.outlier_log2)
        return a

    def __iter__(self):
        return iter(self._order)

    def __len__(self):
        return len(self._order)

    def materialize(self, workers=None):
        return dict(self.items_parallel(workers))

    def items_parallel(self, workers=None, as_bits=False):
        """Yield (name, array) in manifest order, drawing ahead on threads.

        With ``as_bits`` the arrays are uint16 bf16 bit patterns.
        """
        workers = workers or min(16, os.cpu_count() or 1)

        def job(name):
            a = self[name]
            return bf16_bits(a) if as_bits else a

        with ThreadPoolExecutor(workers) as ex:
            pending = []
            it = iter(self._order)
            for name in it:
                pending.append((name, ex.submit(job, name)))
                if len(pending) >= 2 * workers:
                    break
            for name in it:
                n0, f0 = pending.pop(0)
                yield n0, f0.result()
                pending.append((name, ex.submit(job, name)))
            for n0, f0 in pending:
                yield n0, f0.result()


def latent(shape, seed=0):
    """Latent [B, 16, Hl, Wl] ~ N(0, 1), bf16-representable float32."""
    rng = _rng(seed, _LATENT_STREAM)
    return bf16_round(rng.standard_normal(int(np.prod(shape)), dtype=np.float32)).reshape(shape)


def captions(lengths, dim=2560, seed=0):
    """List of caption feature arrays [L_b, dim] ~ N(0, 1), bf16-representable."""
    out = []
    for b, L in enumerate(lengths):
        rng = _rng(seed, _CAPTION_STREAM, bytes([b]))
        out.append(bf16_round(rng.standard_normal(L * dim, dtype=np.float32)).reshape(L, dim))
    return out


def residual(shape, seed=0, tag=b"residual"):
    """A seeded fp32 residual-stream stand-in ~ N(0, 1) for single-block tests."""
    rng = _rng(seed, 5, tag)
    return rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)


def modulation_input(n, dim=256, seed=0, tag=b"c"):
    """A seeded conditioning vector stand-in for single-kernel tests."""
    rng = _rng(seed, 6, tag)
    return rng.standard_normal(n * dim, dtype=np.float32).reshape(n, dim)
