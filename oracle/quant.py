"""Int8 variant of the block projections: what it computes, written plainly.

Test infrastructure only (see oracle/__init__.py).

The pages' quantized transformers store the block linears in 8-bit integers
([MNN] "Conversion details": 8-bit weight quantization of the exported
model; [H3D] the int8 ConvRot transformer file), keep the embedders and the
final layer at full precision ([AIT] "Specifics": t_embedder, cap_embedder,
x_embedder and the final layer are not quantized), and report a single-step
output cosine of about 0.9996 for int8 against fp32 ([MNN] "Performance").
The pages leave the scheme open.  Reading taken here (W8A8, both operands in
int8 so that the product runs on integer matrix units):

  * every linear of a transformer block (to_q, to_k, to_v, to_out, w1, w2,
    w3) has int8 weights, one fp32 scale per output channel (row of W);
  * its input activations are quantized per token (row) at run time;
  * both are symmetric: for a row v (fp32 values) with amax = max |v|,
        scale = fp32(amax / 127),   inv = fp32(127 / amax),
        code  = clamp(rint(fp32(v * inv)), -127, 127)   (rint: half to even)
    and an all-zero row has scale 0 and codes 0 (a row holding NaN or an
    infinity has a NaN scale, so the fault stays visible downstream);
  * the product is exact in integers, acc[i, j] = sum_k qa[i, k] qw[j, k],
    and the output is acc[i, j] * sa[i] * sw[j];
  * weights are quantized from their bf16 values; the normalised block
    inputs h and h2 from their fp32 values; the attention output and the
    SwiGLU product from their bf16 values (the precision each is held in
    when it reaches the projection);
  * the SwiGLU product (w2's input) is heavy-tailed, so before it is
    quantized it is rotated, as the ConvRot quantization of [H3D] ("What was
    changed, and why": ConvRot rotates the activation) rotates activations:
    every 128 consecutive values of a row go through the unnormalised
    Walsh-Hadamard transform (the Sylvester matrix H_128, H H^T = 128 I), and
    w2's weight rows through the same transform, so the product of the two
    rotated operands is 128 times the plain one; the rotated weights'
    scales carry the 1/128 (an exact power of two).  The transform is the
    fast one in fp32: butterflies of stride 1, 2, 4, ..., 64 in that order,
    (a, b) -> (a + b, a - b).
The block's adaLN linears and the attention itself stay in floating point.
"""

import numpy as np


def to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_bf16(x):
    """Round float32 values to nearest-even bfloat16 (returned as float32)."""
    u = to_f32(x).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quantize_rows(x):
    """Symmetric per-row int8 quantization of fp32 rows (last axis).

    Returns (codes int8 [..., K], scales float32 [...]).  Arithmetic is in
    float32, as the definition above states."""
    v = to_f32(x)
    amax = np.max(np.abs(v), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(0), (safe / np.float32(127)).astype(np.float32)).astype(np.float32)
    inv = np.where(zero, np.float32(0), (np.float32(127) / safe).astype(np.float32)).astype(np.float32)
    bad = ~np.all(np.isfinite(v), axis=-1)
    scale = np.where(bad, np.float32(np.nan), scale).astype(np.float32)
    inv = np.where(bad, np.float32(0), inv).astype(np.float32)
    prod = np.nan_to_num((v * inv[..., None]).astype(np.float32))
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return codes, scale


def sylvester_hadamard(n):
    """H_1 = [1]; H_2m = [[H_m, H_m], [H_m, -H_m]] (float64)."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n
    return H


ROT_BLOCK = 128


def fwht_rows(x, n=ROT_BLOCK):
    """Fast Walsh-Hadamard transform of every n consecutive values of each
    row, in fp32: for stride h = 1, 2, ..., n/2, each pair (i, i + h) with
    bit h of i clear becomes (x_i + x_{i+h}, x_i - x_{i+h}), rounded to fp32.
    Equals x times the Sylvester matrix H_n on each block, up to rounding."""
    v = to_f32(x).copy()
    shape = v.shape
    v = v.reshape(-1, n)
    h = 1
    while h < n:
        b = v.reshape(-1, n // (2 * h), 2, h)
        lo, hi = b[:, :, 0, :].copy(), b[:, :, 1, :].copy()
        b[:, :, 0, :] = (lo + hi).astype(np.float32)
        b[:, :, 1, :] = (lo - hi).astype(np.float32)
        v = b.reshape(-1, n)
        h *= 2
    return v.reshape(shape)


def quantize_rotated_rows(x, weight=False):
    """Codes and scales of the rotated rows (the SwiGLU product, held as
    bf16, or w2's weight rows); the weight scales carry the 1/128."""
    q, s = quantize_rows(fwht_rows(x))
    if weight:
        s = (s * np.float32(1.0 / ROT_BLOCK)).astype(np.float32)
    return q, s


def int_matmul(qa, qw):
    """acc[i, j] = sum_k qa[i, k] * qw[j, k], exactly.  Computed as a
    float64 matrix product: each term is an integer of magnitude at most
    127^2 and every partial sum an integer below K * 127^2 < 2^53 for any
    K under 5.5e11, so each float64 addition is exact, whatever order the
    library sums in.  Returned as int64."""
    qa = np.asarray(qa)
    assert qa.shape[-1] * 127 * 127 < 2.0 ** 53
    acc = np.asarray(qa, dtype=np.float64) @ np.asarray(qw, dtype=np.float64).T
    return acc.astype(np.int64)


def int8_product(qa, sa, qw, sw):
    """acc * sa[i] * sw[j] in float64 (the exact integer sum, then the two
    scales)."""
    acc = int_matmul(qa, qw).astype(np.float64)
    return acc * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def int8_linear(x, w, rotate=False):
    """x [M, K] (values as held: fp32 or bf16) times W^T, W [N, K] (bf16
    values), both quantized per row; with ``rotate`` both are first rotated
    by blocks of 128 (see the module docstring)."""
    if rotate:
        qa, sa = quantize_rotated_rows(x)
        qw, sw = quantize_rotated_rows(w, weight=True)
    else:
        qa, sa = quantize_rows(x)
        qw, sw = quantize_rows(w)
    return int8_product(qa, sa, qw, sw)
