"""GEMM parity through the C ABI: the bf16 MFMA projection against the plain
float64 product of the same bf16 values (a library matmul), at shapes that
span several tiles with ragged M tails, every epilogue, and the full-size
projection shapes of the 1024x1024 forward."""

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


def _dev_bf16(a):
    torch = _torch()
    bits = synthetic.bf16_bits(a)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = synthetic.bf16_round(rng.standard_normal((M, K), dtype=np.float32))
    W = synthetic.bf16_round(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.05))
    return A, W


@pytest.mark.parametrize("M,N,K", [(300, 256, 320), (1, 512, 64), (257, 128, 2560), (1000, 768, 128),
                                   (64, 64, 3840), (4608, 3840, 3840)])
def test_gemm_bf16_out(M, N, K):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    A, W = _operands(M, N, K, M + N + K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    binding.gemm_bf16(_dev_bf16(A), _dev_bf16(W), C, binding.EPI_BF16)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy()
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    assert helpers.rel_l2(got, ref) <= 4e-3
    assert np.max(np.abs(got - ref)) <= 8e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("n_steps", [2, 3, 4, 6, 7, 8, 12, 13, 19])
def test_gemm_k_step_counts(n_steps):
    """Every count of 64-wide K-steps around the kernel's six-step groups
    (W rotates through three LDS buffers, A through two): a lone first step,
    zero to three full groups, and tails of one to five steps, each against
    the float64 product with the fp32 epilogue's tight bar."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    M, N, K = 300, 256, 64 * n_steps
    A, W = _operands(M, N, K, 11 * n_steps)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemm_bf16(_dev_bf16(A), _dev_bf16(W), C, binding.EPI_F32_BIAS)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    assert helpers.rel_l2(got, ref) <= 2e-5


@pytest.mark.parametrize("M,N,K", [(257, 64, 3840), (4096, 3840, 64), (33, 256, 2560)])
def test_gemm_f32_bias(M, N, K):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    A, W = _operands(M, N, K, 7 * M + N)
    bias = np.random.default_rng(1).standard_normal(N).astype(np.float32)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemm_bf16(_dev_bf16(A), _dev_bf16(W), C, binding.EPI_F32_BIAS, bias=torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = A.astype(np.float64) @ W.astype(np.float64).T + bias
    assert helpers.rel_l2(got, ref) <= 2e-5


@pytest.mark.parametrize("M,F,K", [(513, 256, 256), (4608, 10240, 3840)])
def test_gemm_swiglu(M, F, K):
    """w1/w3 interleaved in 32-row groups; output silu(h w1^T) * (h w3^T)."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    rng = np.random.default_rng(M + F)
    h = synthetic.bf16_round(rng.standard_normal((M, K), dtype=np.float32))
    w1 = synthetic.bf16_round(rng.standard_normal((F, K), dtype=np.float32) * np.float32(0.03))
    w3 = synthetic.bf16_round(rng.standard_normal((F, K), dtype=np.float32) * np.float32(0.03))
    w13 = np.empty((2 * F, K), np.float32)
    for g in range(F // 32):
        w13[64 * g: 64 * g + 32] = w1[32 * g: 32 * g + 32]
        w13[64 * g + 32: 64 * g + 64] = w3[32 * g: 32 * g + 32]
    C = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    binding.gemm_bf16(_dev_bf16(h), _dev_bf16(w13), C, binding.EPI_SWIGLU)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy()
    h64 = h.astype(np.float64)
    ref = om.silu(h64 @ w1.astype(np.float64).T) * (h64 @ w3.astype(np.float64).T)
    assert helpers.rel_l2(got, ref) <= 5e-3


@pytest.mark.parametrize("epi", ["bf16", "swiglu"])
def test_gemm_strided_output_leaves_other_columns(epi):
    """Row stride ldc > output width, ragged M: only the output columns of the
    M rows change (bf16 tiles are written as whole-row 16-byte runs)."""
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    M, N, K = 300, 512, 256
    A, W = _operands(M, N, K, 11)
    width = N // 2 if epi == "swiglu" else N
    buf = torch.full((M + 8, width + 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    C = buf[:M, :width]
    binding.gemm_bf16(_dev_bf16(A), _dev_bf16(W), C, binding.EPI_SWIGLU if epi == "swiglu" else binding.EPI_BF16)
    torch.cuda.synchronize()
    out = buf.float().cpu().numpy()
    assert np.isnan(out[:, width:]).all() and np.isnan(out[M:]).all()
    got = out[:M, :width]
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    if epi == "swiglu":  # rows of W interleaved in groups of 32: (w1 block, w3 block)
        idx = np.arange(N).reshape(-1, 64)
        ref = om.silu(ref[:, idx[:, :32].ravel()]) * ref[:, idx[:, 32:].ravel()]
    assert helpers.rel_l2(got, ref) <= 5e-3


def test_gemm_rejects_bad_shapes():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    A = torch.zeros((16, 100), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.ZimgError) as ei:
        binding.gemm_bf16(A, W, C)
    assert ei.value.code == binding.ZIMG_EINVAL and "multiple of 64" in str(ei.value)
    A = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    Cw = torch.zeros((16, 70), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.ZimgError) as ei:
        binding.gemm_bf16(A, W, Cw[:, :64])
    assert ei.value.code == binding.ZIMG_EINVAL and "ldc" in str(ei.value)
    # the binding's own checks: output dtype of the epilogue, K agreement, output shape
    with pytest.raises(ValueError, match="dtype"):
        binding.gemm_bf16(A, W, torch.zeros((16, 64), device="cuda"), binding.EPI_BF16)
    with pytest.raises(ValueError, match="disagree on K"):
        binding.gemm_bf16(A, torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda"), C)
    with pytest.raises(ValueError, match="must be"):
        binding.gemm_bf16(A, W, C, binding.EPI_SWIGLU)
    # a row stride past 2^22 elements is refused before any launch (the
    # pointers are never dereferenced)
    with pytest.raises(binding.ZimgError) as ei:
        binding._check(binding.lib().zimg_gemm_bf16(binding._ptr(A), (1 << 22) + 8, binding._ptr(W), 64,
                                                     binding._ptr(C), 64, 16, 64, 64, binding.EPI_BF16, None, None))
    assert ei.value.code == binding.ZIMG_EINVAL and "at most 4194304" in str(ei.value)
