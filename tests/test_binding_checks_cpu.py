"""The Python binding refuses, before any native call, tensors its entry
points cannot read: tensors that are not on the GPU, of another dtype or
rank, or without unit-stride rows.  Runs on the CPU: every case fails in the
binding's own checks."""

import pytest

torch = pytest.importorskip("torch")

from diffusion_transformer_image_amd import binding  # noqa: E402


def test_host_tensors_are_refused():
    A = torch.zeros((256, 64), dtype=torch.bfloat16)
    W = torch.zeros((256, 64), dtype=torch.bfloat16)
    C = torch.zeros((256, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        binding.gemm_bf16(A, W, C)
    with pytest.raises(ValueError, match="CUDA"):
        binding.euler_step(torch.zeros(8), torch.zeros(8), 0.1)
    with pytest.raises(ValueError, match="CUDA"):
        binding.quantize_rows(torch.zeros((4, 128)), torch.zeros((4, 128), dtype=torch.int8), torch.zeros(4))


def test_wrong_dtypes_are_refused():
    with pytest.raises(ValueError, match="fp32 or bf16"):
        binding.quantize_rows(torch.zeros((4, 128), dtype=torch.float64), torch.zeros((4, 128), dtype=torch.int8),
                              torch.zeros(4))


def test_want_rules():
    """The rule set itself, on tensors that only claim to be on the GPU."""

    class FakeCuda(torch.Tensor):
        @property
        def is_cuda(self):
            return True

    def fake(t):
        return t.as_subclass(FakeCuda)

    ok = fake(torch.zeros((4, 8)))
    binding._want(ok, "x", (torch.float32,), 2, contiguous=True)
    with pytest.raises(ValueError, match="dtype"):
        binding._want(ok, "x", (torch.bfloat16,))
    with pytest.raises(ValueError, match="2-d"):
        binding._want(fake(torch.zeros(8)), "x", (torch.float32,), 2)
    with pytest.raises(ValueError, match="unit-stride"):
        binding._want(fake(torch.zeros((8, 4)).t()), "x", (torch.float32,), 2)
    with pytest.raises(ValueError, match="contiguous"):
        binding._want(fake(torch.zeros((4, 16))[:, :8]), "x", (torch.float32,), 2, contiguous=True)
    # a row-sliced view (unit-stride rows, larger leading stride) is accepted without ``contiguous``
    binding._want(fake(torch.zeros((4, 16))[:, :8]), "x", (torch.float32,), 2)
