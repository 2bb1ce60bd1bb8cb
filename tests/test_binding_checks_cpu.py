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


class _FakeCuda(torch.Tensor):
    @property
    def is_cuda(self):
        return True


def _fake(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype).as_subclass(_FakeCuda)


def _handle(**model):
    """A DiT object without a native handle: every case below must be
    refused by the binding before the library is called."""
    d = binding.DiT.__new__(binding.DiT)
    d.cfg = binding.config(max_batch=4, max_image_tokens=256, max_caption_tokens=64, **model)
    d._h = None
    return d


def test_forward_shape_mismatches_are_refused():
    d = _handle()
    lat, out = _fake(2, 16, 8, 8), _fake(2, 16, 8, 8)
    caps = _fake(10, 2560)
    with pytest.raises(ValueError, match="channels"):
        d.forward(_fake(2, 8, 8, 8), caps, [4, 6], [0.5, 0.5], _fake(2, 8, 8, 8))
    with pytest.raises(ValueError, match="caption_lens"):
        d.forward(lat, caps, [10], [0.5, 0.5], out)
    with pytest.raises(ValueError, match="model times"):
        d.forward(lat, caps, [4, 6], [0.5], out)
    with pytest.raises(ValueError, match="caption_feats"):
        d.forward(lat, _fake(9, 2560), [4, 6], [0.5, 0.5], out)
    with pytest.raises(ValueError, match="caption_feats"):
        d.forward(lat, _fake(2560), [4, 6], [0.5, 0.5], out)
    with pytest.raises(ValueError, match="caption_feats"):
        d.forward(lat, _fake(10, 2048), [4, 6], [0.5, 0.5], out)


def test_forward_varsize_shape_mismatches_are_refused():
    d = _handle()
    lats = [_fake(16, 8, 8), _fake(16, 4, 6)]
    outs = [_fake(16, 8, 8), _fake(16, 4, 6)]
    caps = _fake(7, 2560)
    with pytest.raises(ValueError, match="per sample"):
        d.forward_varsize([_fake(8, 8, 8), lats[1]], caps, [3, 4], [0.1, 0.2], [_fake(8, 8, 8), outs[1]])
    with pytest.raises(ValueError, match="matching shapes"):
        d.forward_varsize(lats, caps, [3, 4], [0.1, 0.2], [outs[0], _fake(16, 4, 4)])
    with pytest.raises(ValueError, match="caption_lens"):
        d.forward_varsize(lats, caps, [7], [0.1, 0.2], outs)
    with pytest.raises(ValueError, match="model times"):
        d.forward_varsize(lats, caps, [3, 4], [0.1], outs)
    with pytest.raises(ValueError, match="caption_feats"):
        d.forward_varsize(lats, _fake(6, 2560), [3, 4], [0.1, 0.2], outs)


def test_run_blocks_residual_size_is_checked():
    d = _handle(n_layers=1, n_noise_refiner=0, n_context_refiner=0)
    # one sample, 8x8 latent -> 16 image tokens, caption of 5 -> 16 + 16 rows
    _, _, S = binding.row_layout(1, 16, [5])
    with pytest.raises(ValueError, match="values required"):
        d.run_blocks(_fake(S - 1, d.cfg.hidden), 1, 8, 8, [5], [0.5], 0, 1)
    with pytest.raises(ValueError, match="caption_lens"):
        d.run_blocks(_fake(S, d.cfg.hidden), 1, 8, 8, [5, 5], [0.5], 0, 1)
    with pytest.raises(ValueError, match="model times"):
        d.run_blocks(_fake(S, d.cfg.hidden), 1, 8, 8, [5], [], 0, 1)
    with pytest.raises(ValueError, match="multiples"):
        d.run_blocks(_fake(S, d.cfg.hidden), 1, 7, 8, [5], [0.5], 0, 1)
