"""An engine created from safetensors files (zimg_dit_create_from_safetensors,
one file and two shards of mixed fp32 / bf16 tensors written by the
safetensors library) gives bitwise the forward of an engine given the same
weights in memory; a failed load leaves nothing allocated."""

import os

import numpy as np
import pytest

import synthetic
from tests import helpers

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_forward_from_safetensors_equals_in_memory_weights(tmp_path):
    torch = _torch()
    st = pytest.importorskip("safetensors.torch")
    from diffusion_transformer_image_amd import binding
    wl = synthetic.WORKLOADS["tiny_block"]
    cfg = helpers.engine_config(wl["model"], max_batch=1, max_image_tokens=256, max_caption_tokens=32)
    W = helpers.engine_weights(cfg)
    T = {n: torch.from_numpy(np.ascontiguousarray(W[n])).to(torch.bfloat16) for n in W}
    one = str(tmp_path / "model.safetensors")
    st.save_file(T, one)
    names = list(T)
    a, b = str(tmp_path / "a.safetensors"), str(tmp_path / "b.safetensors")
    st.save_file({n: T[n].float() for n in names[::2]}, a)
    st.save_file({n: T[n] for n in names[1::2]}, b)

    lat = torch.from_numpy(synthetic.latent(wl["latent"])).cuda()
    caps = torch.from_numpy(np.concatenate(synthetic.captions(wl["caption_lens"]))).cuda()
    outs = []
    for make in (lambda: binding.DiT(cfg, W.items_parallel(as_bits=True)),
                 lambda: binding.DiT.from_safetensors(cfg, one),
                 lambda: binding.DiT.from_safetensors(cfg, [a, b])):
        dit = make()
        o = torch.empty_like(lat)
        dit.forward(lat, caps, wl["caption_lens"], wl["t"], o)
        torch.cuda.synchronize()
        outs.append(o.cpu())
        dit.close()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])

    # a broken shard fails before anything is uploaded
    st.save_file({n: T[n] for n in names[1:]}, a)
    with pytest.raises(binding.ZimgError) as ei:
        binding.DiT.from_safetensors(cfg, a)
    assert ei.value.code == binding.ZIMG_EWEIGHT and "missing" in str(ei.value)
    os.remove(a)
