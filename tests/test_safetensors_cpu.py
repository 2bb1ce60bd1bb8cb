"""Strict safetensors ingestion (zimg_safetensors_check; no GPU needed) on
files written by the safetensors library itself and on hand-made broken
ones, and the sorted-key digest of the weight table against the one the
FastVideo handoff prints for the released checkpoint ("Local component
coverage and quality handoff for the zimage FastVideo port", Component
contracts: loading accounts for every parameter, auxiliary tensors are not
ignored; 521 keys with the stated digest)."""

import hashlib
import json
import os
import struct

import numpy as np
import pytest

import synthetic
from tests import helpers

torch = pytest.importorskip("torch")
st = pytest.importorskip("safetensors.torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "diffusion_transformer_image_amd", "libzimg_dit.so")),
    reason="libzimg_dit.so not built")


def _b():
    from diffusion_transformer_image_amd import binding
    return binding


def _tiny():
    wl = synthetic.WORKLOADS["tiny_block"]
    return helpers.engine_config(wl["model"], max_batch=1, max_image_tokens=256, max_caption_tokens=32)


def _tensors(cfg, dtype=torch.bfloat16):
    W = synthetic.SyntheticWeights(_b().manifest(cfg), seed=0)
    return {n: torch.from_numpy(np.ascontiguousarray(W[n])).to(dtype) for n in W}


def _raw_file(path, entries, data=b"", header_len=None, meta=None):
    """A safetensors file from explicit header entries (for broken cases)."""
    hdr = dict(entries)
    if meta is not None:
        hdr["__metadata__"] = meta
    h = json.dumps(hdr).encode()
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(h) if header_len is None else header_len))
        f.write(h)
        f.write(data)
    return path


def _expect(code, match, cfg, paths):
    b = _b()
    with pytest.raises(b.ZimgError) as ei:
        b.safetensors_check(cfg, paths)
    assert ei.value.code == getattr(b, "ZIMG_" + code), str(ei.value)
    assert match in str(ei.value), str(ei.value)


def test_library_written_files_pass(tmp_path):
    cfg = _tiny()
    T = _tensors(cfg)
    one = str(tmp_path / "model.safetensors")
    st.save_file(T, one, metadata={"format": "pt", "note": "synthetic é"})
    assert _b().safetensors_check(cfg, one) == len(T)
    # sharded: two files, fp32 in one and bf16 in the other
    names = list(T)
    a, b = str(tmp_path / "a.safetensors"), str(tmp_path / "b.safetensors")
    st.save_file({n: T[n].float() for n in names[::2]}, a)
    st.save_file({n: T[n] for n in names[1::2]}, b)
    assert _b().safetensors_check(cfg, [a, b]) == len(T)


def test_missing_extra_duplicate_misshaped(tmp_path):
    cfg = _tiny()
    T = _tensors(cfg)
    names = list(T)
    p = str(tmp_path / "x.safetensors")
    st.save_file({n: T[n] for n in names[1:]}, p)
    _expect("EWEIGHT", "missing: " + names[0], cfg, p)
    # an auxiliary tensor the table does not hold is refused, not ignored
    st.save_file(dict(T, **{"layers.0.attention.to_q.scale_weight": torch.ones(1)}), p)
    _expect("EWEIGHT", "unknown tensor 'layers.0.attention.to_q.scale_weight'", cfg, p)
    a, b = str(tmp_path / "a.safetensors"), str(tmp_path / "b.safetensors")
    st.save_file(T, a)
    st.save_file({names[5]: T[names[5]]}, b)
    _expect("EWEIGHT", f"duplicate tensor '{names[5]}'", cfg, [a, b])
    bad = dict(T)
    bad["all_x_embedder.2-1.weight"] = T["all_x_embedder.2-1.weight"][:, :32].contiguous()
    st.save_file(bad, p)
    _expect("EWEIGHT", "'all_x_embedder.2-1.weight' has the wrong shape", cfg, p)


def test_unsupported_dtype(tmp_path):
    cfg = _tiny()
    T = _tensors(cfg)
    T["cap_embedder.0.weight"] = T["cap_embedder.0.weight"].to(torch.float16)
    p = str(tmp_path / "x.safetensors")
    st.save_file(T, p)
    _expect("EUNSUPPORTED", "dtype F16", cfg, p)


def test_broken_files(tmp_path):
    cfg = _tiny()
    name, shape = _b().manifest(cfg)[4]  # cap_embedder.0.weight, a vector
    n = int(np.prod(shape))
    good = {name: {"dtype": "F32", "shape": list(shape), "data_offsets": [0, 4 * n]}}
    data = np.ones(n, np.float32).tobytes()
    p = str(tmp_path / "x.safetensors")
    # the entry itself is fine: only the other tensors are missing
    _raw_file(p, good, data)
    _expect("EWEIGHT", "missing", cfg, p)
    _raw_file(p, {name: dict(good[name], data_offsets=[0, 4 * n + 4])}, data)
    _expect("EWEIGHT", "data_offsets outside", cfg, p)
    _raw_file(p, {name: dict(good[name], data_offsets=[4, 4 * n])}, data)
    _expect("EWEIGHT", "the shape needs", cfg, p)
    _raw_file(p, {name: dict(good[name], shape=[n, -1])}, data)
    _expect("EWEIGHT", "bad dimension", cfg, p)
    _raw_file(p, {name: {"dtype": "F32", "shape": list(shape)}}, data)
    _expect("EWEIGHT", "data_offsets [begin, end] are required", cfg, p)
    _raw_file(p, {name: dict(good[name], extra=1)}, data)
    _expect("EWEIGHT", "unknown field 'extra'", cfg, p)
    _raw_file(p, good, data, meta={"format": 1})
    _expect("EWEIGHT", "not a string", cfg, p)
    _raw_file(p, good, data, header_len=1 << 40)
    _expect("EWEIGHT", "header length", cfg, p)
    with open(p, "wb") as f:
        f.write(struct.pack("<Q", 9) + b'{"a": [1,')
    _expect("EWEIGHT", str(p), cfg, p)
    with open(p, "wb") as f:
        f.write(b"\x01\x02")
    _expect("EWEIGHT", "shorter than its 8-byte header length", cfg, p)
    _expect("EINVAL", "cannot open", cfg, str(tmp_path / "absent.safetensors"))


def test_manifest_digest_matches_page_and_hashlib(golden):
    b = _b()
    full = b.config()
    assert b.manifest_digest(full) == golden["page_constants"]["checkpoint_key_digest"]["value"]
    cfg = _tiny()
    names = sorted(n for n, _ in b.manifest(cfg))
    assert b.manifest_digest(cfg) == hashlib.sha256("".join(n + "\n" for n in names).encode()).hexdigest()
