"""The C-ABI library on a host without a GPU: it loads, exports every
declared symbol, validates configs and arguments before touching HIP, and
its host-built tables match the oracle's bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import ModelConfig, manifest as oracle_manifest
from oracle import model as om
from oracle import sampler as osm
import synthetic
from tests import helpers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "diffusion_transformer_image_amd", "libzimg_dit.so")),
    reason="libzimg_dit.so not built")


def _b():
    from diffusion_transformer_image_amd import binding
    return binding


def _declared_functions():
    names = set()
    for h in ("zimg_dit.h", "zimg_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**\s*(zimg_[a-z0-9_]+)\s*\(", src, re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 19
    L = ctypes.CDLL(_b().LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing
    # and the binding declares a signature for each
    assert names <= set(_b().SIGNATURES), names - set(_b().SIGNATURES)


@pytest.mark.parametrize("wl", ["tiny_block", "block_512", "dit_1024"])
def test_engine_manifest_equals_oracle_manifest(wl):
    model = synthetic.WORKLOADS[wl]["model"]
    eng = _b().manifest(helpers.engine_config(model))
    ora = [(n, tuple(s)) for n, s in oracle_manifest(ModelConfig.from_dict(model))]
    assert eng == ora


def test_full_manifest_counts():
    eng = _b().manifest(_b().config())
    assert len(eng) == 521
    assert sum(int(np.prod(s)) for _, s in eng) == 6_154_908_736


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 3712, "EUNSUPPORTED"),        # != n_heads * 128
    ("max_caption_tokens", 513, "EUNSUPPORTED"),
    ("max_caption_tokens", 0, "EUNSUPPORTED"),
    ("max_batch", 0, "EINVAL"),
    ("ffn", 100, "EUNSUPPORTED"),
    ("rope_axes", (32, 48, 40), "EUNSUPPORTED"),
    ("norm_eps", 0.0, "EINVAL"),
    ("batch_invariant", 2, "EINVAL"),
    ("linear_int8", -1, "EINVAL"),
    ("token_pad", 16, "EUNSUPPORTED"),
    ("check_finite", 2, "EINVAL"),
])
def test_config_validation(field, value, code):
    b = _b()
    cfg = b.config(**{field: value})
    with pytest.raises(b.ZimgError) as ei:
        b.check_config(cfg)
    assert ei.value.code == getattr(b, "ZIMG_" + code)
    assert str(ei.value)


def test_default_config_is_valid():
    b = _b()
    b.check_config(b.config())
    d = b.config().as_dict()
    assert d["hidden"] == 3840 and d["n_heads"] == 30 and d["ffn"] == 10240
    assert d["rope_axes"] == (32, 48, 48) and d["rope_theta"] == 256.0


def test_alloc_without_gpu_fails_with_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    b = _b()
    cfg = helpers.engine_config(synthetic.WORKLOADS["tiny_block"]["model"])
    h = ctypes.c_void_p()
    rc = b.lib().zimg_dit_alloc(ctypes.byref(cfg), None, ctypes.byref(h))
    assert rc == b.ZIMG_EHIP and not h.value
    assert "HIP device" in b.lib().zimg_last_error().decode()


def test_position_ids_equal_oracle():
    for L, Hp, Wp in [(1, 1, 1), (77, 96, 40), (512, 64, 64)]:
        ec, ei = _b().position_ids(L, Hp, Wp)
        oc, oi = om.position_ids(L, Hp, Wp)
        assert np.array_equal(ec, oc) and np.array_equal(ei, oi)


@pytest.mark.parametrize("L,Hp,Wp", [(32, 16, 16), (512, 64, 64), (300, 96, 40)])
def test_rope_tables_bit_exact_vs_oracle(L, Hp, Wp):
    cap, img = om.position_ids(L, Hp, Wp)
    ids = np.concatenate([img, cap])
    ec, es = _b().rope_tables(_b().config(), ids)
    oc, os_ = om.rope_tables(ModelConfig(), ids)
    assert ec.view(np.uint32).tolist() == oc.view(np.uint32).tolist()
    assert es.view(np.uint32).tolist() == os_.view(np.uint32).tolist()


def test_row_layout():
    img, cap, S = _b().row_layout(2, 3840, [77, 300])
    assert img.tolist() == [0, 3840]
    assert cap.tolist() == [7680, 7680 + 80]
    assert S == 7680 + 80 + 304
    img, cap, S = _b().row_layout(1, 4096, [512])
    assert img.tolist() == [0] and cap.tolist() == [4096] and S == 4608
    img, cap, S = _b().row_layout(3, 600, [1, 16, 17])
    assert img.tolist() == [0, 608, 1216] and cap.tolist() == [1824, 1840, 1856] and S == 1888
    with pytest.raises(_b().ZimgError):
        _b().row_layout(1, 16, [0])


def test_row_layout_varsize():
    """Per-sample image counts: 120 -> 128 rows, 6 -> 16, 17 -> 32 (image rows
    of all samples first), then captions 77 -> 80, 1 -> 16, 33 -> 48."""
    img, cap, S = _b().row_layout_varsize([120, 6, 17], [77, 1, 33])
    assert img.tolist() == [0, 128, 144]
    assert cap.tolist() == [176, 256, 272] and S == 320
    # equal counts give the uniform layout
    for n, lens in ((3840, [77, 300]), (600, [1, 16, 17])):
        assert [a.tolist() if hasattr(a, "tolist") else a for a in _b().row_layout_varsize([n] * len(lens), lens)] == \
            [a.tolist() if hasattr(a, "tolist") else a for a in _b().row_layout(len(lens), n, lens)]
    with pytest.raises(_b().ZimgError):
        _b().row_layout_varsize([16, 0], [1, 1])


def test_sampler_schedule_equals_oracle():
    """zimg_flowmatch_schedule (through sampler.schedule) equals the oracle's
    float64 schedule bit for bit, for step counts 1..60 and several shifts."""
    from diffusion_transformer_image_amd import sampler
    for n in list(range(1, 61)) + [1000]:
        for s in (1.0, 3.0, 6.0, 2.5):
            es, et = sampler.schedule(n, s)
            os_, ot = osm.schedule(n, s)
            assert es.view(np.uint64).tolist() == os_.view(np.uint64).tolist(), (n, s)
            assert et.view(np.uint64).tolist() == ot.view(np.uint64).tolist(), (n, s)


def test_flowmatch_schedule_against_exact_fractions(golden):
    """The 8-step shift-3 schedule against the hand-derived fractions: each
    shifted sigma is one correctly rounded division of exactly representable
    values, so it is the nearest double of the fraction, bit for bit; t and
    the increments are within one rounding of theirs."""
    from fractions import Fraction
    g = golden["sampler_schedule"]
    sig, t = _b().flowmatch_schedule(g["n_steps"], g["shift"])
    assert [float(Fraction(v)) for v in g["sigma_shifted"]] == sig.tolist()
    for got, want in zip(t, g["t"]):
        assert abs(got - float(Fraction(want))) <= 2e-16
    for k, want in enumerate(g["dt"]):
        assert abs((sig[k + 1] - sig[k]) - float(Fraction(want))) <= 4e-16


@pytest.mark.parametrize("n,shift", [(0, 3.0), (-2, 3.0), (8, 0.0), (8, float("nan")), (8, -1.0)])
def test_flowmatch_schedule_rejects_bad_arguments(n, shift):
    with pytest.raises(_b().ZimgError) as ei:
        _b().flowmatch_schedule(n, shift)
    assert ei.value.code == _b().ZIMG_EINVAL


def test_missing_library_fails_loudly(monkeypatch):
    from diffusion_transformer_image_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libzimg_dit.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()
