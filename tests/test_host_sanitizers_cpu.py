"""The host side of the C ABI (engine.cpp, loader.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only: the
sanitizer flags are given to the host compilation alone) into a small
driver, tests/native/host_checks.cpp, which runs the host entry points:
configuration checks, the weight table and its digest, position ids, RoPE
tables, row layouts, the flow-match schedule, safetensors validation of
well-formed and broken files, and the allocation path (which fails cleanly
without a GPU).  Any sanitizer report fails the test."""

import json
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PKG = os.path.join(ROOT, "diffusion_transformer_image_amd")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build(tmp):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    objs = []
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    for src in ("engine.cpp", "loader.cpp"):
        o = os.path.join(tmp, src + ".o")
        subprocess.run([HIPCC] + common + SAN + ["-c", os.path.join(PKG, "csrc", src), "-o", o], check=True,
                       capture_output=True)
        objs.append(o)
    # the device kernels' objects are not instrumented (their host stubs only launch)
    for src in ("gemm.hip", "norm.hip", "attention.hip", "misc.hip"):
        pre = os.path.join(ROOT, "_build", src + ".o")
        if not os.path.exists(pre):
            pytest.skip("library objects not built (python -m diffusion_transformer_image_amd.build)")
        objs.append(pre)
    main_o = os.path.join(tmp, "host_checks.o")
    subprocess.run([HIPCC] + common + SAN + ["-c", os.path.join(ROOT, "tests", "native", "host_checks.cpp"), "-o",
                                             main_o], check=True, capture_output=True)
    drv = os.path.join(tmp, "host_checks")
    p = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + [main_o] + objs + ["-o", drv], capture_output=True,
                       text=True)
    assert p.returncode == 0, p.stderr[-3000:]
    return drv


def _files(tmp):
    """(expected code, path) pairs: the full tiny-model table written by the
    safetensors library, and hand-made broken files."""
    torch = pytest.importorskip("torch")
    st = pytest.importorskip("safetensors.torch")
    import synthetic
    from diffusion_transformer_image_amd import binding
    from tests import helpers
    wl = synthetic.WORKLOADS["tiny_block"]
    cfg = helpers.engine_config(wl["model"], max_batch=1, max_image_tokens=256, max_caption_tokens=32)
    W = synthetic.SyntheticWeights(binding.manifest(cfg), seed=0)
    good = os.path.join(tmp, "good.safetensors")
    st.save_file({n: torch.from_numpy(np.ascontiguousarray(W[n])).to(torch.bfloat16) for n in W}, good)
    out = [(binding.ZIMG_OK, good)]

    def raw(name, header, data=b"", hlen=None):
        p = os.path.join(tmp, name)
        h = header if isinstance(header, bytes) else json.dumps(header).encode()
        with open(p, "wb") as f:
            f.write(struct.pack("<Q", len(h) if hlen is None else hlen) + h + data)
        return p

    out.append((binding.ZIMG_EWEIGHT, raw("trunc.safetensors", b'{"a": {"dtype": "F32", "shape": [2', b"")))
    out.append((binding.ZIMG_EWEIGHT, raw("deep.safetensors", b"[" * 200 + b"]" * 200)))
    out.append((binding.ZIMG_EWEIGHT, raw("escape.safetensors", b'{"\\ud800x": 1}')))
    out.append((binding.ZIMG_EWEIGHT, raw("hlen.safetensors", {"a": 1}, hlen=1 << 62)))
    out.append((binding.ZIMG_EWEIGHT, raw("offs.safetensors",
                                          {"cap_embedder.0.weight": {"dtype": "F32", "shape": [2560],
                                                                     "data_offsets": [0, 99999999999999999]}})))
    out.append((binding.ZIMG_EUNSUPPORTED, raw("dtype.safetensors",
                                               {"cap_embedder.0.weight": {"dtype": "I8", "shape": [2560],
                                                                          "data_offsets": [0, 2560]}},
                                               b"\0" * 2560)))
    out.append((binding.ZIMG_EINVAL, os.path.join(tmp, "absent.safetensors")))
    return out


def test_host_entry_points_under_sanitizers(tmp_path):
    if shutil.which("llvm-symbolizer") is None and not os.path.exists("/opt/rocm/llvm/bin/llvm-symbolizer"):
        pass  # reports are still produced, only less readable
    drv = _build(str(tmp_path))
    args = ["tiny"]
    for code, path in _files(str(tmp_path)):
        args += [str(code), path]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               ASAN_SYMBOLIZER_PATH="/opt/rocm/llvm/bin/llvm-symbolizer")
    p = subprocess.run([drv] + args, capture_output=True, text=True, env=env, timeout=600)
    report = p.stdout + p.stderr
    assert p.returncode == 0, report[-4000:]
    assert "host checks: all passed" in p.stdout, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
