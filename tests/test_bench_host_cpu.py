"""bench.py's host logic, without a GPU: HBM traffic is taken from a committed
counter summary only while that summary's source digest matches the kernel
sources as they stand, and the digest follows every byte of those sources."""

import os
import shutil

import pytest

import bench


def _summary(tmp_root, kernel, digest, traffic="1.25e+09"):
    os.makedirs(os.path.join(tmp_root, "profiles"), exist_ok=True)
    with open(os.path.join(tmp_root, "profiles", f"{kernel}_dit_1024_pmc.md"), "w") as f:
        f.write(f"# counters\n\ntraffic_bytes_per_launch: {traffic}\nkernel_source_digest: {digest}\n")


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources in a scratch root that bench.py reads."""
    src = os.path.join(bench.ROOT, "diffusion_transformer_image_amd", "csrc")
    dst = os.path.join(tmp_path, "diffusion_transformer_image_amd", "csrc")
    os.makedirs(dst)
    for f in ("gemm.hip", "attention.hip", "norm.hip", "common.h"):
        shutil.copy(os.path.join(src, f), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return str(tmp_path)


def test_traffic_used_only_with_matching_digest(tree):
    k = "gemm_w13_swiglu"
    _summary(tree, k, bench.source_digest(k))
    assert bench.committed_traffic(k, "dit_1024") == 1.25e9
    _summary(tree, k, "0" * 16)
    assert bench.committed_traffic(k, "dit_1024") is None
    os.remove(os.path.join(tree, "profiles", f"{k}_dit_1024_pmc.md"))
    assert bench.committed_traffic(k, "dit_1024") is None


@pytest.mark.parametrize("edited,changes", [("gemm.hip", True), ("common.h", True), ("attention.hip", False)])
def test_digest_follows_the_kernel_sources(tree, edited, changes):
    """A one-byte edit (an appended newline) of the GEMM source or the shared header
    invalidates the GEMM counters; an edit of another kernel's file does not."""
    k = "gemm_w13_swiglu"
    before = bench.source_digest(k)
    with open(os.path.join(tree, "diffusion_transformer_image_amd", "csrc", edited), "a") as f:
        f.write("\n")
    assert (bench.source_digest(k) != before) == changes

