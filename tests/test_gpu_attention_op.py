"""The attention op (zimg_attention) on caller buffers against the oracle's
attention, per sample, through the C ABI: small mixed segments, the
1024x1024 joint geometry (30 heads over 4,608 rows, where the last round of
work is split along keys) and the batch-2 geometry of the 1536x640 Euler
workload; with the full workspace and with one that only holds the work
list (no split)."""

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


def make_inputs(rows, H, S_pad, seed):
    """bf16-representable q | k | v rows (N(0, 1)) and the transposed v."""
    D = H * 128
    qkv = synthetic.bf16_round(synthetic.residual((rows, 3 * D), seed=seed, tag=b"attention op"))
    vT = np.zeros((D, S_pad), np.float32)
    vT[:, :rows] = qkv[:, 2 * D:].T
    return qkv, vT


def oracle_rows(qkv, H, seg_b, qrows):
    """om.attention for the queries ``qrows`` (indexes into the sample's
    rows) of one sample whose rows are the union of its two ranges."""
    D = H * 128
    rows = np.concatenate([np.arange(seg_b[0], seg_b[0] + seg_b[1]), np.arange(seg_b[2], seg_b[2] + seg_b[3])])
    x = qkv[rows].astype(np.float64)
    q = x[qrows, :D].reshape(-1, H, 128)
    k = x[:, D:2 * D].reshape(-1, H, 128)
    v = x[:, 2 * D:].reshape(-1, H, 128)
    return rows[qrows], om.attention(q, k, v).reshape(-1, D)


def run_op(qkv, vT, H, seg, small_workspace=False):
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    to_bf16 = lambda a: torch.from_numpy(synthetic.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    qkv_d, vT_d = to_bf16(qkv), to_bf16(vT)
    out = torch.zeros((qkv.shape[0], H * 128), dtype=torch.bfloat16, device="cuda")
    ws = None
    if small_workspace:
        ws = torch.empty(1024 + 16 * 4096 + 256, dtype=torch.uint8, device="cuda")
        off = (-ws.data_ptr()) % 256
        ws = ws[off:off + 1024 + 16 * 4096]
    binding.attention(qkv_d, vT_d, out, H, seg, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def check(got, qkv, H, seg, n_sample=None, seed=0):
    rng = np.random.default_rng(seed)
    worst_r = worst_row = 0.0
    for b, sg in enumerate(seg):
        n = sg[1] + sg[3]
        qrows = np.arange(n) if n_sample is None or n <= n_sample else \
            np.unique(np.concatenate([[0, n - 1, sg[1] - 1, min(sg[1], n - 1)], rng.choice(n, n_sample, replace=False)]))
        rows, want = oracle_rows(qkv, H, sg, qrows)
        r, _ = helpers.assert_parity(got[rows], want, f"sample {b} attention")
        rw = float(helpers.row_rel_l2(got[rows], want).max())
        assert rw <= 3e-2, f"sample {b}: worst row rel-L2 {rw:.3e}"
        worst_r, worst_row = max(worst_r, r), max(worst_row, rw)
    return worst_r, worst_row


@pytest.mark.parametrize("small_workspace", [False, True])
def test_attention_op_mixed_segments(small_workspace):
    H, S_pad = 4, 448
    seg = [(0, 120, 128, 77), (208, 5, 216, 0), (224, 64, 288, 65)]
    qkv, vT = make_inputs(360, H, S_pad, seed=1)
    got = run_op(qkv, vT, H, seg, small_workspace)
    r, rw = check(got, qkv, H, seg)
    # rows no segment covers stay untouched
    covered = np.zeros(360, bool)
    for a, n, c, m in seg:
        covered[a:a + n] = True
        covered[c:c + m] = True
    assert np.all(got[~covered] == 0)
    print(f"rel-L2 {r:.2e}, worst row {rw:.2e}")


def test_attention_op_joint_1024_split():
    from diffusion_transformer_image_amd import binding
    H, N, L = 30, 4096, 512
    S_pad = N + L + 64
    seg = [(0, N, N, L)]
    qkv, vT = make_inputs(N + L, H, S_pad, seed=2)
    # the last round of 1080 (q-tile, head) pairs is split: the plan needs partials
    assert binding.attention_workspace_size(H, seg, S_pad) > 1024 + 16 * 36 + 256
    got = run_op(qkv, vT, H, seg)
    r, rw = check(got, qkv, H, seg, n_sample=48, seed=3)
    got_nosplit = run_op(qkv, vT, H, seg, small_workspace=True)
    check(got_nosplit, qkv, H, seg, n_sample=48, seed=3)
    d = helpers.rel_l2(got, got_nosplit)
    print(f"rel-L2 {r:.2e}, worst row {rw:.2e}; split vs whole {d:.2e}")
    assert d <= 2e-3


def test_attention_op_euler_geometry():
    from diffusion_transformer_image_amd import binding
    H, n_img, lens = 30, 3840, [77, 300]
    img_off, cap_off, S = binding.row_layout(2, n_img, lens)
    S_pad = (S + 63) // 64 * 64 + 64
    seg = [(int(img_off[b]), n_img, int(cap_off[b]), lens[b]) for b in range(2)]
    qkv, vT = make_inputs(S, H, S_pad, seed=4)
    got = run_op(qkv, vT, H, seg)
    r, rw = check(got, qkv, H, seg, n_sample=40, seed=5)
    print(f"rel-L2 {r:.2e}, worst row {rw:.2e}")


def test_attention_op_argument_errors():
    torch = _torch()
    from diffusion_transformer_image_amd import binding
    H = 2
    qkv = torch.zeros((64, 3 * H * 128), dtype=torch.bfloat16, device="cuda")
    vT = torch.zeros((H * 128, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((64, H * 128), dtype=torch.bfloat16, device="cuda")
    for seg, msg in [([(4, 10, 0, 0)], "multiple of 8"), ([(0, 0, 8, 8)], "first range is empty"),
                     ([(64, 64, 0, 0)], "rows of qkv")]:
        with pytest.raises((binding.ZimgError, ValueError), match=msg):
            binding.attention(qkv, vT, out, H, seg)
    big = torch.zeros((256, 3 * H * 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.ZimgError, match="exceed S_pad"):
        binding.attention(big, vT, torch.zeros((256, H * 128), dtype=torch.bfloat16, device="cuda"), H,
                          [(80, 60, 0, 0)])
