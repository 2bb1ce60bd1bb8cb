"""The five synthetic workloads: model sizes, input shapes, timesteps, seeds.

Pure data.  Sizes come from the pages: latent 16 x H/8 x W/8 and 2x2 patches
([AIT] "Latent space": 512^2 -> 1,024 tokens, 1024^2 -> 4,096, 2048^2 ->
16,384); up to 512 caption tokens ([FV] "Pinned official pipeline context":
max_sequence_length 512); the full model of [AIT] "Architecture"; the 8-step
shift-3.0 Euler loop of [MNN] "Scheduler".
"""

FULL_MODEL = dict(hidden=3840, n_heads=30, ffn=10240, n_layers=30,
                  n_noise_refiner=2, n_context_refiner=2)

WORKLOADS = {
    # tiny single block: hidden 512 (4 heads), FFN 1536, 32 caption + 256 image tokens
    "tiny_block": dict(
        model=dict(hidden=512, n_heads=4, ffn=1536, n_layers=1,
                   n_noise_refiner=0, n_context_refiner=0),
        latent=(1, 16, 32, 32), caption_lens=(32,), t=(0.5,), seed=0),
    # one full-width block at 512x512: 128 caption + 1024 image tokens
    "block_512": dict(
        model=dict(FULL_MODEL, n_layers=1, n_noise_refiner=0, n_context_refiner=0),
        latent=(1, 16, 64, 64), caption_lens=(128,), t=(0.75,), seed=0),
    # the full 34-block forward at 1024x1024: 512 caption + 4096 image tokens
    "dit_1024": dict(
        model=dict(FULL_MODEL),
        latent=(1, 16, 128, 128), caption_lens=(512,), t=(0.5,), seed=0),
    # attention-dominated 2048x2048: 512 caption + 16,384 image tokens
    "dit_2048": dict(
        model=dict(FULL_MODEL),
        latent=(1, 16, 256, 256), caption_lens=(512,), t=(0.5,), seed=0),
    # 8-step Euler loop at 1536x640, batch 2, captions of 77 and 300 tokens,
    # w2 outliers scaled by 2**16 (|w2 output| peaks in (5e5, 1e6])
    "euler_1536x640": dict(
        model=dict(FULL_MODEL),
        latent=(2, 16, 192, 80), caption_lens=(77, 300), t=None, seed=0,
        steps=8, shift=3.0, outlier_log2=16),
}
