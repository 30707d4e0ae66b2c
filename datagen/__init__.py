"""Seeded synthetic inputs shaped like video-DiT attention layers.

This package draws random numbers and builds position masks. It holds none of the
attention, clustering or counting arithmetic of the method: the GPU library and the
CPU oracle both take its arrays as inputs and nothing else from it.
"""
from .video_layers import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    get_config,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    head_tensors,
    drift_noise,
    block_mask,
    cache_init_indices,
    cache_init,
    make_layer,
    drift_layer,
)
