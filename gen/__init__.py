"""Seeded synthetic inputs shared by the oracle tests and the HIP path (no FFN arithmetic)."""
from .layers import CONFIGS, LayerConfig, make_layer, make_hidden, bias_for_density, f32_to_bf16_bits, bf16_bits_to_f32, density_threshold  # noqa: F401
