"""MI355X-native per-rank attention for context-parallel diffusion transformers."""
