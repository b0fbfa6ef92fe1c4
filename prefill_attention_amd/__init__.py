"""MI355X-native causal prefill flash-attention (gfx950 HIP kernel behind a C ABI)."""
