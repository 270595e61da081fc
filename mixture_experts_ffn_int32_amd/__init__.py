"""MI355X-native fused MoE-FFN experts (placeholder; the API lands with the C-ABI)."""
