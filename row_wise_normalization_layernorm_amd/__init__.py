"""MI355X-native forward row-wise normalization (LayerNorm, RMSNorm)."""
