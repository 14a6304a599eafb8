"""MI355X-native chunkwise retention / causal linear attention (placeholder)."""
