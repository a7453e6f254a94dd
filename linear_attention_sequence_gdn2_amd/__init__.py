"""MI355X-native Gated DeltaNet-2 chunkwise operator (placeholder; binding follows)."""
