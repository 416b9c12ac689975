"""MI355X-native Momentum DeltaNet hot path (placeholder; binding added with the C-ABI)."""
