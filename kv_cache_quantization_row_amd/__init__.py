"""MI355X-native KV-cache quantization: symmetric q8/q6/q4 paged storage, KIVI, KVQuant-style NUQ."""
