"""MI355X-native product-VQ KV-cache hot path (encode, decode, attention from codes)."""
