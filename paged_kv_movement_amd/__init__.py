"""MI355X-native paged <-> chunk KV-cache movement (binding over libkvmove.so)."""
