"""MI355X-native CacheBlend KV-fusion step (binding over libcacheblend.so)."""
