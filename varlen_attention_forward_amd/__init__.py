"""MI355X-native fused variable-length attention forward (placeholder, binding follows)."""
