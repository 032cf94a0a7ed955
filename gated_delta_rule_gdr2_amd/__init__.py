"""MI355X-native Gated Delta Rule-2 operator (placeholder; binding added with the HIP library)."""
