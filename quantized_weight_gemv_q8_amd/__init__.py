"""MI355X-native Q8_0 weight-only GEMV for LLM decode (HIP, gfx950)."""
