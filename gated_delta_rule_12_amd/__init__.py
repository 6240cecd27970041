"""MI355X-native chunkwise gated delta rule forward (gfx950 HIP kernels)."""
