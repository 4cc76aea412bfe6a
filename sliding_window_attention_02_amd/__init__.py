"""MI355X-native SWA(w,s) attention: prefill and ring-buffer decode (HIP kernels for gfx950)."""
