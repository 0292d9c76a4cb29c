"""MI355X (gfx950) fused attention: Python binding of the libfa C ABI."""
