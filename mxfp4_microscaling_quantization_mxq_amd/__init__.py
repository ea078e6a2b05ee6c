"""MXFP4 / NVFP4 microscaling on AMD MI355X (gfx950): Python binding."""
