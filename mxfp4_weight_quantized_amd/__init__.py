"""MXFP4 weight-quantized MoE MLP for MI355X (gfx950): Python binding of the C-ABI library."""
