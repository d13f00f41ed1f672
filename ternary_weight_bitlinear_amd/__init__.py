"""W1.58A8 BitLinear on MI355X (gfx950): Python binding of the C-ABI library."""
