"""libgdn: the gated delta rule on MI355X (gfx950) through a C ABI."""
