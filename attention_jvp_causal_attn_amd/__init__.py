"""MI355X (gfx950) forward-mode JVP of masked scaled-dot-product attention."""
