"""SepLLM separator-mask attention and SepCache decode for MI355X (gfx950)."""
