"""CSA/HCA compressed attention for MI355X (gfx950): Python binding package."""
