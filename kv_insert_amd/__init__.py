"""libqkvfront: the decode-batch attention front on MI355X (gfx950)."""
