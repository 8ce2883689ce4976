"""KV-cache block checksums on MI355X (gfx950)."""
