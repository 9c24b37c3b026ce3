"""libxattn: plan/run paged attention on MI355X (gfx950)."""
