"""Exact per-row top-k selection for MI355X (gfx950), hand-written HIP."""
