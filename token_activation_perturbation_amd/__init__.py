"""Dust per-token zeroth-order estimator on MI355X (placeholder; binding follows)."""
