"""Piecewise (exact-or-approximate) block-sparse attention on MI355X."""
