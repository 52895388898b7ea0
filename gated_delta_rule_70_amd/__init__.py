"""Gated delta rule on MI355X."""
