"""Seeded synthetic input generators shared by the oracle side and the GPU side."""
