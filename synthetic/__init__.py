"""Seeded synthetic input generators shared by tests, smoke and bench."""
