"""Seeded synthetic inputs (shared by tests, oracle checks and the benchmark)."""
