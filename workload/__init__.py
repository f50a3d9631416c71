"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark (no model arithmetic)."""
