"""Seeded input generators for the tests, the oracle's stored expected values
and the benchmark (not part of the library: it holds no step of the method)."""
