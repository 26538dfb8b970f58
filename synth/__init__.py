"""Seeded synthetic workloads shared by the oracle-side tests and the HIP-path tests."""
