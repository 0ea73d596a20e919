"""Seeded synthetic workloads (shapes and input generators) shared by tests, smoke and bench."""
