"""Seeded synthetic workloads (random draws and shapes only)."""
