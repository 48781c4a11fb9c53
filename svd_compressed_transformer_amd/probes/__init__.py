"""Measurement probes built beside the library (standalone executables, not part of its ABI)."""
