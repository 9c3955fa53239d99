"""Measurement tools run by bench.py (not part of the library)."""
