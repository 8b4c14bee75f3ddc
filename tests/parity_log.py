"""Parity figures recorded by the tests: (workload, tensor, max-abs-rel,
tolerance); tests/conftest.py prints them in the terminal summary."""
PARITY = []
