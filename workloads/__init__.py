"""Seeded synthetic inputs for the CSA hot path (shared by the tests, the oracle checks and the bench).

Holds encoders and random draws only; no part of the method's arithmetic lives here.
"""
from . import codec, configs  # noqa: F401
