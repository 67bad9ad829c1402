"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package draws random bytes and numbers only; it computes no part of the MoE layer.
"""
from .inputs import *  # noqa: F401,F403
