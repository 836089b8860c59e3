"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package holds random-number generation and the conversion of the drawn
float32 values to bfloat16 storage only -- none of the layer or optimizer
arithmetic. Both the GPU library and the CPU oracle receive the identical
values it produces.
"""
from .inputs import *  # noqa: F401,F403
