"""Seeded synthetic inputs shared by the oracle's tests and the HIP path's tests.

This package only draws and lays out inputs (activations, weights, cached K/V
pages, page tables, peer stand-in buffers, decode context lengths, waterfill
decode state).  It holds none of the layer's or the dispatcher's arithmetic.
"""
from .workloads import *  # noqa: F401,F403
