"""MI355X (gfx950) hot path of one GPU's share of a Conflux Parallelism layer step.

The compute runs in ``libxp.so`` (HIP kernels behind the C ABI of
``include/xp.h``); this package is its Python binding.  Importing the package
does not load the library; the first call does, and fails loudly if the library
has not been built.
"""
from ._lib import *  # noqa: F401,F403
from .layer import ChunkedStep, LayerStep, StackStep, batch_desc, layer_shape, layer_weights  # noqa: F401
