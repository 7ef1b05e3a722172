"""MI355X-native CosmoFlow-style 3D-CNN training step.

The computation lives in libcf.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/cf.h); ``cnn_cosmology_volumes_amd.cf`` is its ctypes
binding and ``configs`` holds the network descriptions and work counters.
"""
from . import configs  # noqa: F401
