"""MI355X-native (gfx950) BF16 encoder forward pass.

The compute path is the HIP library ``liblaya_encoder.so`` (kernels in
``csrc/``, C ABI in ``include/laya_encoder.h``); ``binding`` is its ctypes
binding and ``inputs`` the seeded synthetic workload generator.  Importing
the package loads nothing; ``binding.load()`` loads the library and fails
loudly if it has not been built.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "binding"]
