"""MI355X-native speculative-decoding verify step.

The compute path is the HIP library ``libspec.so`` (``csrc/``) behind the C ABI declared
in ``include/spec.h``; ``binding`` is a thin ctypes layer over it (argument marshalling
only).  ``synth`` draws the seeded synthetic inputs.  Importing this package loads
nothing; ``binding.lib()`` loads the library and raises if it is missing.
"""
