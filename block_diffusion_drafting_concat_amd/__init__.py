"""MI355X (gfx950) implementation of the DFlash draft-proposal path.

The compute lives in a C-ABI shared library of hand-written HIP kernels (csrc/, declared in
include/dflash.h). `binding` is a thin ctypes layer over it, and `synth` draws the seeded
synthetic inputs. Importing the package loads nothing; `binding.lib()` loads the library and
raises if it has not been built.
"""
