"""Block-causal masked-diffusion denoising step for AMD Instinct MI355X (gfx950).

The computation lives in a C-ABI shared library built from hand-written HIP
kernels (``csrc/``, declared in ``include/bc.h``).  ``binding`` loads it and
exposes the same entry points to Python with argument marshalling only;
``decode`` drives the calls through whole decode schedules; ``synth`` makes
seeded synthetic inputs.  PyTorch provides device memory and streams.

Importing the package does not load the library; ``binding.lib()`` does, and
raises if the library was not built.
"""

__all__ = ["binding", "synth", "decode"]
