"""MI355X (gfx950) lossless block speculative-decoding step: HIP kernels behind a C ABI
(include/dflash.h), loaded through a thin ctypes binding (``binding``) with the same names.

The binding is imported lazily so that ``python -m speculative_decoding_dflash_amd.build`` can
rebuild the library without loading the old one; importing any dflash_* name loads it and fails
loudly if it has not been built.
"""


def __getattr__(name):
    if name.startswith("dflash_") or name == "DflashError":
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
