"""Batch-1 weight-streaming GEMV for LLM decode on MI355X (gfx950).

The compute path is the HIP library ``libwsgemv.so`` behind a C ABI
(``include/wsgemv.h``); ``wsgemv`` is its thin ctypes binding.  ``synth``
draws the seeded synthetic inputs.  Importing this package loads nothing:
the library is opened on first use, and a missing library is an error.
"""
__all__ = ["synth", "wsgemv"]
