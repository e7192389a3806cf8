"""Chunked prefill of recurrent sequence mixers on MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI declared in
``include/lrc.h`` (library ``liblrc.so``).  ``linear_recurrence_chunked_amd.lrc``
is the thin ctypes binding; ``linear_recurrence_chunked_amd.inputs`` holds the
seeded synthetic input generators.  Importing the package itself loads
nothing; importing ``lrc`` loads the HIP library and raises if it is missing.
"""

__all__ = ["lrc", "inputs"]
