"""MI355X-native FlashCart hot path: Cartesian edge convolution (+VJP,
VJP-of-VJP) and node-local correlation ladder as a C-ABI HIP library for
gfx950 (``libflashcart.so``), with a thin ctypes binding (``flashcart``).

Importing the package loads nothing; ``flashcart.lib()`` loads the library
on first use and raises if it has not been built.
"""

__all__ = ["flashcart", "inputs", "build"]
