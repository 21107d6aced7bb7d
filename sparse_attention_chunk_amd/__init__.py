"""MI355X (gfx950) implementation of the FlashMemory Memory-Indexer scoring pass.

libfm.so (HIP kernels + C ABI, include/fm.h) does the work; `_lib` is the
ctypes binding with the C entry points' names and `retriever` the README's
retriever interface on top.  Importing raises if libfm.so is not built.
"""

from . import _lib  # noqa: F401  (raises ImportError if libfm.so is missing)
from .retriever import LAYER_NAMES, FlashMemoryRetriever, weights_to_device  # noqa: F401
