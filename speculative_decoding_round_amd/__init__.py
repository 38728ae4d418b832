"""MI355X (gfx950) EAGLE-3 draft-tree + tree-verification hot path.

The compute lives in the HIP library libeagle3.so (built from csrc/); `capi` is the thin
ctypes binding over its C-ABI.  Importing this package does not load the library; the
first call through `capi` does, and fails loudly if it is missing.
"""
