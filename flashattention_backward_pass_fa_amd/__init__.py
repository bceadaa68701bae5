"""FlashAttention backward pass for AMD MI355X (gfx950), hand-written HIP.

The compute lives in the C-ABI library libfa.so (include/fa.h); this package
is its thin Python binding.  Importing the package does not load the library;
the first call into `binding` does, and fails loudly if it is not built.
"""
