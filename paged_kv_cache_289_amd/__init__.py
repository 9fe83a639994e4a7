"""MI355X-native paged decode attention.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libpagedattn.so``, declared in ``include/paged_attn.h``); the Python
binding in :mod:`paged_kv_cache_289_amd.ops` only marshals torch tensors into
pointers and a stream.  Importing this package loads nothing; importing
``ops`` loads the library and fails loudly if it has not been built.
"""
