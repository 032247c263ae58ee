"""ARL2 hybrid attention step for MI355X (gfx950).

The compute path is the C-ABI library ``libarl2.so`` (hand-written HIP
kernels); ``hybrid_linear_memory_amd.arl2`` is its thin ctypes binding and
``hybrid_linear_memory_amd.synth`` the seeded input generator. Importing the
package itself loads nothing native.
"""
