"""ZHA (Zyphra Hierarchical Attention) decode hot path for MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of ``include/zha.h``
(``libzha.so``); ``hierarchical_tree_indexed_03_amd.zha`` is the ctypes binding.
Build with ``python -m hierarchical_tree_indexed_03_amd.build_lib``.
"""
