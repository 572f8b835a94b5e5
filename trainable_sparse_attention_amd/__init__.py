"""MI355X-native Qwen Sparse Attention (QSA) hot path.

The compute lives in the HIP library ``lib/libqsa.so`` (C ABI declared in
``include/qsa.h``).  ``trainable_sparse_attention_amd.qsa`` is a thin ctypes
binding with the same entry-point names; it only marshals arguments.
Submodules are imported explicitly (``from trainable_sparse_attention_amd
import qsa, inputs``).
"""
