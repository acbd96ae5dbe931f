"""gated_delta_rule_decay_amd: the gated delta rule-2 (GDN-2) token mixer on MI355X.

The compute path is a HIP library for gfx950 (``libgdn2.so``, C ABI declared
in ``include/gdn2.h``): a chunkwise-parallel forward and an O(1)-memory
recurrent decode step, plus the chunkwise backward, both also over packed
sequences.  ``chunk_fwd``, ``chunk_fwd_static`` (no allocation: the
library's static scratch), ``chunk_fwd_varlen``, ``chunk_bwd``,
``chunk_bwd_varlen`` and ``recurrent_step`` below only
marshal torch tensors into that ABI; importing this package does not load
the library, calling either function does (and fails loudly if it is not
built).
"""
from .binding import (chunk_fwd, chunk_fwd_static, chunk_fwd_varlen, chunk_bwd, chunk_bwd_varlen, recurrent_step,  # noqa: F401
                      chunk_fwd_workspace, chunk_fwd_varlen_workspace, chunk_bwd_workspace,
                      chunk_bwd_varlen_workspace, library_path, abi_version)

__all__ = ["chunk_fwd", "chunk_fwd_static", "chunk_fwd_varlen", "chunk_bwd", "chunk_bwd_varlen", "recurrent_step",
           "chunk_fwd_workspace", "chunk_fwd_varlen_workspace", "chunk_bwd_workspace",
           "chunk_bwd_varlen_workspace", "library_path", "abi_version"]
