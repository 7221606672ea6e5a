"""Kimi Delta Attention forward for AMD MI355X: Python binding of libkda.

`chunk_fwd` (chunkwise prefill over packed sequences) and `decode_step`
(batched T=1 step) call the HIP kernels in libkda.so through its C ABI
(include/kda.h). Importing the package fails if the library is not built.
"""
from .kda import (KDAError, Workspace, check_cu_seqlens, chunk_fwd, decode_step, version,
                  workspace_size, LIB_PATH)

__all__ = ["KDAError", "Workspace", "check_cu_seqlens", "chunk_fwd", "decode_step", "version",
           "workspace_size", "LIB_PATH"]
