"""Kimi Delta Attention forward for AMD MI355X: Python binding of libkda.

`short_conv` (the q/k/v front end: causal depthwise short conv + SiLU),
`chunk_fwd` (chunkwise prefill over packed sequences), `decode_step` (batched
T=1 step, optionally with the output epilogue fused) and `output_norm_gate`
(the output epilogue: per-head RMS norm and sigmoid gate), `backward` (the
training backward of the recurrence) and `recurrent_fwd` (the forward for head
sizes other than 128) call the HIP kernels (`stream_copy` is the streaming copy the
benchmark measures the achievable HBM rate with)
in libkda.so through its C ABI (include/kda.h). Importing the package fails if
the library is not built.
"""
from .kda import (KDAError, Workspace, backward, backward_workspace_size, check_cu_seqlens,
                  chunk_fwd, decode_step,
                  output_norm_gate, recurrent_fwd, short_conv, stream_copy, version,
                  workspace_size, LIB_PATH, NORM_EPS)

__all__ = ["KDAError", "Workspace", "backward", "backward_workspace_size", "check_cu_seqlens", "chunk_fwd", "decode_step",
           "output_norm_gate", "recurrent_fwd", "short_conv", "stream_copy", "version", "workspace_size", "LIB_PATH", "NORM_EPS"]
