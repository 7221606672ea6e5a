"""Thin ctypes binding over libkda (include/kda.h).

Argument marshalling only: this module checks tensor placement, dtype, shape
and contiguity, allocates outputs and the caller-owned workspace with torch,
and passes raw device pointers plus the current HIP stream to the library.
Every step of the computation runs in libkda's HIP kernels. There is no CPU
fallback: if libkda.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1

# Every symbol include/kda.h declares.
EXPORTS = ("kda_version", "kda_status_string", "kda_last_error",
           "kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_intra",
           "kda_chunk_fwd_inter", "kda_decode_step", "kda_decode_step_gated",
           "kda_decode_step_slots", "kda_output_norm_gate", "kda_short_conv",
           "kda_short_conv_slots",
           "kda_backward_workspace_size", "kda_backward", "kda_chunk_fwd_grouped",
           "kda_decode_step_grouped", "kda_backward_grouped", "kda_recurrent_fwd",
           "kda_check_cu_seqlens", "kda_chunk_fwd_noalloc", "kda_stream_copy",
           "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_workspace_size")

NORM_EPS = 1e-5   # default epsilon of the output norm (the pages give none)

if not os.path.exists(LIB_PATH):
    raise ImportError("libkda.so not found at %s: build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_lib.kda_version.restype = ctypes.c_int
_lib.kda_version.argtypes = []
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_status_string.argtypes = [ctypes.c_int]
_lib.kda_last_error.restype = ctypes.c_char_p
_lib.kda_last_error.argtypes = []
_lib.kda_chunk_fwd_workspace_size.restype = _sz
_lib.kda_chunk_fwd_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
for _name in ("kda_chunk_fwd", "kda_chunk_fwd_intra", "kda_chunk_fwd_inter"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _i64,
                                     _i32, _i32, _i32, _i32, ctypes.c_int, _P, _P, _P,
                                     ctypes.c_int, _P, _sz, _P]
_lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
_lib.kda_chunk_fwd_noalloc.argtypes = _lib.kda_chunk_fwd.argtypes[:21] + [_P]
NOALLOC_SCRATCH_BYTES = 128 << 20    # the fixed scratch of kda_chunk_fwd_noalloc
_lib.kda_chunk_fwd_gated_workspace_size.restype = _sz
_lib.kda_chunk_fwd_gated_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32,
                                                    ctypes.c_int, ctypes.c_int]
_lib.kda_chunk_fwd_gated.restype = ctypes.c_int
_lib.kda_chunk_fwd_gated.argtypes = _lib.kda_chunk_fwd.argtypes + [_P, _P, _f32]
_lib.kda_chunk_fwd_grouped.restype = ctypes.c_int
_lib.kda_chunk_fwd_grouped.argtypes = _lib.kda_chunk_fwd.argtypes + [_i32]
_STAGE_FN = {None: _lib.kda_chunk_fwd, "intra": _lib.kda_chunk_fwd_intra,
             "inter": _lib.kda_chunk_fwd_inter}
_lib.kda_decode_step.restype = ctypes.c_int
_lib.kda_decode_step.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _P, ctypes.c_int,
                                 _i32, _i32, _i32, _i32, ctypes.c_int, _P]
_lib.kda_decode_step_gated.restype = ctypes.c_int
_lib.kda_decode_step_gated.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _P, ctypes.c_int,
                                       _i32, _i32, _i32, _i32, ctypes.c_int, _P, _P, _f32, _P]
_lib.kda_decode_step_slots.restype = ctypes.c_int
_lib.kda_decode_step_slots.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _P, _P,
                                       ctypes.c_int, _i32, _i32, _i32, _i32, ctypes.c_int, _P, _P,
                                       _f32, _P]
_lib.kda_output_norm_gate.restype = ctypes.c_int
_lib.kda_output_norm_gate.argtypes = [_P, _P, _P, _f32, _i64, _i32, ctypes.c_int, _P, _P]
_lib.kda_short_conv.restype = ctypes.c_int
_lib.kda_short_conv.argtypes = [_P, _i64, _P, _i32, _P, _i32, _i64, _i64, ctypes.c_int, _P, _P,
                                _P, _P]
_lib.kda_short_conv_slots.restype = ctypes.c_int
_lib.kda_short_conv_slots.argtypes = [_P, _i64, _P, _i32, _P, _i32, _i64, _i64, ctypes.c_int, _P,
                                      _i32, _P, _P, _P]
_lib.kda_backward_workspace_size.restype = _sz
_lib.kda_backward_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32]
_lib.kda_backward.restype = ctypes.c_int
_lib.kda_backward.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _i64, _i32, _i32,
                              _i32, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P, _P, _P, _P, _P,
                              _P, _P, _P, _P, _sz, _P]
_lib.kda_decode_step_grouped.restype = ctypes.c_int
_lib.kda_decode_step_grouped.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _P, _P,
                                         ctypes.c_int, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                         _P, _P, _f32, _P]
_lib.kda_backward_grouped.restype = ctypes.c_int
_lib.kda_backward_grouped.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _i64, _i32,
                                      _i32, _i32, _i32, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
_lib.kda_recurrent_fwd.restype = ctypes.c_int
_lib.kda_recurrent_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _i32, _i64,
                                   _i32, _i32, _i32, _i32, ctypes.c_int, _P, _P, _P,
                                   ctypes.c_int, _P]
_lib.kda_stream_copy.restype = ctypes.c_int
_lib.kda_stream_copy.argtypes = [_P, _P, _sz, _P]
_lib.kda_check_cu_seqlens.restype = ctypes.c_int
_lib.kda_check_cu_seqlens.argtypes = [_P, _i32, _i64, _P]

lib = _lib


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.kda_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, _lib.kda_status_string(status).decode(), detail))


def _check(status: int, where: str):
    if status != KDA_OK:
        raise KDAError(status, where)


def version() -> int:
    return int(_lib.kda_version())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise RuntimeError("%s must be a GPU tensor (libkda has no CPU path)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(total_tokens: int, num_seqs: int, H: int, chunk_size: int,
                   in_dtype=torch.bfloat16, K: int = 128, V: int = 128) -> int:
    d = KDA_BF16 if in_dtype == torch.bfloat16 else KDA_F32
    n = int(_lib.kda_chunk_fwd_workspace_size(int(total_tokens), int(num_seqs), int(H), int(K),
                                              int(V), int(chunk_size), d))
    if n == 0:
        raise ValueError("kda_chunk_fwd_workspace_size: " + _lib.kda_last_error().decode())
    return n


class Workspace:
    """Caller-owned device scratch for chunk_fwd, grown on demand and reused.

    Reuse is safe on one stream: every call rewrites what it reads.
    """

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else torch.device("cuda")
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        return self.buf


def chunk_fwd(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, *, scale: float = None,
              chunk_size: int = 64, lower_bound: float = -5.0,
              initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
              o_dtype=None, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[Workspace] = None,
              stage: Optional[str] = None,
              gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
              norm_eps: float = NORM_EPS) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill over packed sequences (libkda kda_chunk_fwd).

    q, k: [T, H_qk, K] and v: [T, H, V], bf16 or fp32 (same dtype); H_qk < H
    (a divisor) selects grouped value heads (kda_chunk_fwd_grouped); g: [T, H, K] fp32;
    beta_raw: [T, H] fp32; A_log: [H] fp32; dt_bias: [H, K] fp32;
    cu_seqlens: [N+1] int64 on the GPU; initial_state: [N, H, V, K] fp32 or None.
    Returns (o [T, H, V] in o_dtype (default: q's dtype), final_state or None).
    Head sizes: K = V = 128; any 1 <= K, V <= 128; and 1 <= K, V <= 256 with
    chunk_size 64 and bf16 inputs (the library rejects others with ValueError;
    recurrent_fwd takes them).
    stage: None runs both kernels; "intra" / "inter" run one stage (kda_chunk_fwd_intra /
    kda_chunk_fwd_inter), which must share the same workspace and arguments.
    With `gate` (logits [T, H, V] in q's dtype) and `norm_weight` ([V] fp32) the output
    epilogue of output_norm_gate is applied in the o store (kda_chunk_fwd_gated) and the
    returned o is its result.
    """
    T, Hqk, K = q.shape
    H, V = v.shape[1], v.shape[2]          # value heads (grouped value heads: a multiple of Hqk)
    N = cu_seqlens.numel() - 1
    in_dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    _dev(q, "q", shape=(T, Hqk, K))
    _dev(k, "k", dtype=q.dtype, shape=(T, Hqk, K))
    _dev(v, "v", dtype=q.dtype, shape=(T, H, V))
    _dev(g, "g", torch.float32, (T, H, K))
    _dev(beta_raw, "beta_raw", torch.float32, (T, H))
    _dev(A_log, "A_log", torch.float32, (H,))
    _dev(dt_bias, "dt_bias", torch.float32, (H, K))
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    device = q.device
    h0_ptr = None
    if initial_state is not None:
        h0_ptr = _dev(initial_state, "initial_state", torch.float32, (N, H, V, K))
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((T, H, V), dtype=o_dtype, device=device)
    o_ptr = _dev(out, "out", o_dtype, (T, H, V))
    ht_ptr = None
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=device)
        ht_ptr = _dev(final_state, "final_state", torch.float32, (N, H, V, K))
    else:
        final_state = None
    if gate is None:
        need = workspace_size(T, N, H, chunk_size, q.dtype, K, V)
    else:
        need = int(_lib.kda_chunk_fwd_gated_workspace_size(T, N, H, K, V, int(chunk_size), in_dt,
                                                           _dt(out)))
        if need == 0:
            raise ValueError("kda_chunk_fwd_gated_workspace_size: " +
                             _lib.kda_last_error().decode())
    ws = (workspace or Workspace(device)).get(need)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta_raw.data_ptr(),
            A_log.data_ptr(), dt_bias.data_ptr(), float(scale), float(lower_bound),
            cu_seqlens.data_ptr(), N, T, H, K, V, int(chunk_size), in_dt, h0_ptr, ht_ptr, o_ptr,
            _dt(out), ws.data_ptr(), ws.numel(), _stream_ptr(device))
    if gate is not None:
        if stage is not None or Hqk != H:
            raise ValueError("the gated prefill runs both stages without grouped heads")
        _dev(gate, "gate", q.dtype, (T, H, V))
        if norm_weight is None:
            raise ValueError("norm_weight is required with gate")
        _dev(norm_weight, "norm_weight", torch.float32, (V,))
        fn, args = _lib.kda_chunk_fwd_gated, args + (gate.data_ptr(), norm_weight.data_ptr(),
                                                     float(norm_eps))
    elif Hqk != H:
        if stage is not None:
            raise ValueError("grouped value heads run both stages (stage must be None)")
        fn, args = _lib.kda_chunk_fwd_grouped, args + (Hqk,)
    else:
        fn = _STAGE_FN[stage]
    st = fn(*args)
    _check(st, fn.__name__)
    return out, final_state


def decode_step(q, k, v, g, beta_raw, A_log, dt_bias, state, *, scale: float = None,
                lower_bound: float = -5.0, o_dtype=None,
                out: Optional[torch.Tensor] = None,
                gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                norm_eps: float = NORM_EPS,
                slot_idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One T=1 decode step for B requests; `state` [B, H, 128, 128] fp32 is updated in place.

    q, k: [B, H_qk, 128] and v: [B, H, 128], bf16 or fp32 (H_qk < H: grouped value heads,
    kda_decode_step_grouped); g: [B, H, 128] fp32; beta_raw: [B, H] fp32.
    Returns o [B, H, 128] in o_dtype (default: q's dtype). With `gate` (logits
    [B, H, 128] in q's dtype) and `norm_weight` ([128] fp32) the output epilogue
    of output_norm_gate is fused into the store (kda_decode_step_gated). With
    `slot_idx` (int32 [B] on the GPU), `state` is a pool [S, H, 128, 128] and
    request b uses entry slot_idx[b]; indices outside [0, S) mark padding
    requests (zero output, no state touched) (kda_decode_step_slots).
    Head sizes other than 128 (1 <= K, V <= 256: q, k, g [B, H, K], v [B, H, V],
    state [B, H, V, K]) run on the token-by-token kernel; slot_idx and gate are accepted
    there too (norm_weight [V]), the epilogue then applied as a second pass over o.
    """
    B, Hqk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    _dev(q, "q", shape=(B, Hqk, K))
    _dev(k, "k", dtype=q.dtype, shape=(B, Hqk, K))
    _dev(v, "v", dtype=q.dtype, shape=(B, H, V))
    _dev(g, "g", torch.float32, (B, H, K))
    _dev(beta_raw, "beta_raw", torch.float32, (B, H))
    _dev(A_log, "A_log", torch.float32, (H,))
    _dev(dt_bias, "dt_bias", torch.float32, (H, K))
    if slot_idx is None:
        _dev(state, "state", torch.float32, (B, H, V, K))
    else:
        _dev(state, "state")
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, V, K) or state.dtype != torch.float32:
            raise ValueError("state must be an fp32 pool [S, %d, %d, %d]" % (H, V, K))
        _dev(slot_idx, "slot_idx", torch.int32, (B,))
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, V), dtype=o_dtype, device=q.device)
    _dev(out, "out", o_dtype, (B, H, V))
    if Hqk != H:
        zp = wp = None
        if gate is not None:
            _dev(gate, "gate", q.dtype, (B, H, V))
            if norm_weight is None:
                raise ValueError("norm_weight is required with gate")
            _dev(norm_weight, "norm_weight", torch.float32, (V,))
            zp, wp = gate.data_ptr(), norm_weight.data_ptr()
        st = _lib.kda_decode_step_grouped(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta_raw.data_ptr(),
            A_log.data_ptr(), dt_bias.data_ptr(), float(scale), float(lower_bound),
            state.data_ptr(), int(state.shape[0]) if slot_idx is not None else 0,
            None if slot_idx is None else slot_idx.data_ptr(), out.data_ptr(), _dt(out), B, H,
            Hqk, K, V, _dt(q), zp, wp, float(norm_eps), _stream_ptr(q.device))
        _check(st, "kda_decode_step_grouped")
        return out
    if slot_idx is not None:
        zp = wp = None
        if gate is not None:
            _dev(gate, "gate", q.dtype, (B, H, V))
            if norm_weight is None:
                raise ValueError("norm_weight is required with gate")
            _dev(norm_weight, "norm_weight", torch.float32, (V,))
            zp, wp = gate.data_ptr(), norm_weight.data_ptr()
        st = _lib.kda_decode_step_slots(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                        beta_raw.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
                                        float(scale), float(lower_bound), state.data_ptr(),
                                        int(state.shape[0]), slot_idx.data_ptr(), out.data_ptr(),
                                        _dt(out), B, H, K, V, _dt(q), zp, wp, float(norm_eps),
                                        _stream_ptr(q.device))
        _check(st, "kda_decode_step_slots")
        return out
    if gate is None:
        st = _lib.kda_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                  beta_raw.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
                                  float(scale), float(lower_bound), state.data_ptr(),
                                  out.data_ptr(), _dt(out), B, H, K, V, _dt(q),
                                  _stream_ptr(q.device))
        _check(st, "kda_decode_step")
        return out
    _dev(gate, "gate", q.dtype, (B, H, V))
    if norm_weight is None:
        raise ValueError("norm_weight is required with gate")
    _dev(norm_weight, "norm_weight", torch.float32, (V,))
    st = _lib.kda_decode_step_gated(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                    beta_raw.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
                                    float(scale), float(lower_bound), state.data_ptr(),
                                    out.data_ptr(), _dt(out), B, H, K, V, _dt(q),
                                    gate.data_ptr(), norm_weight.data_ptr(), float(norm_eps),
                                    _stream_ptr(q.device))
    _check(st, "kda_decode_step_gated")
    return out


def output_norm_gate(o: torch.Tensor, gate: torch.Tensor, norm_weight: torch.Tensor, *,
                     eps: float = NORM_EPS, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Output epilogue (kda_output_norm_gate): per-row RMS norm over the last axis
    (128 features, or any width up to 256), channel weight, sigmoid gate.

    o, gate: [..., D] bf16 or fp32 (same dtype); norm_weight: [D] fp32.
    Returns y with o's shape and dtype (`out` may be `o` itself).
    """
    D = o.shape[-1]
    rows = o.numel() // D if D else 0
    _dev(o, "o")
    _dev(gate, "gate", o.dtype, tuple(o.shape))
    _dev(norm_weight, "norm_weight", torch.float32, (D,))
    if out is None:
        out = torch.empty_like(o)
    _dev(out, "out", o.dtype, tuple(o.shape))
    st = _lib.kda_output_norm_gate(o.data_ptr(), gate.data_ptr(), norm_weight.data_ptr(),
                                   float(eps), int(rows), int(D), _dt(o), out.data_ptr(),
                                   _stream_ptr(o.device))
    _check(st, "kda_output_norm_gate")
    return out


def short_conv(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor, *,
               initial_state: Optional[torch.Tensor] = None, output_final_state: bool = False,
               final_state: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, state_pool: Optional[torch.Tensor] = None,
               slot_idx: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Front end for one of q, k, v (kda_short_conv): causal depthwise short
    conv along time over packed sequences, then SiLU.

    x: [T, H, 128] or [T, C] bf16 or fp32; the token axis may be strided (a
    slice of a fused projection output), the rest must be contiguous.
    weight: [H, 128, W] or [C, W] fp32 (W <= 4). cu_seqlens: [N+1] int64 on the GPU.
    initial_state / final_state: [N, W-1, *x.shape[1:]] in x's dtype (the last
    W - 1 inputs of each sequence so far, oldest first); final_state may be
    initial_state itself. Returns (y with x's shape, contiguous; final_state or None).
    With `slot_idx` (int32 [N] on the GPU) the states live in `state_pool`
    [S, W-1, *x.shape[1:]] instead, sequence n using entry slot_idx[n], updated in
    place (kda_short_conv_slots); indices outside [0, S) mark padding sequences
    (zero outputs, no state touched). Returns (y, state_pool).
    """
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise RuntimeError("x must be a GPU tensor (libkda has no CPU path)")
    if slot_idx is not None:
        return _short_conv_slots(x, weight, cu_seqlens, state_pool, slot_idx, out)
    T = x.shape[0]
    feat = tuple(x.shape[1:])
    C = int(math.prod(feat))
    N = cu_seqlens.numel() - 1
    if x.dim() < 2 or (T > 0 and x[0].numel() > 0 and not x[0].is_contiguous()):
        raise ValueError("x must be [T, ...] with contiguous rows")
    stride = x.stride(0) if T > 1 else C
    W = weight.shape[-1]
    _dev(weight, "weight", torch.float32, feat + (W,))
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    sshape = (N, W - 1) + feat
    si = so = None
    if initial_state is not None:
        si = _dev(initial_state, "initial_state", x.dtype, sshape)
    if output_final_state or final_state is not None:
        if final_state is None:
            final_state = torch.empty(sshape, dtype=x.dtype, device=x.device)
        so = _dev(final_state, "final_state", x.dtype, sshape)
    if out is None:
        out = torch.empty((T,) + feat, dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, (T,) + feat)
    st = _lib.kda_short_conv(x.data_ptr() if T else None, int(stride), weight.data_ptr(), int(W),
                             cu_seqlens.data_ptr(), N, int(T), C, _dt(x), si, so,
                             out.data_ptr() if T else None, _stream_ptr(x.device))
    _check(st, "kda_short_conv")
    return out, final_state


def _short_conv_slots(x, weight, cu_seqlens, state_pool, slot_idx, out):
    T = x.shape[0]
    feat = tuple(x.shape[1:])
    C = int(math.prod(feat))
    N = cu_seqlens.numel() - 1
    if x.dim() < 2 or (T > 0 and x[0].numel() > 0 and not x[0].is_contiguous()):
        raise ValueError("x must be [T, ...] with contiguous rows")
    stride = x.stride(0) if T > 1 else C
    W = weight.shape[-1]
    _dev(weight, "weight", torch.float32, feat + (W,))
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    _dev(slot_idx, "slot_idx", torch.int32, (N,))
    if state_pool is None:
        raise ValueError("state_pool is required with slot_idx")
    _dev(state_pool, "state_pool", x.dtype)
    if tuple(state_pool.shape[1:]) != (W - 1,) + feat:
        raise ValueError("state_pool must be [S, %d, %s]" % (W - 1, ", ".join(map(str, feat))))
    if out is None:
        out = torch.empty((T,) + feat, dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, (T,) + feat)
    st = _lib.kda_short_conv_slots(x.data_ptr() if T else None, int(stride), weight.data_ptr(),
                                   int(W), cu_seqlens.data_ptr(), N, int(T), C, _dt(x),
                                   state_pool.data_ptr() if state_pool.numel() else None,
                                   int(state_pool.shape[0]), slot_idx.data_ptr(),
                                   out.data_ptr() if T else None, _stream_ptr(x.device))
    _check(st, "kda_short_conv_slots")
    return out, state_pool


def backward_workspace_size(total_tokens: int, num_seqs: int, H: int, K: int = 128,
                            V: int = 128) -> int:
    n = int(_lib.kda_backward_workspace_size(int(total_tokens), int(num_seqs), int(H), int(K),
                                             int(V)))
    if n == 0:
        raise ValueError("kda_backward_workspace_size: " + _lib.kda_last_error().decode())
    return n


def backward(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, d_o, *, scale: float = None,
             lower_bound: float = -5.0, initial_state: Optional[torch.Tensor] = None,
             d_final_state: Optional[torch.Tensor] = None, need_d_initial_state: bool = True,
             workspace: Optional[Workspace] = None) -> dict:
    """Training backward of the recurrence (kda_backward): gradients of
    sum(o * d_o) + sum(final_state * d_final_state) w.r.t. every input.

    Inputs as chunk_fwd (q, k may have fewer heads: grouped value heads, dq and dk then
    [T, H_qk, K]); d_o: [T, H, V] bf16 or fp32; d_final_state: [N, H, V, K]
    fp32 or None. Returns a dict of fp32 tensors dq, dk, dg [T, H, K], dv [T, H, V],
    dbeta [T, H], dA_log [H], ddt_bias [H, K] and dh0 [N, H, V, K] (None unless
    requested). K = V = 128, or head sizes up to 128 (zero-padded inside the library).
    """
    T, Hqk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    _dev(q, "q", shape=(T, Hqk, K))
    _dev(k, "k", dtype=q.dtype, shape=(T, Hqk, K))
    _dev(v, "v", dtype=q.dtype, shape=(T, H, V))
    _dev(g, "g", torch.float32, (T, H, K))
    _dev(beta_raw, "beta_raw", torch.float32, (T, H))
    _dev(A_log, "A_log", torch.float32, (H,))
    _dev(dt_bias, "dt_bias", torch.float32, (H, K))
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    _dev(d_o, "d_o", shape=(T, H, V))
    dev = q.device
    h0p = None if initial_state is None else _dev(initial_state, "initial_state", torch.float32,
                                                  (N, H, V, K))
    dhtp = None if d_final_state is None else _dev(d_final_state, "d_final_state", torch.float32,
                                                   (N, H, V, K))
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((T, Hqk, K), **f32), dk=torch.empty((T, Hqk, K), **f32),
               dv=torch.empty((T, H, V), **f32), dg=torch.empty((T, H, K), **f32),
               dbeta=torch.empty((T, H), **f32), dA_log=torch.empty((H,), **f32),
               ddt_bias=torch.empty((H, K), **f32),
               dh0=torch.empty((N, H, V, K), **f32) if need_d_initial_state else None)
    need = backward_workspace_size(T, N, H, K, V)
    ws = (workspace or Workspace(dev)).get(need)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = _lib.kda_backward_grouped(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                           beta_raw.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(), float(scale),
                           float(lower_bound), cu_seqlens.data_ptr(), N, T, H, Hqk, K, V, _dt(q), h0p,
                           d_o.data_ptr(), _dt(d_o), dhtp, out["dq"].data_ptr(),
                           out["dk"].data_ptr(), out["dv"].data_ptr(), out["dg"].data_ptr(),
                           out["dbeta"].data_ptr(), out["dA_log"].data_ptr(),
                           out["ddt_bias"].data_ptr(), ptr(out["dh0"]), ws.data_ptr(), ws.numel(),
                           _stream_ptr(dev))
    _check(st, "kda_backward_grouped")
    return out


def recurrent_fwd(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, *, scale: float = None,
                  lower_bound: float = -5.0, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, final_state: Optional[torch.Tensor] = None,
                  o_dtype=None, out: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KDA forward for any head sizes 1 <= K, V <= 256 (libkda kda_recurrent_fwd).

    q, k: [T, H_qk, K] and v: [T, H, V], bf16 or fp32 (same dtype), H_qk dividing H;
    g: [T, H, K] fp32; beta_raw: [T, H] fp32; A_log: [H]; dt_bias: [H, K];
    cu_seqlens: [N+1] int64 on the GPU; initial_state: [N, H, V, K] fp32 or None.
    final_state may be initial_state itself (updated in place): a batched decode
    step is this call with cu_seqlens = [0, 1, ..., B].
    Returns (o [T, H, V] in o_dtype (default: q's dtype), final_state or None).
    """
    T, Hqk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    _dev(q, "q", shape=(T, Hqk, K))
    _dev(k, "k", dtype=q.dtype, shape=(T, Hqk, K))
    _dev(v, "v", dtype=q.dtype, shape=(T, H, V))
    _dev(g, "g", torch.float32, (T, H, K))
    _dev(beta_raw, "beta_raw", torch.float32, (T, H))
    _dev(A_log, "A_log", torch.float32, (H,))
    _dev(dt_bias, "dt_bias", torch.float32, (H, K))
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    h0_ptr = None
    if initial_state is not None:
        h0_ptr = _dev(initial_state, "initial_state", torch.float32, (N, H, V, K))
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((T, H, V), dtype=o_dtype, device=q.device)
    o_ptr = _dev(out, "out", o_dtype, (T, H, V))
    ht_ptr = None
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
        ht_ptr = _dev(final_state, "final_state", torch.float32, (N, H, V, K))
    else:
        final_state = None
    st = _lib.kda_recurrent_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                beta_raw.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
                                float(scale), float(lower_bound), cu_seqlens.data_ptr(), N, T, H,
                                Hqk, K, V, _dt(q), h0_ptr, ht_ptr, o_ptr, _dt(out),
                                _stream_ptr(q.device))
    _check(st, "kda_recurrent_fwd")
    return out, final_state


def check_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int) -> None:
    """Validate packed offsets (synchronises the current stream); raises on bad values."""
    N = cu_seqlens.numel() - 1
    _dev(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,))
    st = _lib.kda_check_cu_seqlens(cu_seqlens.data_ptr(), N, int(total_tokens),
                                   _stream_ptr(cu_seqlens.device))
    _check(st, "kda_check_cu_seqlens")


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Copy src into dst with the library's streaming kernel (kda_stream_copy):
    the measured HBM reference of the benchmark. Both contiguous, same size in
    bytes (a multiple of 16), on the GPU."""
    _dev(src, "src")
    _dev(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(_lib.kda_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream_ptr(src.device)),
           "kda_stream_copy")
    return dst
