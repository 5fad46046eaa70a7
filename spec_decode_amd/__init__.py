"""Python binding of libkda, the gfx950 KDA gated delta-rule state-update library.

Argument marshalling only: each function passes device pointers, sizes and the
current HIP stream to the C entry point of the same name (declared in
include/kda.h) and raises on a non-zero return code. Every step of the
computation runs in the library's HIP kernels; there is no fallback path. If
libkda.so is missing the import fails.

Tensors are torch tensors on a ROCm device: BF16 data as torch.bfloat16, FP32
as torch.float32, indices as torch.int32, all contiguous.
"""
import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "kda_decay", "kda_commit", "kda_verify", "kda_fused_replay_verify",
    "kda_fused_conv_replay_verify", "kda_gate_projection",
    "kda_defer_commit", "kda_flush_plan", "kda_last_error", "kda_abi_version",
    "kda_page_rw_probe",
    "library_path", "KdaError", "KDA_STATE_F32", "KDA_STATE_BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the same library (a measurement variant,
# see build.py); by default the in-tree libkda.so.
_LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_EINVAL, KDA_ELAUNCH = 0, 1, 2
KDA_STATE_F32, KDA_STATE_BF16 = 0, 1

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc --offload-arch=gfx950) first")

_lib = ctypes.CDLL(_LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float
_u64a = ctypes.POINTER(ctypes.c_uint64)
_i64a = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_abi_version": (_i, []),
    "kda_decay": (_i, [_p, _i64, _i, _p, _p, _f, _p, _p]),
    "kda_commit": (_i, [_i, _i, _i, _i, _i, _u64a, _i64a, _u64a, _i64a, _u64a, _i64a,
                        _p, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p]),
    "kda_verify": (_i, [_i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _i64, _p, _i,
                        _p, _p, _i, _p, _p, _p, _p, _f, _p, _p]),
    "kda_fused_replay_verify": (_i, [_i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _i64,
                                     _p, _i, _p, _p, _i, _p, _p, _p, _p, _p, _p, _p, _f, _p,
                                     _p]),
    "kda_fused_conv_replay_verify": (_i, [_i, _i, _i, _p, _i64, _p, _p, _p, _i64, _i64, _i64,
                                          _f, _p, _p, _p, _p, _f, _i, _p, _i64, _p, _i, _p,
                                          _p, _i, _p, _p, _p, _p, _p, _p, _f, _p, _p]),
    "kda_gate_projection": (_i, [_i64, _i, _p, _i64, _p, _p, _p]),
    "kda_defer_commit": (_i, [_i, _p, _p, _p, _p, _p, _i, _p]),
    "kda_flush_plan": (_i, [_i, _i, _p, _p, _p, _p, _p, _p, _p, _i, _p]),
    "kda_page_rw_probe": (_i, [_i, _i, _p, _i64, _p, _i, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class KdaError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def kda_last_error() -> str:
    return _lib.kda_last_error().decode()


def kda_abi_version() -> int:
    return _lib.kda_abi_version()


def _check(rc: int) -> None:
    if rc != KDA_OK:
        raise KdaError(f"[{rc}] {kda_last_error()}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    """Device address of a contiguous device tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on a ROCm device (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    return t.data_ptr()


def _need(t: Optional[torch.Tensor], count: int, name: str) -> None:
    """Per-request device arrays are read at indices below ``count``: a shorter
    tensor would be read past its end, so reject it on the host."""
    if t is not None and isinstance(t, torch.Tensor) and t.numel() < count:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {count}")


def _ptr_rows(t: torch.Tensor, dtype, row_stride: int, name: str):
    """Device address of a row-major 2-D view whose rows are ``row_stride``
    elements apart (e.g. a column slice of a wider tensor)."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a tensor on a ROCm device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) != row_stride):
        raise TypeError(f"{name} must be 2-D with unit column stride and row stride "
                        f"{row_stride}")
    return t.data_ptr()


def _stream(stream, ref: Optional[torch.Tensor]) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    dev = ref.device if ref is not None else None
    return torch.cuda.current_stream(dev).cuda_stream


def kda_decay(raw_g: torch.Tensor, a_log: torch.Tensor, dt_bias: torch.Tensor,
              lower_bound: float, out: torch.Tensor, stream=None) -> torch.Tensor:
    """out[i,h,c] = exp(lb * sigmoid(exp(a_log[h]) * (raw_g[i,h,c] + dt_bias[h,c])))."""
    tokens, heads = raw_g.shape[0], raw_g.shape[1]
    _check(_lib.kda_decay(_ptr(raw_g, torch.bfloat16, "raw_g"), tokens, heads,
                          _ptr(a_log, torch.float32, "a_log"),
                          _ptr(dt_bias, torch.float32, "dt_bias"), float(lower_bound),
                          _ptr(out, torch.float32, "out"), _stream(stream, raw_g)))
    return out


def _table(values, ctype):
    arr = (ctype * len(values))(*[int(v) for v in values])
    return arr


def kda_commit(*, heads: int, window: int, batch: int, state_dtype: int,
               state_addrs: Sequence[int], state_slot_strides: Sequence[int],
               corr_addrs: Sequence[int], corr_row_strides: Sequence[int],
               kg_addrs: Sequence[int], kg_row_strides: Sequence[int],
               a_log: torch.Tensor, dt_bias: torch.Tensor, sources: torch.Tensor,
               commit_lens: torch.Tensor, destinations: torch.Tensor,
               boundaries: Optional[torch.Tensor] = None,
               boundary_lens: Optional[torch.Tensor] = None,
               record_rows: Optional[torch.Tensor] = None, lower_bound: float,
               null_slot: int = 0, stream=None) -> None:
    """RecoverSSM commit over L layers. ``*_addrs`` are per-layer device base
    addresses (``tensor.data_ptr()``), strides in elements."""
    L = len(state_addrs)
    if not (len(state_slot_strides) == len(corr_addrs) == len(corr_row_strides)
            == len(kg_addrs) == len(kg_row_strides) == L):
        raise ValueError("per-layer tables must all have one entry per layer")
    st, sst = _table(state_addrs, ctypes.c_uint64), _table(state_slot_strides, ctypes.c_int64)
    ca, cst = _table(corr_addrs, ctypes.c_uint64), _table(corr_row_strides, ctypes.c_int64)
    ka, kst = _table(kg_addrs, ctypes.c_uint64), _table(kg_row_strides, ctypes.c_int64)
    i32 = torch.int32
    for t, name in ((sources, "sources"), (commit_lens, "commit_lens"),
                    (destinations, "destinations"), (boundaries, "boundaries"),
                    (boundary_lens, "boundary_lens"), (record_rows, "record_rows")):
        _need(t, batch, name)
    _check(_lib.kda_commit(
        L, heads, window, batch, state_dtype, st, sst, ca, cst, ka, kst,
        _ptr(a_log, torch.float32, "a_log"), _ptr(dt_bias, torch.float32, "dt_bias"),
        _ptr(sources, i32, "sources"), _ptr(commit_lens, i32, "commit_lens"),
        _ptr(destinations, i32, "destinations"), _ptr(boundaries, i32, "boundaries"),
        _ptr(boundary_lens, i32, "boundary_lens"), _ptr(record_rows, i32, "record_rows"),
        float(lower_bound), int(null_slot), _stream(stream, sources)))


def _verify_args(q, k, v, raw_g, raw_beta, a_log, dt_bias, state, state_indices, corr, kg,
                 record_rows, out):
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    return (_ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"), _ptr(raw_g, bf, "raw_g"),
            _ptr(raw_beta, bf, "raw_beta"), _ptr(a_log, f32, "a_log"),
            _ptr(dt_bias, f32, "dt_bias"), _ptr(state, None, "state"),
            _ptr(state_indices, i32, "state_indices"), _ptr(corr, f32, "corr"),
            _ptr(kg, bf, "kg"), _ptr(record_rows, i32, "record_rows"), _ptr(out, bf, "out"))


def _state_dtype(state) -> int:
    """KDA_STATE_F32 for a float32 pool, KDA_STATE_BF16 for a bfloat16 one."""
    if state.dtype == torch.float32:
        return KDA_STATE_F32
    if state.dtype == torch.bfloat16:
        return KDA_STATE_BF16
    raise TypeError(f"state must be float32 or bfloat16 (got {state.dtype})")


def _gate_args(gate, norm_weight):
    return (_ptr(gate, torch.bfloat16, "gate"), _ptr(norm_weight, torch.float32, "norm_weight"))


def kda_verify(*, heads: int, tokens: int, batch: int, q, k, v, raw_g, raw_beta, a_log,
               dt_bias, lower_bound: float, state, state_slot_stride: int, state_indices,
               corr, kg, record_tokens: int, out, record_rows=None, null_slot: int = 0,
               gate=None, norm_weight=None, norm_eps: float = 1e-5, query_start_loc=None,
               stream=None):
    """Stock verify: writes out (o, or its gated RMSNorm with gate and
    norm_weight) and the records, never the state. The pool's element type
    (float32 or bfloat16) is that of ``state``."""
    _need(state_indices, batch, "state_indices")
    _need(record_rows, batch, "record_rows")
    _need(query_start_loc, batch + 1 if batch else 0, "query_start_loc")
    (pq, pk, pv, pg, pb, pa, pd, ps, psi, pc, pkg, prr, po) = _verify_args(
        q, k, v, raw_g, raw_beta, a_log, dt_bias, state, state_indices, corr, kg,
        record_rows, out)
    _check(_lib.kda_verify(heads, tokens, batch, pq, pk, pv, pg, pb, pa, pd,
                           float(lower_bound), _state_dtype(state), ps, int(state_slot_stride),
                           psi, int(null_slot), pc, pkg, int(record_tokens), prr,
                           _ptr(query_start_loc, torch.int32, "query_start_loc"),
                           *_gate_args(gate, norm_weight),
                           float(norm_eps), po, _stream(stream, state)))
    return out


def kda_fused_replay_verify(*, heads: int, tokens: int, batch: int, q, k, v, raw_g, raw_beta,
                            a_log, dt_bias, lower_bound: float, state, state_slot_stride: int,
                            state_indices, corr, kg, record_tokens: int, record_rows, pending,
                            out, null_slot: int = 0, gate=None, norm_weight=None,
                            norm_eps: float = 1e-5, query_start_loc=None, boundaries=None,
                            boundary_lens=None, stream=None):
    """Replay each request's pending tokens into its page, then verify the
    window. The pool's element type (float32 or bfloat16) is that of ``state``."""
    for t, name in ((state_indices, "state_indices"), (record_rows, "record_rows"),
                    (boundaries, "boundaries"), (boundary_lens, "boundary_lens")):
        _need(t, batch, name)
    _need(query_start_loc, batch + 1 if batch else 0, "query_start_loc")
    (pq, pk, pv, pg, pb, pa, pd, ps, psi, pc, pkg, prr, po) = _verify_args(
        q, k, v, raw_g, raw_beta, a_log, dt_bias, state, state_indices, corr, kg,
        record_rows, out)
    _check(_lib.kda_fused_replay_verify(
        heads, tokens, batch, pq, pk, pv, pg, pb, pa, pd, float(lower_bound),
        _state_dtype(state), ps,
        int(state_slot_stride), psi, int(null_slot), pc, pkg, int(record_tokens), prr,
        _ptr(pending, torch.int32, "pending"),
        _ptr(query_start_loc, torch.int32, "query_start_loc"),
        _ptr(boundaries, torch.int32, "boundaries"),
        _ptr(boundary_lens, torch.int32, "boundary_lens"), *_gate_args(gate, norm_weight),
        float(norm_eps), po, _stream(stream, state)))
    return out


def kda_fused_conv_replay_verify(*, heads: int, tokens: int, batch: int, x, x_row_stride: int,
                                 conv_weight, conv_state, conv_slot_stride: int,
                                 conv_channel_stride: int, conv_tap_stride: int,
                                 q_scale: float, raw_g, raw_beta, a_log, dt_bias,
                                 lower_bound: float, state, state_slot_stride: int,
                                 state_indices, corr, kg, record_tokens: int, record_rows,
                                 pending, out, conv_bias=None, null_slot: int = 0, gate=None,
                                 norm_weight=None, norm_eps: float = 1e-5, boundaries=None,
                                 boundary_lens=None, stream=None):
    """The fused step with its convolution prologue: q, k, v from the packed
    pre-activations ``x`` (rows of ``x_row_stride`` elements) and each channel's
    window in ``conv_state`` (BF16, rewritten in place). Strides in elements."""
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    for t, name in ((state_indices, "state_indices"), (record_rows, "record_rows"),
                    (boundaries, "boundaries"), (boundary_lens, "boundary_lens")):
        _need(t, batch, name)
    _check(_lib.kda_fused_conv_replay_verify(
        heads, tokens, batch, _ptr_rows(x, bf, int(x_row_stride), "x"), int(x_row_stride),
        _ptr(conv_weight, bf, "conv_weight"),
        _ptr(conv_bias, bf, "conv_bias"), _ptr(conv_state, bf, "conv_state"),
        int(conv_slot_stride), int(conv_channel_stride), int(conv_tap_stride),
        float(q_scale), _ptr(raw_g, bf, "raw_g"), _ptr(raw_beta, bf, "raw_beta"),
        _ptr(a_log, f32, "a_log"), _ptr(dt_bias, f32, "dt_bias"), float(lower_bound),
        _state_dtype(state), _ptr(state, None, "state"), int(state_slot_stride),
        _ptr(state_indices, i32, "state_indices"), int(null_slot), _ptr(corr, f32, "corr"),
        _ptr(kg, bf, "kg"), int(record_tokens), _ptr(record_rows, i32, "record_rows"),
        _ptr(pending, i32, "pending"), _ptr(boundaries, i32, "boundaries"),
        _ptr(boundary_lens, i32, "boundary_lens"), *_gate_args(gate, norm_weight),
        float(norm_eps), _ptr(out, bf, "out"), _stream(stream, state)))
    return out


def kda_gate_projection(*, tokens: int, heads: int, f_a, f_a_row_stride: int, f_b, raw_g,
                        stream=None):
    """raw_g [tokens, heads*128] = BF16(F_A F_B^T): f_a rows of ``f_a_row_stride``
    elements (columns 0..127 read), f_b [heads*128, 128]."""
    bf = torch.bfloat16
    _check(_lib.kda_gate_projection(int(tokens), int(heads),
                                    _ptr_rows(f_a, bf, int(f_a_row_stride), "f_a"),
                                    int(f_a_row_stride), _ptr(f_b, bf, "f_b"),
                                    _ptr(raw_g, bf, "raw_g"), _stream(stream, f_b)))
    return raw_g


def kda_defer_commit(*, batch: int, state_indices, commit_lens, record_rows, pending,
                     eager=None, null_slot: int = 0, stream=None):
    i32 = torch.int32
    for t, name in ((state_indices, "state_indices"), (commit_lens, "commit_lens"),
                    (record_rows, "record_rows"), (eager, "eager")):
        _need(t, batch, name)
    _check(_lib.kda_defer_commit(batch, _ptr(state_indices, i32, "state_indices"),
                                 _ptr(commit_lens, i32, "commit_lens"),
                                 _ptr(record_rows, i32, "record_rows"),
                                 _ptr(pending, i32, "pending"), _ptr(eager, i32, "eager"),
                                 int(null_slot), _stream(stream, commit_lens)))


def kda_flush_plan(*, batch: int, spec_query_len: int, state_indices, record_rows, pending,
                   commit_lens, final_indices, boundaries, boundary_lens, null_slot: int = 0,
                   stream=None):
    i32 = torch.int32
    for t, name in ((state_indices, "state_indices"), (record_rows, "record_rows"),
                    (commit_lens, "commit_lens"), (final_indices, "final_indices"),
                    (boundaries, "boundaries"), (boundary_lens, "boundary_lens")):
        _need(t, batch, name)
    _check(_lib.kda_flush_plan(batch, int(spec_query_len),
                               _ptr(state_indices, i32, "state_indices"),
                               _ptr(record_rows, i32, "record_rows"),
                               _ptr(pending, i32, "pending"),
                               _ptr(commit_lens, i32, "commit_lens"),
                               _ptr(final_indices, i32, "final_indices"),
                               _ptr(boundaries, i32, "boundaries"),
                               _ptr(boundary_lens, i32, "boundary_lens"), int(null_slot),
                               _stream(stream, commit_lens)))


def kda_page_rw_probe(*, heads: int, batch: int, state, state_slot_stride: int, state_indices,
                      null_slot: int = 0, stream=None):
    """Measurement aid: read and rewrite every named page unchanged (the pool's
    in-place read+write ceiling in the fused kernel's access pattern)."""
    _check(_lib.kda_page_rw_probe(heads, batch, _ptr(state, torch.float32, "state"),
                                  int(state_slot_stride),
                                  _ptr(state_indices, torch.int32, "state_indices"),
                                  int(null_slot), _stream(stream, state)))
