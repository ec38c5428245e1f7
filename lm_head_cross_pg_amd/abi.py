"""ctypes binding of libpg_lmhead.so with the C ABI's entry-point names (include/pg_lmhead.h).

Argument marshalling only: every step of the computation runs in the HIP library. Tensors must be
contiguous CUDA (HIP) tensors; the call is enqueued on torch's current stream. bf16 data may be
passed as ``torch.bfloat16`` tensors or as ``torch.uint16``/``torch.int16`` bit patterns.
The library must have been built (``python -m lm_head_cross_pg_amd.build``); loading fails loudly
otherwise. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpg_lmhead.so")

PG_OK = 0
PG_DTYPE_BF16 = 0
PG_DTYPE_F32 = 1
PG_OP_FWD, PG_OP_BWD, PG_OP_BPB, PG_OP_FWD_Q8, PG_OP_FWD_BWD = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "PG_OK", -1: "PG_ERR_NULL", -2: "PG_ERR_SHAPE", -3: "PG_ERR_DTYPE", -4: "PG_ERR_SOFTCAP",
                -5: "PG_ERR_WORKSPACE", -6: "PG_ERR_ALIGN", -7: "PG_ERR_DEVICE", -8: "PG_ERR_HIP",
                -9: "PG_ERR_SCRATCH"}

# every symbol the header declares
EXPORTS = ("pg_lmhead_ce_fwd", "pg_lmhead_ce_fwd_noalloc", "pg_lmhead_ce_bwd", "pg_lmhead_ce_fwd_bwd", "pg_lmhead_ce_fwd_asym", "pg_lmhead_ce_bwd_asym",
           "pg_lmhead_ce_fwd_bwd_asym",
           "pg_quantize_q8", "pg_lmhead_ce_fwd_q8", "pg_bpb_reduce", "pg_bpb_accumulate", "pg_window_count",
           "pg_window_scored", "pg_window_rows", "pg_sgd_step_bf16", "pg_workspace_bytes", "pg_status_str",
           "pg_abi_version")


class PgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m lm_head_cross_pg_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pg_lmhead_ce_fwd.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_fwd.restype = i32
    lib.pg_lmhead_ce_fwd_noalloc.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, f32, vp, vp, vp]
    lib.pg_lmhead_ce_fwd_noalloc.restype = i32
    lib.pg_lmhead_ce_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i32, i32, f32, f32, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_bwd.restype = i32
    lib.pg_lmhead_ce_fwd_bwd.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, f32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_fwd_bwd.restype = i32
    lib.pg_lmhead_ce_fwd_bwd_asym.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, f32, f32, f32, vp, vp, vp, vp, vp,
                                              sz, vp]
    lib.pg_lmhead_ce_fwd_bwd_asym.restype = i32
    lib.pg_lmhead_ce_fwd_asym.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, f32, f32, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_fwd_asym.restype = i32
    lib.pg_lmhead_ce_bwd_asym.argtypes = [vp, vp, i32, vp, vp, vp, i64, i32, i32, f32, f32, f32, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_bwd_asym.restype = i32
    lib.pg_quantize_q8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.pg_quantize_q8.restype = i32
    lib.pg_lmhead_ce_fwd_q8.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.pg_lmhead_ce_fwd_q8.restype = i32
    lib.pg_bpb_reduce.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp, vp, sz, vp]
    lib.pg_bpb_reduce.restype = i32
    lib.pg_bpb_accumulate.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp, vp, sz, vp]
    lib.pg_bpb_accumulate.restype = i32
    lib.pg_window_count.argtypes = [i64, i32, i32]
    lib.pg_window_count.restype = i64
    lib.pg_window_scored.argtypes = [i64, i32, i32, i64, i32]
    lib.pg_window_scored.restype = i64
    lib.pg_window_rows.argtypes = [vp, i64, i32, i32, i64, i32, vp, vp, vp]
    lib.pg_window_rows.restype = i32
    lib.pg_sgd_step_bf16.argtypes = [vp, vp, f32, i64, vp, vp]
    lib.pg_sgd_step_bf16.restype = i32
    lib.pg_workspace_bytes.argtypes = [i32, i64, i32, i32]
    lib.pg_workspace_bytes.restype = sz
    lib.pg_status_str.argtypes = [i32]
    lib.pg_status_str.restype = ctypes.c_char_p
    lib.pg_abi_version.argtypes = []
    lib.pg_abi_version.restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().pg_status_str(int(status)).decode()


def abi_version() -> int:
    return int(load().pg_abi_version())


def workspace_bytes(op: int, T: int, D: int, V: int) -> int:
    return int(load().pg_workspace_bytes(int(op), int(T), int(D), int(V)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


_BF16 = (torch.bfloat16, torch.uint16, torch.int16)
_MASK = (torch.uint8, torch.bool)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype in _BF16:
        return PG_DTYPE_BF16
    if t.dtype == torch.float32:
        return PG_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bf16 or float32)")


class _Args:
    """Checks of the tensors of one call, made before the library is touched: dtype, element count
    and layout of each tensor first, then that every one of them lives on one CUDA (HIP) device. The
    C ABI takes bare pointers and sizes, so a wrong shape or dtype would otherwise reach the kernels
    as out-of-bounds accesses or silently misread data."""

    def __init__(self, where: str):
        self.where = where
        self.seen = []

    def __call__(self, t, name, dtypes, numel=None, shape=None, min_numel=None, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.where}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            raise ValueError(f"{self.where}: {name} has dtype {t.dtype}; expected one of "
                             f"{', '.join(str(d) for d in dtypes)}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.where}: {name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{self.where}: {name} has {t.numel()} elements; expected {numel}")
        if min_numel is not None and t.numel() < min_numel:
            raise ValueError(f"{self.where}: {name} has {t.numel()} elements; at least {min_numel} needed")
        if not t.is_contiguous():
            raise ValueError(f"{self.where}: {name} must be contiguous")
        self.seen.append((name, t))
        return t

    def same_device(self):
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{self.where}: {name} is on {t.device}; every tensor must be on a CUDA (HIP) device")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.where}: {name} is on {t.device}, other tensors on {dev}")


def _matrix(a: _Args, t, name, dtypes):
    a(t, name, dtypes)
    if t.dim() != 2:
        raise ValueError(f"{a.where}: {name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _head(a: _Args, hidden, embed, target, score_mask, hidden_dtypes=_BF16 + (torch.float32,)):
    """hidden [T, D] and embed [V, D] of one dtype, target int32 [T], score_mask uint8/bool [T]."""
    T, D = _matrix(a, hidden, "hidden", hidden_dtypes)
    V, De = _matrix(a, embed, "embed", _BF16 if hidden.dtype in _BF16 else (torch.float32,))
    if De != D:
        raise ValueError(f"{a.where}: embed has {De} columns, hidden {D}")
    a(target, "target", (torch.int32,), numel=T)
    a(score_mask, "score_mask", _MASK, numel=T, optional=True)
    return T, D, V


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _workspace(a: _Args, op: int, T: int, D: int, V: int, ref: torch.Tensor, workspace):
    if workspace is not None:
        a(workspace, "workspace", (torch.uint8, torch.int8))
        a.same_device()
        return workspace
    a.same_device()
    return torch.empty(max(workspace_bytes(op, T, D, V), 256), dtype=torch.uint8, device=ref.device)


def _check(status: int, where: str):
    if status != PG_OK:
        raise PgError(status, where)


def pg_lmhead_ce_fwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                     score_mask: Optional[torch.Tensor], softcap: float,
                     nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T, optional=True)
    ws = _workspace(a, PG_OP_FWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                 T, D, V, float(softcap), _ptr(nats), _ptr(lse), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(st, "pg_lmhead_ce_fwd")


def pg_lmhead_ce_fwd_noalloc(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                             score_mask: Optional[torch.Tensor], softcap: float,
                             nats: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd_noalloc")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T, optional=True)
    a.same_device()
    st = load().pg_lmhead_ce_fwd_noalloc(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                         _ptr(score_mask), T, D, V, float(softcap), _ptr(nats), _ptr(lse),
                                         _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_noalloc")


def _bwd_outputs(a: _Args, T, D, V, dhidden, dembed):
    a(dhidden, "dhidden", (torch.float32,), numel=T * D, optional=True)   # None: no dH
    a(dembed, "dembed", (torch.float32,), numel=V * D)


def pg_lmhead_ce_bwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                     score_mask: Optional[torch.Tensor], lse: torch.Tensor, softcap: float,
                     grad_scale: float, dhidden: Optional[torch.Tensor], dembed: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_bwd")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(lse, "lse", (torch.float32,), numel=T)
    _bwd_outputs(a, T, D, V, dhidden, dembed)
    ws = _workspace(a, PG_OP_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_bwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                 _ptr(lse), T, D, V, float(softcap), float(grad_scale), _ptr(dhidden),
                                 _ptr(dembed), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_bwd")


def pg_lmhead_ce_fwd_bwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                         score_mask: Optional[torch.Tensor], softcap: float, grad_scale: float,
                         nats: torch.Tensor, lse: torch.Tensor, dhidden: Optional[torch.Tensor], dembed: torch.Tensor,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd_bwd")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T)
    _bwd_outputs(a, T, D, V, dhidden, dembed)
    ws = _workspace(a, PG_OP_FWD_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_bwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                     T, D, V, float(softcap), float(grad_scale), _ptr(nats), _ptr(lse),
                                     _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_bwd")


def pg_lmhead_ce_fwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                          score_mask: Optional[torch.Tensor], cap_pos: float, cap_neg: float,
                          nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd_asym")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T, optional=True)
    ws = _workspace(a, PG_OP_FWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                      _ptr(score_mask), T, D, V, float(cap_pos), float(cap_neg), _ptr(nats),
                                      _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_asym")


def pg_lmhead_ce_bwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                          score_mask: Optional[torch.Tensor], lse: torch.Tensor, cap_pos: float, cap_neg: float,
                          grad_scale: float, dhidden: Optional[torch.Tensor], dembed: torch.Tensor,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_bwd_asym")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(lse, "lse", (torch.float32,), numel=T)
    _bwd_outputs(a, T, D, V, dhidden, dembed)
    ws = _workspace(a, PG_OP_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_bwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                      _ptr(score_mask), _ptr(lse), T, D, V, float(cap_pos), float(cap_neg),
                                      float(grad_scale), _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(),
                                      _stream(stream))
    _check(st, "pg_lmhead_ce_bwd_asym")


def pg_lmhead_ce_fwd_bwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                              score_mask: Optional[torch.Tensor], cap_pos: float, cap_neg: float, grad_scale: float,
                              nats: torch.Tensor, lse: torch.Tensor, dhidden: Optional[torch.Tensor], dembed: torch.Tensor,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd_bwd_asym")
    T, D, V = _head(a, hidden, embed, target, score_mask)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T)
    _bwd_outputs(a, T, D, V, dhidden, dembed)
    ws = _workspace(a, PG_OP_FWD_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_bwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                          _ptr(score_mask), T, D, V, float(cap_pos), float(cap_neg), float(grad_scale),
                                          _ptr(nats), _ptr(lse), _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(),
                                          _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_bwd_asym")


def pg_quantize_q8(embed: torch.Tensor, embed_q8: torch.Tensor, embed_scale: torch.Tensor, stream=None) -> None:
    a = _Args("pg_quantize_q8")
    V, D = _matrix(a, embed, "embed", _BF16 + (torch.float32,))
    a(embed_q8, "embed_q8", (torch.int8,), numel=V * D)
    a(embed_scale, "embed_scale", (torch.float32,), numel=V)
    a.same_device()
    st = load().pg_quantize_q8(_ptr(embed), _dtype_code(embed), V, D, _ptr(embed_q8), _ptr(embed_scale),
                               _stream(stream))
    _check(st, "pg_quantize_q8")


def pg_lmhead_ce_fwd_q8(hidden: torch.Tensor, embed_q8: torch.Tensor, embed_scale: torch.Tensor,
                        target: torch.Tensor, score_mask: Optional[torch.Tensor], softcap: float,
                        nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    a = _Args("pg_lmhead_ce_fwd_q8")
    T, D = _matrix(a, hidden, "hidden", _BF16)
    V, Dq = _matrix(a, embed_q8, "embed_q8", (torch.int8,))
    if Dq != D:
        raise ValueError(f"pg_lmhead_ce_fwd_q8: embed_q8 has {Dq} columns, hidden {D}")
    a(embed_scale, "embed_scale", (torch.float32,), numel=V)
    a(target, "target", (torch.int32,), numel=T)
    a(score_mask, "score_mask", _MASK, numel=T, optional=True)
    a(nats, "nats", (torch.float32,), numel=T)
    a(lse, "lse", (torch.float32,), numel=T, optional=True)
    ws = _workspace(a, PG_OP_FWD_Q8, T, D, V, embed_q8, workspace)
    st = load().pg_lmhead_ce_fwd_q8(_ptr(hidden), _ptr(embed_q8), _ptr(embed_scale), _ptr(target),
                                    _ptr(score_mask), T, D, V, float(softcap), _ptr(nats), _ptr(lse), _ptr(ws),
                                    ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_q8")


def pg_bpb_reduce(nats: torch.Tensor, target: Optional[torch.Tensor], score_mask: Optional[torch.Tensor],
                  byte_len: Optional[torch.Tensor], byte_per_pos: Optional[torch.Tensor], V: int,
                  out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None,
                  _entry: str = "pg_bpb_reduce") -> None:
    a = _Args(_entry)
    a(nats, "nats", (torch.float32,))
    T = nats.numel()
    a(byte_per_pos, "byte_per_pos", (torch.int32,), numel=T, optional=True)
    a(target, "target", (torch.int32,), numel=T, optional=byte_per_pos is not None)
    a(byte_len, "byte_len", (torch.int32,), min_numel=int(V), optional=byte_per_pos is not None)
    a(score_mask, "score_mask", _MASK, numel=T, optional=True)
    a(out, "out", (torch.float64,), min_numel=4)
    ws = _workspace(a, PG_OP_BPB, T, 1, V, out, workspace)
    st = getattr(load(), _entry)(_ptr(nats), _ptr(target), _ptr(score_mask), _ptr(byte_len), _ptr(byte_per_pos),
                                 T, int(V), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, _entry)


def pg_bpb_accumulate(nats: torch.Tensor, target: Optional[torch.Tensor], score_mask: Optional[torch.Tensor],
                      byte_len: Optional[torch.Tensor], byte_per_pos: Optional[torch.Tensor], V: int,
                      out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """pg_bpb_reduce adding into the running sums held in out[0..2]."""
    pg_bpb_reduce(nats, target, score_mask, byte_len, byte_per_pos, V, out, workspace, stream,
                  _entry="pg_bpb_accumulate")


def pg_window_count(n_tokens: int, window: int, stride: int) -> int:
    n = int(load().pg_window_count(int(n_tokens), int(window), int(stride)))
    if n < 0:
        raise PgError(n, "pg_window_count")
    return n


def pg_window_scored(n_tokens: int, window: int, stride: int, first_window: int, n_windows: int) -> int:
    n = int(load().pg_window_scored(int(n_tokens), int(window), int(stride), int(first_window), int(n_windows)))
    if n < 0:
        raise PgError(n, "pg_window_scored")
    return n


def pg_window_rows(tokens: torch.Tensor, window: int, stride: int, first_window: int, n_windows: int,
                   target: torch.Tensor, score_mask: torch.Tensor, stream=None) -> None:
    a = _Args("pg_window_rows")
    a(tokens, "tokens", (torch.int32,))
    rows = int(n_windows) * int(window)
    a(target, "target", (torch.int32,), min_numel=rows)
    a(score_mask, "score_mask", _MASK, min_numel=rows)
    a.same_device()
    st = load().pg_window_rows(_ptr(tokens), tokens.numel(), int(window), int(stride), int(first_window),
                               int(n_windows), _ptr(target), _ptr(score_mask), _stream(stream))
    _check(st, "pg_window_rows")


def pg_sgd_step_bf16(master: torch.Tensor, grad: torch.Tensor, lr: float, embed: torch.Tensor, stream=None) -> None:
    a = _Args("pg_sgd_step_bf16")
    a(master, "master", (torch.float32,))
    n = master.numel()
    a(grad, "grad", (torch.float32,), numel=n)
    a(embed, "embed", _BF16, numel=n)
    a.same_device()
    st = load().pg_sgd_step_bf16(_ptr(master), _ptr(grad), float(lr), n, _ptr(embed), _stream(stream))
    _check(st, "pg_sgd_step_bf16")


def to_device(inp: dict, device="cuda") -> dict:
    """Move one synthetic workload (from lm_head_cross_pg_amd.synth) to the GPU as tensors."""
    def bf16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16)
    if inp["dtype"] == "bf16":
        H, E = bf16(inp["hidden"]), bf16(inp["embed"])
    else:
        H, E = torch.from_numpy(inp["hidden"]), torch.from_numpy(inp["embed"])
    out = dict(hidden=H.to(device), embed=E.to(device), target=torch.from_numpy(inp["target"]).to(device),
               byte_len=torch.from_numpy(inp["byte_len"]).to(device),
               mask=None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to(device))
    return out
