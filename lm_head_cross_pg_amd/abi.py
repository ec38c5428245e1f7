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
                -5: "PG_ERR_WORKSPACE", -6: "PG_ERR_ALIGN", -7: "PG_ERR_DEVICE", -8: "PG_ERR_HIP"}

# every symbol the header declares
EXPORTS = ("pg_lmhead_ce_fwd", "pg_lmhead_ce_bwd", "pg_lmhead_ce_fwd_bwd", "pg_lmhead_ce_fwd_asym", "pg_lmhead_ce_bwd_asym",
           "pg_lmhead_ce_fwd_bwd_asym",
           "pg_quantize_q8", "pg_lmhead_ce_fwd_q8", "pg_bpb_reduce", "pg_workspace_bytes", "pg_status_str",
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
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        return PG_DTYPE_BF16
    if t.dtype == torch.float32:
        return PG_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bf16 or float32)")


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _workspace(op: int, T: int, D: int, V: int, ref: torch.Tensor, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(workspace_bytes(op, T, D, V), 256), dtype=torch.uint8, device=ref.device)


def _check(status: int, where: str):
    if status != PG_OK:
        raise PgError(status, where)


def pg_lmhead_ce_fwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                     score_mask: Optional[torch.Tensor], softcap: float,
                     nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_FWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                 T, D, V, float(softcap), _ptr(nats), _ptr(lse), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(st, "pg_lmhead_ce_fwd")


def pg_lmhead_ce_bwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                     score_mask: Optional[torch.Tensor], lse: torch.Tensor, softcap: float,
                     grad_scale: float, dhidden: torch.Tensor, dembed: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_bwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                 _ptr(lse), T, D, V, float(softcap), float(grad_scale), _ptr(dhidden),
                                 _ptr(dembed), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_bwd")


def pg_lmhead_ce_fwd_bwd(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                         score_mask: Optional[torch.Tensor], softcap: float, grad_scale: float,
                         nats: torch.Tensor, lse: torch.Tensor, dhidden: torch.Tensor, dembed: torch.Tensor,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_FWD_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_bwd(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target), _ptr(score_mask),
                                     T, D, V, float(softcap), float(grad_scale), _ptr(nats), _ptr(lse),
                                     _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_bwd")


def pg_lmhead_ce_fwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                          score_mask: Optional[torch.Tensor], cap_pos: float, cap_neg: float,
                          nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_FWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                      _ptr(score_mask), T, D, V, float(cap_pos), float(cap_neg), _ptr(nats),
                                      _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_asym")


def pg_lmhead_ce_bwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                          score_mask: Optional[torch.Tensor], lse: torch.Tensor, cap_pos: float, cap_neg: float,
                          grad_scale: float, dhidden: torch.Tensor, dembed: torch.Tensor,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_bwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                      _ptr(score_mask), _ptr(lse), T, D, V, float(cap_pos), float(cap_neg),
                                      float(grad_scale), _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(),
                                      _stream(stream))
    _check(st, "pg_lmhead_ce_bwd_asym")


def pg_lmhead_ce_fwd_bwd_asym(hidden: torch.Tensor, embed: torch.Tensor, target: torch.Tensor,
                              score_mask: Optional[torch.Tensor], cap_pos: float, cap_neg: float, grad_scale: float,
                              nats: torch.Tensor, lse: torch.Tensor, dhidden: torch.Tensor, dembed: torch.Tensor,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed.shape[0]
    ws = _workspace(PG_OP_FWD_BWD, T, D, V, embed, workspace)
    st = load().pg_lmhead_ce_fwd_bwd_asym(_ptr(hidden), _ptr(embed), _dtype_code(hidden), _ptr(target),
                                          _ptr(score_mask), T, D, V, float(cap_pos), float(cap_neg), float(grad_scale),
                                          _ptr(nats), _ptr(lse), _ptr(dhidden), _ptr(dembed), _ptr(ws), ws.numel(),
                                          _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_bwd_asym")


def pg_quantize_q8(embed: torch.Tensor, embed_q8: torch.Tensor, embed_scale: torch.Tensor, stream=None) -> None:
    V, D = embed.shape
    st = load().pg_quantize_q8(_ptr(embed), _dtype_code(embed), V, D, _ptr(embed_q8), _ptr(embed_scale),
                               _stream(stream))
    _check(st, "pg_quantize_q8")


def pg_lmhead_ce_fwd_q8(hidden: torch.Tensor, embed_q8: torch.Tensor, embed_scale: torch.Tensor,
                        target: torch.Tensor, score_mask: Optional[torch.Tensor], softcap: float,
                        nats: torch.Tensor, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T, D = hidden.shape
    V = embed_q8.shape[0]
    ws = _workspace(PG_OP_FWD_Q8, T, D, V, embed_q8, workspace)
    st = load().pg_lmhead_ce_fwd_q8(_ptr(hidden), _ptr(embed_q8), _ptr(embed_scale), _ptr(target),
                                    _ptr(score_mask), T, D, V, float(softcap), _ptr(nats), _ptr(lse), _ptr(ws),
                                    ws.numel(), _stream(stream))
    _check(st, "pg_lmhead_ce_fwd_q8")


def pg_bpb_reduce(nats: torch.Tensor, target: torch.Tensor, score_mask: Optional[torch.Tensor],
                  byte_len: torch.Tensor, byte_per_pos: Optional[torch.Tensor], V: int,
                  out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    T = nats.shape[0]
    ws = _workspace(PG_OP_BPB, T, 1, V, out, workspace)
    st = load().pg_bpb_reduce(_ptr(nats), _ptr(target), _ptr(score_mask), _ptr(byte_len), _ptr(byte_per_pos),
                              T, int(V), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "pg_bpb_reduce")


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
