"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the float64
oracle on the same seeded inputs. Tolerances: BPB relative 1e-4, per-row nats absolute 2e-2,
gradients relative L2 1e-2 (bf16 inputs, float32 accumulation)."""
import os

import numpy as np
import torch

from lm_head_cross_pg_amd import abi, build, synth
from oracle import oracle as ora

NATS_ATOL = 2e-2
BPB_RTOL = 1e-4
GRAD_RL2 = 1e-2


def ensure_lib():
    if not os.path.exists(abi.LIB_PATH):
        build.build()
    return abi.load()


def gpu_forward(d, T, D, V, softcap, mask=None):
    nats = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask, softcap, nats, lse)
    torch.cuda.synchronize()
    return nats.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def gpu_bpb(nats_t, d, V, mask=None, byte_per_pos=None):
    out = torch.zeros(4, dtype=torch.float64, device="cuda")
    abi.pg_bpb_reduce(nats_t, d["target"], mask, d["byte_len"], byte_per_pos, V, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def host_inputs(inp):
    H = synth.as_f64(inp["hidden"], inp["dtype"])
    E = synth.as_f64(inp["embed"], inp["dtype"])
    return H, E


def oracle_forward_chunked(H, E, y, c, mask=None, rows_per_chunk=4096):
    """The oracle's per-row forward over row chunks (rows are independent by definition)."""
    T = H.shape[0]
    nats = np.zeros(T)
    lse = np.zeros(T)
    for b in range(0, T, rows_per_chunk):
        e = min(T, b + rows_per_chunk)
        m = None if mask is None else mask[b:e]
        nats[b:e], lse[b:e] = ora.forward(H[b:e], E, y[b:e], c, m)
    return nats, lse


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
