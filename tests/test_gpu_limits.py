"""GPU parity at the size limits of the C ABI: the widest vocabulary (V = 2^20) and the widest hidden
state (D = 2^20) the entry points accept, and a vocabulary beyond 2^16 through one-call training,
against the float64 oracle."""

import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from oracle import oracle as ora
from tests.gpu_helpers import BPB_RTOL, GRAD_RL2, NATS_ATOL, ensure_lib, gpu_bpb, host_inputs

pytestmark = pytest.mark.gpu

MAX_WIDTH = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def make(name, stream, T, D, V, **kw):
    return synth.make_inputs(synth.Workload(name=name, stream=stream, T=T, D=D, V=V, dtype="bf16", **kw), 0)


def forward_check(inp, c=30.0):
    T, V = inp["T"], inp["V"]
    d = abi.to_device(inp)
    nats = torch.full((T,), float("nan"), device="cuda")
    lse = torch.full((T,), float("nan"), device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse)
    out = gpu_bpb(nats, d, V)
    H, E = host_inputs(inp)
    onats, olse = ora.forward(H, E, inp["target"], c)
    assert np.max(np.abs(nats.cpu().numpy() - onats)) <= NATS_ATOL
    assert np.max(np.abs(lse.cpu().numpy() - olse)) <= NATS_ATOL
    b_ora = ora.bpb(onats, inp["target"], inp["byte_len"])[3]
    assert abs(out[3] - b_ora) <= BPB_RTOL * b_ora
    return d, H, E


def test_widest_vocabulary_forward():
    """V = 2^20 (the largest accepted), T = 64, D = 32: 16384 vocabulary tiles split over the
    workgroups, merged in the finalise kernel."""
    inp = make("v_max", 200, T=64, D=32, V=MAX_WIDTH)
    print(f"[case] forward V={inp['V']} T={inp['T']} D={inp['D']}", flush=True)
    forward_check(inp)


def test_vocabulary_beyond_2_16_training_one_call():
    """V = 65537 (one row past a power of two), T = 300, D = 64: the one-call training path with a
    ragged last vocabulary tile, against the oracle's gradients."""
    inp = make("v_65537", 201, T=300, D=64, V=65537)
    T, D, V = inp["T"], inp["D"], inp["V"]
    print(f"[case] training one call V={V} T={T} D={D}", flush=True)
    d = abi.to_device(inp)
    nats, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    dH = torch.full((T, D), float("nan"), device="cuda")
    dE = torch.full((V, D), float("nan"), device="cuda")
    g = 1.0 / T
    abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], None, 30.0, g, nats, lse, dH, dE)
    torch.cuda.synchronize()
    H, E = host_inputs(inp)
    onats, _ = ora.forward(H, E, inp["target"], 30.0)
    assert np.max(np.abs(nats.cpu().numpy() - onats)) <= NATS_ATOL
    odH, odE = ora.backward(H, E, inp["target"], 30.0, g)
    dHn, dEn = dH.cpu().numpy().astype(np.float64), dE.cpu().numpy().astype(np.float64)
    assert rel_l2(dHn, odH) <= GRAD_RL2, rel_l2(dHn, odH)
    assert rel_l2(dEn, odE) <= GRAD_RL2, rel_l2(dEn, odE)


def test_widest_hidden_state():
    """D = 2^20 (the largest accepted), T = 3, V = 5: the plain vector kernels, forward and both
    training entry points. The embedding is scaled to 0.02 / 32 so that z stays near unit size over
    a million products."""
    inp = make("d_max", 202, T=3, D=MAX_WIDTH, V=5, embed_std=0.02 / 32)
    T, D, V = inp["T"], inp["D"], inp["V"]
    print(f"[case] D={D} T={T} V={V}", flush=True)
    d, H, E = forward_check(inp)
    g = 1.0 / T
    odH, odE = ora.backward(H, E, inp["target"], 30.0, g)
    for fused in (False, True):
        print(f"[case] D={D} training fused={fused}", flush=True)
        nats, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
        dH = torch.full((T, D), float("nan"), device="cuda")
        dE = torch.full((V, D), float("nan"), device="cuda")
        if fused:
            abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], None, 30.0, g, nats, lse, dH, dE)
        else:
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, 30.0, nats, lse)
            abi.pg_lmhead_ce_bwd(d["hidden"], d["embed"], d["target"], None, lse, 30.0, g, dH, dE)
        torch.cuda.synchronize()
        dHn, dEn = dH.cpu().numpy().astype(np.float64), dE.cpu().numpy().astype(np.float64)
        assert rel_l2(dHn, odH) <= GRAD_RL2, rel_l2(dHn, odH)
        assert rel_l2(dEn, odE) <= GRAD_RL2, rel_l2(dEn, odE)
