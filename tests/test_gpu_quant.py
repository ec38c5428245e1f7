"""GPU parity of the quantised tied head (per-row int8 embedding) against the float64 oracle,
through the C ABI: the quantiser bit for bit, the forward within the usual tolerances."""
import dataclasses

import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from oracle import oracle as ora
from tests.gpu_helpers import BPB_RTOL, NATS_ATOL, ensure_lib, host_inputs, oracle_forward_chunked

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def workload(name, **over):
    return dataclasses.replace(synth.WORKLOADS[name], **over)


def quantize_gpu(d_embed):
    V, D = d_embed.shape
    q = torch.empty((V, D), dtype=torch.int8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    abi.pg_quantize_q8(d_embed, q, s)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("name,over", [("fwd_v8192", {}), ("tiny_f32", {}), ("stress", {"D": 48, "stream": 110})])
def test_quantiser_bit_exact(name, over):
    inp = synth.make_inputs(workload(name, **over), 0)
    print(f"[case] quantise {name} V={inp['V']} D={inp['D']} dtype={inp['dtype']}", flush=True)
    d = abi.to_device(inp)
    q, s = quantize_gpu(d["embed"])
    _, E = host_inputs(inp)
    oq, os_ = ora.quantize_rows_q8(E)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)


def test_quantiser_zero_rows_and_exact_grid():
    rng = np.random.default_rng(5)
    V, D = 64, 128
    k = rng.integers(-127, 128, size=(V, D))
    k[:, 0] = 127
    E = (k * np.ldexp(1.0, rng.integers(-12, 0, size=V))[:, None]).astype(np.float32)
    E[7] = 0.0
    q, s = quantize_gpu(torch.from_numpy(E).cuda())
    oq, os_ = ora.quantize_rows_q8(E)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)
    assert s[7].item() == 0.0 and torch.all(q[7] == 0)


def run_q8(inp, sample_rows=None):
    T, D, V, c = inp["T"], inp["D"], inp["V"], inp["softcap"]
    print(f"[case] q8 forward {inp['workload']} T={T} D={D} V={V}", flush=True)
    d = abi.to_device(inp)
    q, s = quantize_gpu(d["embed"])
    nats = torch.full((T,), float("nan"), device="cuda")
    lse = torch.full((T,), float("nan"), device="cuda")
    abi.pg_lmhead_ce_fwd_q8(d["hidden"], q, s, d["target"], None, c, nats, lse)
    torch.cuda.synchronize()
    H, E = host_inputs(inp)
    oq, os_ = ora.quantize_rows_q8(E)
    Ed = ora.dequantize_rows_q8(oq, os_)
    rows = np.arange(T) if sample_rows is None else np.asarray(sample_rows)
    onats, olse = oracle_forward_chunked(H[rows], Ed, inp["target"][rows], c)
    g = nats.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g[rows] - onats)) <= NATS_ATOL
    assert np.max(np.abs(lse.cpu().numpy()[rows] - olse)) <= NATS_ATOL
    # the same head through the bf16 entry point, with the oracle's dequantised embedding: same bits
    Eb = torch.from_numpy(synth.bf16_bits(Ed.astype(np.float32)).view(np.int16)).cuda()
    ref = torch.empty(T, device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], Eb, d["target"], None, c, ref, None)
    torch.cuda.synchronize()
    assert torch.equal(ref, nats)
    return g, H, Ed


def test_quantised_forward_small():
    run_q8(synth.make_inputs(workload("fwd_v8192", T=700, V=1500, stream=111), 0))


def test_quantised_forward_full_size():
    inp = synth.make_inputs("fwd_v8192", 0)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.choice(65536, 256, replace=False), [0, 65535]]))
    g, H, Ed = run_q8(inp, sample_rows=rows)
    onats, _ = oracle_forward_chunked(H, Ed, inp["target"], inp["softcap"])
    b_gpu = ora.bpb(g, inp["target"], inp["byte_len"])[3]
    b_ora = ora.bpb(onats, inp["target"], inp["byte_len"])[3]
    assert abs(b_gpu - b_ora) <= BPB_RTOL * b_ora
