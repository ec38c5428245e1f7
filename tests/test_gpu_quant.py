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


def run_q8(inp, sample_rows=None, mask=None):
    T, D, V, c = inp["T"], inp["D"], inp["V"], inp["softcap"]
    print(f"[case] q8 forward {inp['workload']} T={T} D={D} V={V} masked={mask is not None}", flush=True)
    d = abi.to_device(inp)
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    q, s = quantize_gpu(d["embed"])
    nats = torch.full((T,), float("nan"), device="cuda")
    lse = torch.full((T,), float("nan"), device="cuda")
    abi.pg_lmhead_ce_fwd_q8(d["hidden"], q, s, d["target"], mask_t, c, nats, lse)
    torch.cuda.synchronize()
    H, E = host_inputs(inp)
    oq, os_ = ora.quantize_rows_q8(E)
    Ed = ora.dequantize_rows_q8(oq, os_)
    rows = np.arange(T) if sample_rows is None else np.asarray(sample_rows)
    onats, olse = ora.forward_q8(H[rows], oq, os_, inp["target"][rows], c, None if mask is None else mask[rows])
    g = nats.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g[rows] - onats)) <= NATS_ATOL
    assert np.max(np.abs(lse.cpu().numpy()[rows] - olse)) <= NATS_ATOL
    if mask is not None:
        assert np.all(g[mask == 0] == 0.0)
    # the same head through the bf16 entry point, with the oracle's dequantised embedding: same bits
    Eb = torch.from_numpy(synth.bf16_bits(Ed.astype(np.float32)).view(np.int16)).cuda()
    ref = torch.empty(T, device="cuda")
    ref_lse = torch.full((T,), float("nan"), device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], Eb, d["target"], mask_t, c, ref, ref_lse)
    torch.cuda.synchronize()
    assert torch.equal(ref, nats) and torch.equal(ref_lse, lse)
    return g, H, Ed


def test_quantised_forward_small():
    run_q8(synth.make_inputs(workload("fwd_v8192", T=700, V=1500, stream=111), 0))


@pytest.mark.parametrize("T,D,masked", [(700, 512, True), (4097, 512, False), (300, 48, True), (255, 64, False)])
def test_quantised_forward_masked_ragged_and_generic(T, D, masked):
    """The int8 head with a scored-row mask, ragged row counts, and a width without an MFMA
    instantiation (D = 48, the vector kernel) against the oracle's forward on the dequantised head."""
    inp = synth.make_inputs(workload("fwd_v8192", T=T, D=D, V=1000, stream=112 + D), 0)
    mask = (np.random.default_rng(T).random(T) < 0.4).astype(np.uint8) if masked else None
    run_q8(inp, mask=mask)


@pytest.mark.parametrize("T,V,masked,cap,hscale", [
    (8192, 8192, False, 30.0, 1.0),    # 32 row tiles: 8 vocabulary splits of 16 tiles, the pipelined conversion
    (8192, 8192, True, 30.0, 8.0),     # the same with a mask, logits on the exact softcap
    (20000, 8192, "all", 30.0, 1.0),   # a mask scoring every row: 79 row tiles over the whole vocabulary each
    (20000, 8192, False, 30.0, 1.0),   # the same rows without a mask: the dequantising pass
    (2048, 4133, True, 30.0, 1.0),     # ragged vocabulary: the last tile partial
    (1, 8192, False, 30.0, 1.0),       # one row: every split a single tile
    (300, 64, False, 30.0, 1.0),       # one tile in all
    (300, 65, True, 30.0, 1.0),        # one full tile and one row
    (1000, 8192, False, 50.0, 1.0),    # a cap above the fixed-shift range: the dequantising pass
    (1000, 1000, False, 0.0, 1.0),     # no cap: the dequantising pass
])
def test_q8_on_chip_conversion_same_bits(T, V, masked, cap, hscale):
    """At D = 512 with one cap in (0, 40] the forward converts each int8 tile into bf16 on chip; the
    other caps rebuild the bf16 head first. Either way nats and lse are the bits of the bf16 entry
    point on the dequantised head (torch.equal on every row), and the sampled rows are within the
    tolerance of the oracle's forward on the quantised head."""
    inp = synth.make_inputs(workload("fwd_v8192", T=T, V=V, softcap=cap, hidden_scale=hscale, stream=150 + V % 97), 0)
    mask = (np.random.default_rng(T + V).random(T) < 0.5).astype(np.uint8) if masked else None
    if masked == "all":
        mask[:] = 1
    if mask is not None:
        mask[0] = 1
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(T, min(T, 96), replace=False), [0, T - 1]]))
    run_q8(inp, sample_rows=rows, mask=mask)


def test_quantised_forward_full_size():
    inp = synth.make_inputs("fwd_v8192", 0)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.choice(65536, 256, replace=False), [0, 65535]]))
    g, H, Ed = run_q8(inp, sample_rows=rows)
    onats, _ = oracle_forward_chunked(H, Ed, inp["target"], inp["softcap"])
    b_gpu = ora.bpb(g, inp["target"], inp["byte_len"])[3]
    b_ora = ora.bpb(onats, inp["target"], inp["byte_len"])[3]
    assert abs(b_gpu - b_ora) <= BPB_RTOL * b_ora


def test_rounding_ties_bit_exact():
    """The ties of tests/golden/rounding_ties.json on the GPU: quotients that are exact halves give
    the even codes (bf16 and f32 input), and a head whose q * scale products lie halfway between
    two bfloat16 values scores exactly as the bf16 entry point does on the fixture's even-rounded
    embedding (torch.equal on nats), so the dequantisation rounds those ties to even too."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "rounding_ties.json")) as f:
        g = json.load(f)
    rows = np.array(g["q8"]["rows"], dtype=np.float32)
    print("[case] q8 ties", flush=True)
    for Et in (torch.from_numpy(rows).cuda(),
               torch.from_numpy(synth.bf16_bits(rows).view(np.int16)).cuda().view(torch.bfloat16)):
        q, s = quantize_gpu(Et)
        for row in q.cpu().numpy():
            np.testing.assert_array_equal(row, g["q8"]["codes"])
        np.testing.assert_array_equal(s.cpu().numpy(), np.array(g["q8"]["scales"], dtype=np.float32))
    # dequantised ties: V = 6 rows, row j = codes * scale * 2^-j (powers of two keep every tie)
    dq = g["dequant"]
    V, D, T = 6, len(dq["codes"]), 256
    base = np.array(dq["rows_f32"][0], dtype=np.float64)
    E32 = np.stack([base * 2.0 ** -j for j in range(V)]).astype(np.float32)
    Eexp = np.stack([np.array(dq["bf16"]) * 2.0 ** -j for j in range(V)])
    q, s = quantize_gpu(torch.from_numpy(E32).cuda())
    for j in range(V):
        np.testing.assert_array_equal(q.cpu().numpy()[j], dq["codes"])
    np.testing.assert_array_equal(ora.dequantize_rows_q8(q.cpu().numpy(), s.cpu().numpy()), Eexp)
    rng = np.random.default_rng(17)
    Hb = synth.bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    Ht = torch.from_numpy(Hb.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.from_numpy(rng.integers(0, V, T).astype(np.int32)).cuda()
    nats, ref = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    abi.pg_lmhead_ce_fwd_q8(Ht, q, s, y, None, 30.0, nats, None)
    Eb = torch.from_numpy(synth.bf16_bits(Eexp.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    abi.pg_lmhead_ce_fwd(Ht, Eb, y, None, 30.0, ref, None)
    torch.cuda.synchronize()
    assert torch.equal(nats, ref)
    onats, _ = ora.forward(synth.bf16_to_f64(Hb), Eexp, y.cpu().numpy(), 30.0)
    assert np.max(np.abs(nats.cpu().numpy() - onats)) <= NATS_ATOL
