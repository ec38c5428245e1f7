"""GPU parity of the sliding-window evaluation driver (score-first test-time training included)
against the oracle's plain loop, through the C ABI: the batch rows bit for bit, the SGD step bit for
bit, and per batch the nats, the gradients and the running bits per byte."""

import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from lm_head_cross_pg_amd.window_eval import SlidingWindowEval
from oracle import oracle as ora
from tests.gpu_helpers import BPB_RTOL, GRAD_RL2, NATS_ATOL, ensure_lib, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _expected_rows(tokens, window, stride, w0, nw):
    """Targets and mask of a batch, from the oracle's schedule and the batch layout (row (b, r) is
    input position (w0 + b) stride + r; its target is the next token, 0 past the stream)."""
    n = len(tokens)
    sched = ora.window_schedule(n, window, stride)
    tgt = np.zeros(nw * window, np.int32)
    msk = np.zeros(nw * window, np.uint8)
    for b in range(nw):
        w = w0 + b
        for r in range(window):
            p = w * stride + r
            if p + 1 < n:
                tgt[b * window + r] = tokens[p + 1]
        for p in (sched[w] if w < len(sched) else []):
            msk[b * window + p - w * stride] = 1
    return tgt, msk


@pytest.mark.parametrize("n,window,stride,w0,nw", [(14, 8, 2, 0, 4), (14, 8, 2, 1, 3), (12, 6, 4, 0, 3),
                                                   (4625, 2048, 64, 0, 8), (4625, 2048, 64, 40, 2),
                                                   (4625, 2048, 64, 3, 20), (1000, 2048, 64, 0, 1),
                                                   (300, 16, 16, 2, 9)])
def test_window_rows_bit_exact(n, window, stride, w0, nw):
    print(f"[case] window rows n={n} L={window} s={stride} w0={w0} nw={nw}", flush=True)
    tokens = np.random.default_rng(n).integers(0, 1000, n).astype(np.int32)
    t = torch.from_numpy(tokens).cuda()
    tgt = torch.full((nw * window,), -7, dtype=torch.int32, device="cuda")
    msk = torch.full((nw * window,), 9, dtype=torch.uint8, device="cuda")
    abi.pg_window_rows(t, window, stride, w0, nw, tgt, msk)
    torch.cuda.synchronize()
    et, em = _expected_rows(tokens, window, stride, w0, nw)
    np.testing.assert_array_equal(tgt.cpu().numpy(), et)
    np.testing.assert_array_equal(msk.cpu().numpy(), em)
    assert int(em.sum()) == abi.pg_window_scored(n, window, stride, w0, nw)


def test_sgd_step_bit_exact():
    rng = np.random.default_rng(4)
    n = 1_000_003
    m = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    lr = 3.7
    mt, gt = torch.from_numpy(m.copy()).cuda(), torch.from_numpy(g).cuda()
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    print("[case] sgd step", flush=True)
    abi.pg_sgd_step_bf16(mt, gt, lr, out)
    torch.cuda.synchronize()
    exp = m - np.float32(lr) * g
    np.testing.assert_array_equal(mt.cpu().numpy(), exp)
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), synth.bf16_bits(exp))


def _run(seed, n_tokens, windows_per_batch, lr, D=512, V=8192, window=2048, stride=64, keep_dhidden=True):
    st = synth.make_stream(seed, n_tokens, V, D=D)
    tokens, blen = st["tokens"], st["byte_len"]
    sched = ora.window_schedule(n_tokens, window, stride)

    def hid(w, n):
        return synth.window_hidden(seed, w, n, D)

    E16 = torch.from_numpy(st["embed"].view(np.int16)).cuda().view(torch.bfloat16)
    master = torch.from_numpy(synth.bf16_to_f64(st["embed"]).astype(np.float32)).cuda() if lr else None
    drv = SlidingWindowEval(torch.from_numpy(tokens).cuda(), torch.from_numpy(blen).cuda(), V, D, window, stride,
                            windows_per_batch, 30.0, ttt_lr=lr, embed_master=master, keep_dhidden=keep_dhidden)
    assert drv.n_windows == len(sched)
    got = []
    for w0, nw in drv.batches():
        H = np.zeros((nw * window, D), np.uint16)
        for b in range(nw):
            w = w0 + b
            r0 = sched[w][0] - w * stride
            H[b * window + r0: b * window + r0 + len(sched[w])] = hid(w, len(sched[w]))
        Ht = torch.from_numpy(H.view(np.int16)).cuda().view(torch.bfloat16)
        print(f"[case] window driver seed={seed} n={n_tokens} batch w0={w0} nw={nw} lr={lr}", flush=True)
        n = drv.step(Ht, E16, w0, nw)
        rows = nw * window
        mask = drv.mask[:rows].bool()
        rec = {"n": n, "nats": drv.nats[:rows][mask].cpu().numpy().astype(np.float64)}
        if lr:
            rec["dE"] = drv.dE.cpu().numpy().astype(np.float64)
            if keep_dhidden:
                rec["dH"] = drv.dH[:rows][mask].cpu().numpy().astype(np.float64)
        got.append(rec)
    torch.cuda.synchronize()
    ref = ora.sliding_window_eval(tokens, blen, lambda w, n: synth.bf16_to_f64(hid(w, n)),
                                  synth.bf16_to_f64(st["embed"]), 30.0, window, stride, windows_per_batch, lr=lr)
    return drv, got, ref


def _check(drv, got, ref):
    assert len(got) == len(ref["batches"])
    for g, r in zip(got, ref["batches"]):
        assert g["n"] == len(r["positions"]) == len(g["nats"])
        assert np.all(g["nats"] >= 0.0)
        assert np.max(np.abs(g["nats"] - r["nats"])) <= NATS_ATOL
        if "dE" in r:
            assert rel_l2(g["dE"], r["dE"]) <= GRAD_RL2, rel_l2(g["dE"], r["dE"])
            if "dH" in g:
                assert rel_l2(g["dH"], r["dH"]) <= GRAD_RL2, rel_l2(g["dH"], r["dH"])
    sn, sb, n, b = drv.result()
    assert n == ref["n_scored"] and sb == ref["sum_bytes"]
    assert abs(sn - ref["sum_nats"]) <= BPB_RTOL * ref["sum_nats"]
    assert abs(b - ref["bpb"]) <= BPB_RTOL * ref["bpb"], (b, ref["bpb"])


def test_driver_stride64_eval():
    """42 windows of 2048 at stride 64 (a ragged last window), 8 windows per batch: D = 512, V = 8192."""
    drv, got, ref = _run(0, 4625, 8, 0.0)
    _check(drv, got, ref)


def test_driver_score_first_ttt():
    """The same stream with one SGD step of the tied embedding after each batch is scored. At this
    rate one step moves some rows' nats by whole nats, so a batch scored with the wrong embedding
    (before its predecessors' steps, or after its own) would miss the oracle's nats by far more than
    the tolerance."""
    base, got0, _ = _run(1, 4625, 8, 0.0)
    drv, got, ref = _run(1, 4625, 8, 2.0)
    _check(drv, got, ref)
    # the first batch is scored before any update; every later one after the earlier steps
    np.testing.assert_allclose(got[0]["nats"], got0[0]["nats"], rtol=0, atol=1e-6)
    for k in range(1, len(got)):
        assert np.max(np.abs(got[k]["nats"] - got0[k]["nats"])) > 0.5


def test_driver_masked_workload_scale():
    """Batches of 32 windows of 2048 (65,536 rows, the masked workload's shape; the first batch
    scores window 0's 2048 predictions and 64 for each later window) over 96 windows, with TTT."""
    drv, got, ref = _run(2, 2048 + 64 * 95 + 1, 32, 2.0)
    assert len(got) == 3
    _check(drv, got, ref)


def test_driver_ttt_without_dhidden():
    """Score-first training as the driver runs it by default, without the hidden states' gradient
    (its product is left out): the nats, dE and bits per byte of every batch are those of the run
    that also computes dH, bit for bit (dE does not depend on dH), and match the oracle."""
    drv_h, got_h, _ = _run(3, 4625, 8, 2.0, keep_dhidden=True)
    drv, got, ref = _run(3, 4625, 8, 2.0, keep_dhidden=False)
    assert drv.dH is None
    _check(drv, got, ref)
    for a, b in zip(got, got_h):
        np.testing.assert_array_equal(a["nats"], b["nats"])
        np.testing.assert_array_equal(a["dE"], b["dE"])
    assert drv.result() == drv_h.result()


@pytest.mark.parametrize("n_tokens", [1, 2, 3, 1000, 2049])
def test_driver_short_streams(n_tokens):
    """Streams shorter than two windows: none to predict (one token: no window, BPB NaN as 0 / 0),
    one prediction, part of one window, exactly one window, one window and one more token."""
    drv, got, ref = _run(4, n_tokens, 8, 0.0, keep_dhidden=False)
    sn, sb, n, b = drv.result()
    assert drv.n_windows == len(ora.window_schedule(n_tokens, 2048, 64))
    if n_tokens < 2:
        assert len(got) == 0 and n == 0 and np.isnan(b) and np.isnan(ref["bpb"])
    else:
        _check(drv, got, ref)


def test_driver_int8_head():
    """Sliding-window evaluation of the int8 head (evaluation after quantisation): the driver's
    int8 steps against the oracle's loop on the dequantised embedding, and bit for bit the nats and
    sums of the bf16 driver run on that embedding's bf16 form."""
    seed, n_tokens, window, stride, D, V, per_batch = 5, 4625, 2048, 64, 512, 8192, 8
    st = synth.make_stream(seed, n_tokens, V, D=D)
    tokens, blen = st["tokens"], st["byte_len"]
    sched = ora.window_schedule(n_tokens, window, stride)
    E16 = torch.from_numpy(st["embed"].view(np.int16)).cuda().view(torch.bfloat16)
    q8 = torch.empty((V, D), dtype=torch.int8, device="cuda")
    sc8 = torch.empty(V, dtype=torch.float32, device="cuda")
    abi.pg_quantize_q8(E16, q8, sc8)
    Ed = ora.dequantize_rows_q8(*ora.quantize_rows_q8(synth.bf16_to_f64(st["embed"])))
    Ed16 = torch.from_numpy(synth.bf16_bits(Ed.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    t, b = torch.from_numpy(tokens).cuda(), torch.from_numpy(blen).cuda()
    drv8 = SlidingWindowEval(t, b, V, D, window, stride, per_batch, 30.0, int8_head=True)
    drv = SlidingWindowEval(t, b, V, D, window, stride, per_batch, 30.0)
    got = []
    for w0, nw in drv8.batches():
        H = np.zeros((nw * window, D), np.uint16)
        for k in range(nw):
            w = w0 + k
            r0 = sched[w][0] - w * stride
            H[k * window + r0: k * window + r0 + len(sched[w])] = synth.window_hidden(seed, w, len(sched[w]), D)
        Ht = torch.from_numpy(H.view(np.int16)).cuda().view(torch.bfloat16)
        print(f"[case] int8 window driver batch w0={w0} nw={nw}", flush=True)
        n = drv8.step_int8(Ht, q8, sc8, w0, nw)
        assert drv.step(Ht, Ed16, w0, nw) == n
        rows = nw * window
        assert torch.equal(drv8.nats[:rows], drv.nats[:rows])
        got.append({"n": n, "nats": drv8.nats[:rows][drv8.mask[:rows].bool()].cpu().numpy().astype(np.float64)})
    torch.cuda.synchronize()
    assert drv8.result() == drv.result()
    ref = ora.sliding_window_eval(tokens, blen, lambda w, k: synth.bf16_to_f64(synth.window_hidden(seed, w, k, D)),
                                  Ed, 30.0, window, stride, per_batch)
    _check(drv8, got, ref)
    with pytest.raises(ValueError):
        drv.step_int8(Ht, q8, sc8, 0, 1)
