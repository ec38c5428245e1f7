"""Pins of the oracle's sliding-window evaluation (schedule, bits per byte across windows, score-first
test-time training) against what the rule fixes, and of the C ABI's host-side schedule arithmetic
against the oracle's schedule (integers, bit for bit)."""
import json
import os

import numpy as np
import pytest

from lm_head_cross_pg_amd import abi, build, synth
from oracle import oracle as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    with open(os.path.join(GOLDEN, "window_schedules.json")) as f:
        return json.load(f)["cases"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        build.build()
    return abi.load()


def test_schedule_matches_hand_derived_cases():
    for case in _fixture():
        assert ora.window_schedule(case["n_tokens"], case["window"], case["stride"]) == case["windows"], case


@pytest.mark.parametrize("seed", range(6))
def test_schedule_scores_each_prediction_once_with_growing_context(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        window = int(rng.integers(1, 40))
        stride = int(rng.integers(1, window + 1))
        n_tokens = int(rng.integers(0, 300))
        sched = ora.window_schedule(n_tokens, window, stride)
        flat = [p for w in sched for p in w]
        assert flat == list(range(max(n_tokens - 1, 0)))          # once each, in stream order
        for w, ps in enumerate(sched):
            assert ps, "every window adds predictions"
            for p in ps:
                ctx = p - w * stride + 1                           # tokens of the window up to p
                assert 1 <= ctx <= window
                if w > 0:
                    assert ctx >= window - stride + 1             # at least window - stride before it


def test_abi_schedule_arithmetic_matches_oracle(lib):
    """pg_window_count and pg_window_scored (host arithmetic of the library) against the oracle's
    schedule, on the fixture and on random shapes, including partial batches."""
    cases = [(c["n_tokens"], c["window"], c["stride"]) for c in _fixture()]
    rng = np.random.default_rng(11)
    cases += [(int(rng.integers(0, 5000)), int(w), int(rng.integers(1, w + 1)))
              for w in rng.integers(1, 300, size=60)]
    cases += [(65536 * 3 + 17, 2048, 64), (4097, 2048, 64), (2049, 2048, 64), (2050, 2048, 64)]
    for n, L, s in cases:
        sched = ora.window_schedule(n, L, s)
        assert abi.pg_window_count(n, L, s) == len(sched), (n, L, s)
        for w0 in range(0, len(sched), 3):
            nw = min(5, len(sched) - w0)
            assert abi.pg_window_scored(n, L, s, w0, nw) == sum(len(x) for x in sched[w0:w0 + nw])
    assert lib.pg_window_count(10, 4, 5) == -2 and lib.pg_window_count(-1, 4, 2) == -2
    assert lib.pg_window_scored(10, 4, 2, -1, 1) == -2 and lib.pg_window_count(10, 0, 1) == -2


def test_abi_schedule_bounds(lib):
    """Runs that reach past the last window score only up to the end of the stream; a first window
    past the one after the last, or a stream beyond 2^40 tokens, is a shape error; huge counts
    are arithmetic, not loops."""
    n, L, s = 4625, 2048, 64
    count = abi.pg_window_count(n, L, s)
    assert count == 42
    assert lib.pg_window_scored(n, L, s, count, 5) == 0                 # the empty run just past the end
    assert lib.pg_window_scored(n, L, s, count + 1, 1) == -2
    assert lib.pg_window_scored(n, L, s, 0, 2**31 - 1) == n - 1         # every prediction once
    assert lib.pg_window_scored(n, L, s, 40, 2**31 - 1) == sum(len(w) for w in ora.window_schedule(n, L, s)[40:])
    big = 2**40
    assert lib.pg_window_count(big, L, s) == 1 + (big - 1 - L + s - 1) // s
    assert lib.pg_window_scored(big, L, s, 0, 2**31 - 1) == L + (2**31 - 2) * s
    assert lib.pg_window_count(big + 1, L, s) == -2
    assert lib.pg_window_scored(big + 1, L, s, 0, 1) == -2


def _stream(seed=0, n=700, V=300, D=16):
    st = synth.make_stream(seed, n, V, bos_rate=1 / 50, D=D)
    return st["tokens"], st["byte_len"], synth.bf16_to_f64(st["embed"])


def test_context_free_hidden_gives_the_plain_bpb():
    """When a position's hidden state does not depend on its window, the windows change nothing:
    the sliding-window bits per byte is the bits per byte of one forward over all predictions."""
    tokens, blen, E = _stream()
    n_pred, D = len(tokens) - 1, E.shape[1]
    Hpos = np.random.default_rng(3).standard_normal((n_pred, D))
    sched = ora.window_schedule(len(tokens), 64, 16)

    def hid(w, n):
        return Hpos[sched[w]]
    res = ora.sliding_window_eval(tokens, blen, hid, E, 30.0, 64, 16, 5)
    nats, _ = ora.forward(Hpos, E, tokens[1:], 30.0)
    sn, sb, n, b = ora.bpb(nats, tokens[1:], blen)
    assert res["n_scored"] == n == n_pred and res["sum_bytes"] == sb
    assert res["sum_nats"] == pytest.approx(sn, rel=1e-12) and res["bpb"] == pytest.approx(b, rel=1e-12)


def test_batch_gradients_add_up_to_the_whole_stream():
    """With lr = 0 the embedding never changes, and the batches' gradients of their mean losses,
    each times its scored count, add up to the gradient of the summed loss over every prediction."""
    tokens, blen, E = _stream(1)
    D = E.shape[1]

    def hid(w, n):
        return synth.bf16_to_f64(synth.window_hidden(5, w, n, D))
    res = ora.sliding_window_eval(tokens, blen, hid, E, 30.0, 48, 8, 4, lr=0.0)
    assert all("dE" not in b for b in res["batches"])
    tot_E, tot_H = 0.0, []
    for b in res["batches"]:
        H = np.vstack([hid(w, len(ora.window_schedule(len(tokens), 48, 8)[w]))
                       for w in range(b["first_window"], b["first_window"] + 4)
                       if w < len(ora.window_schedule(len(tokens), 48, 8))])
        y = tokens[b["positions"] + 1]
        dH, dE = ora.backward(H, E, y, 30.0, 1.0)
        tot_E = tot_E + dE
        tot_H.append(dH)
    sched = ora.window_schedule(len(tokens), 48, 8)
    Hall = np.vstack([hid(w, len(sched[w])) for w in range(len(sched))])
    pos = np.concatenate([b["positions"] for b in res["batches"]])
    dH_all, dE_all = ora.backward(Hall, E, tokens[pos + 1], 30.0, 1.0)
    np.testing.assert_allclose(tot_E, dE_all, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(np.vstack(tot_H), dH_all, rtol=1e-9, atol=1e-12)


def test_score_first_ttt():
    """The first batch is scored before any update (its nats equal those without training), later
    batches with the updated embedding (they differ), every batch's embedding is the one the
    previous batches' steps produced, and one step lowers the loss of the batch it was taken on."""
    tokens, blen, E = _stream(2, n=900, V=200, D=16)
    D = E.shape[1]

    def hid(w, n):
        return synth.bf16_to_f64(synth.window_hidden(6, w, n, D))
    base = ora.sliding_window_eval(tokens, blen, hid, E, 30.0, 64, 16, 6, lr=0.0)
    lr = 200.0
    tt = ora.sliding_window_eval(tokens, blen, hid, E, 30.0, 64, 16, 6, lr=lr)
    assert len(tt["batches"]) >= 4
    np.testing.assert_array_equal(tt["batches"][0]["nats"], base["batches"][0]["nats"])
    np.testing.assert_array_equal(tt["batches"][0]["embed"], E)
    for k in range(1, len(tt["batches"])):
        assert not np.array_equal(tt["batches"][k]["embed"], E)
        assert not np.allclose(tt["batches"][k]["nats"], base["batches"][k]["nats"], rtol=0, atol=1e-9)
    sched = ora.window_schedule(len(tokens), 64, 16)
    b0 = tt["batches"][0]
    H0 = np.vstack([hid(w, len(sched[w])) for w in range(0, 6)])
    y0 = tokens[b0["positions"] + 1]
    after, _ = ora.forward(H0, tt["batches"][1]["embed"], y0, 30.0)
    assert after.mean() < b0["nats"].mean()
    # the step itself: float32 master weights, each operation rounded to float32, bf16 for the head
    m = E.astype(np.float32) - np.float32(lr) * b0["dE"].astype(np.float32)
    np.testing.assert_array_equal(tt["batches"][1]["embed"], ora._bf16_round(m))
