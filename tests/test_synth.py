"""The seeded generator: determinism and the distributions the workloads ask for."""
import hashlib
import math

import numpy as np
import pytest

from lm_head_cross_pg_amd import synth


def _digest(inp):
    h = hashlib.sha256()
    for k in ("hidden", "embed", "target", "byte_len", "mask"):
        if inp[k] is not None:
            h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def test_deterministic_and_seed_sensitive():
    a = synth.make_inputs("tiny_f32", seed=42)
    b = synth.make_inputs("tiny_f32", seed=42)
    c = synth.make_inputs("tiny_f32", seed=1234)
    assert _digest(a) == _digest(b) != _digest(c)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1e-40, 3.0e38], dtype=np.float32)
    bits = synth.bf16_bits(x)
    back = synth.bf16_to_f64(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # tie -> even (mantissa 0)
    assert back[2] == 1.0 + 4 * 2 ** -8         # tie -> even (rounds up)
    assert back[3] == 1.0
    assert back[4] == -2.5
    # every value is within half an ulp of bf16
    rel = np.abs(back[:5] - x[:5]) / np.abs(x[:5])
    assert np.all(rel <= 2 ** -8)


def test_tiny_shapes_and_laws():
    inp = synth.make_inputs("tiny_f32", seed=0)
    assert inp["hidden"].shape == (256, 64) and inp["hidden"].dtype == np.float32
    assert inp["embed"].shape == (512, 64)
    assert inp["byte_len"].min() >= 1 and inp["byte_len"].max() <= 8
    assert abs(inp["embed"].std() - 0.02) < 0.001
    assert inp["mask"] is None


@pytest.mark.slow
def test_main_workload_statistics():
    inp = synth.make_inputs("fwd_v8192", seed=0)
    T, D, V = 65536, 512, 8192
    assert inp["hidden"].shape == (T, D) and inp["hidden"].dtype == np.uint16
    H = synth.bf16_to_f64(inp["hidden"][:4096])
    rms = np.sqrt((H ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1) < 4e-3)                   # unit RMS up to bf16 rounding
    E = synth.bf16_to_f64(inp["embed"])
    assert abs(E.std() - 0.02) < 2e-4
    y = inp["target"]
    pmf = synth.zipf_pmf(V, 1.1)
    assert abs(pmf[0] - 0.1533) < 1e-3
    assert abs(np.mean(y == 0) - pmf[0]) < 5 * math.sqrt(pmf[0] / T)
    blen = inp["byte_len"]
    assert blen.min() >= 1 and blen.max() <= 16
    assert abs(blen.mean() - 3.7) < 0.1


def test_baseline_vocab_bytes():
    inp = synth.make_inputs("fwd_v1024", seed=0, T=2048)
    blen = inp["byte_len"]
    assert blen.min() >= 1 and blen.max() <= 12 and abs(blen.mean() - 2.5) < 0.15
    assert abs(synth.zipf_pmf(1024, 1.1)[0] - 0.1791) < 1e-3


def test_masked_workload_bos_and_mask():
    inp = synth.make_inputs("masked_stride64", seed=0)
    mask, y, blen = inp["mask"], inp["target"], inp["byte_len"]
    assert mask.sum() == 2048
    assert np.all(mask.reshape(32, 2048)[:, -64:] == 1) and np.all(mask.reshape(32, 2048)[:, :-64] == 0)
    assert blen[0] == 0
    rate = np.mean(y == 0)
    assert abs(rate - 1 / 700) < 4 * math.sqrt((1 / 700) / 65536)
    assert np.all(y[y != 0] >= 1)


def test_stress_reaches_several_caps():
    inp = synth.make_inputs("stress", seed=0)
    H = synth.bf16_to_f64(inp["hidden"])
    E = synth.bf16_to_f64(inp["embed"])
    z = H @ E.T
    assert np.max(np.abs(z)) > 5 * 30.0
