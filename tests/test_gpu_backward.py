"""GPU parity of the backward (dH, dE) against the float64 oracle through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from oracle import oracle as ora
from tests.gpu_helpers import GRAD_RL2, NATS_ATOL, ensure_lib, host_inputs, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def workload(name, **over):
    return dataclasses.replace(synth.WORKLOADS[name], **over)


def run_bwd(inp, softcap=None, mask=None, grad_scale=None, fused=False):
    """The backward on the GPU against the oracle; fused: through pg_lmhead_ce_fwd_bwd, whose nats
    and lse are checked against the oracle's forward as well."""
    T, D, V = inp["T"], inp["D"], inp["V"]
    c = inp["softcap"] if softcap is None else softcap
    mask = inp["mask"] if mask is None else mask
    n_scored = T if mask is None else int(mask.sum())
    g = (1.0 / max(n_scored, 1)) if grad_scale is None else grad_scale
    print(f"[case] bwd{' fused' if fused else ''} {inp['workload']} seed={inp['seed']} T={T} D={D} V={V} c={c} "
          f"masked={mask is not None}", flush=True)
    d = abi.to_device(inp)
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    nats = torch.empty(T, device="cuda")
    lse = torch.empty(T, device="cuda")
    dH = torch.full((T, D), float("nan"), device="cuda")
    dE = torch.full((V, D), float("nan"), device="cuda")
    if fused:
        if isinstance(c, tuple):
            abi.pg_lmhead_ce_fwd_bwd_asym(d["hidden"], d["embed"], d["target"], mask_t, c[0], c[1], g, nats, lse,
                                          dH, dE)
        else:
            abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], mask_t, c, g, nats, lse, dH, dE)
        torch.cuda.synchronize()
        H, E = host_inputs(inp)
        onats, olse = ora.forward(H, E, inp["target"], c, mask)
        assert np.max(np.abs(nats.cpu().numpy() - onats)) <= NATS_ATOL
        assert np.max(np.abs(lse.cpu().numpy() - olse)) <= NATS_ATOL
    elif isinstance(c, tuple):
        abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], mask_t, c[0], c[1], nats, lse)
        abi.pg_lmhead_ce_bwd_asym(d["hidden"], d["embed"], d["target"], mask_t, lse, c[0], c[1], g, dH, dE)
    else:
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask_t, c, nats, lse)
        abi.pg_lmhead_ce_bwd(d["hidden"], d["embed"], d["target"], mask_t, lse, c, g, dH, dE)
    torch.cuda.synchronize()
    dH, dE = dH.cpu().numpy().astype(np.float64), dE.cpu().numpy().astype(np.float64)
    H, E = host_inputs(inp)
    odH, odE = ora.backward(H, E, inp["target"], c, g, mask)
    assert np.all(np.isfinite(dH)) and np.all(np.isfinite(dE))
    cp, cn = (c if isinstance(c, tuple) else (c, c))
    one_pass = fused and inp["dtype"] == "bf16" and D in (32, 64, 128, 256, 512) and 0 < cp <= 40 and 0 < cn <= 40
    if not np.any(odH) and not np.any(odE):
        # V = 1: the softmax of one entry is 1 and the gradient exactly 0.
        if one_pass:
            # p_y = e^-nats, and the forward's nats is exactly 0 there (its target term is all of the sum)
            assert not np.any(dH) and not np.any(dE)
        else:
            # the recomputing backward forms p = 2^(s log2 e - lse log2 e) from the saved lse, which
            # carries a few float32 roundings of M = c log2 e (ulp 3.8e-6 at c = 30): |p - 1| stays
            # below 3e-5, so |dH| <= 3e-5 g max|E| and |dE| <= 3e-5 g sum_t max_d |H[t]|
            tH = 3e-5 * g * np.max(np.abs(E))
            tE = 3e-5 * g * np.sum(np.max(np.abs(H), axis=1))
            assert np.max(np.abs(dH)) <= tH and np.max(np.abs(dE)) <= tE, (np.max(np.abs(dH)), tH,
                                                                            np.max(np.abs(dE)), tE)
        return dH, dE
    assert rel_l2(dH, odH) <= GRAD_RL2, rel_l2(dH, odH)
    assert rel_l2(dE, odE) <= GRAD_RL2, rel_l2(dE, odE)
    if mask is not None:
        assert np.all(dH[~mask.astype(bool)] == 0.0)
    return dH, dE


def test_fd_shape_f32():
    run_bwd(synth.make_inputs("fd", 0))


def test_fd_shape_bf16():
    run_bwd(synth.make_inputs(workload("fd", dtype="bf16"), 0))


@pytest.mark.parametrize("seed", [0, 42])
def test_training_shape_small(seed):
    run_bwd(synth.make_inputs("train_v8192", seed, T=700))


@pytest.mark.parametrize("D,V", [(64, 1000), (128, 777), (256, 300), (48, 200), (512, 1), (64, 1)])
def test_widths(D, V):
    run_bwd(synth.make_inputs(workload("train_v8192", D=D, V=V, T=520, stream=70 + D), 0))


@pytest.mark.parametrize("c", [0.0, 5.0, 50.0])
def test_caps(c):
    run_bwd(synth.make_inputs(workload("train_v8192", V=1500, T=400, stream=80, softcap=c), 1), softcap=c)


def test_stress():
    run_bwd(synth.make_inputs("stress", 0))


def test_masked():
    inp = synth.make_inputs("masked_stride64", 0, T=4096)
    run_bwd(inp)


def test_masked_full_size():
    """Stride-64 scoring at T = 65536: 2048 scored rows, every other dH row zero."""
    run_bwd(synth.make_inputs("masked_stride64", 0))


# ------------------------------------------------ forward and backward in one call (pg_lmhead_ce_fwd_bwd)

def test_fused_fd_shapes():
    run_bwd(synth.make_inputs("fd", 0), fused=True)                                  # f32: two calls
    run_bwd(synth.make_inputs(workload("fd", dtype="bf16"), 0), fused=True)          # one pass


@pytest.mark.parametrize("seed", [0, 42])
def test_fused_training_shape_small(seed):
    run_bwd(synth.make_inputs("train_v8192", seed, T=700), fused=True)


@pytest.mark.parametrize("D,V", [(32, 4000), (64, 1000), (128, 777), (256, 300), (48, 200), (512, 130),
                                 (512, 1), (64, 65)])
def test_fused_widths(D, V):
    run_bwd(synth.make_inputs(workload("train_v8192", D=D, V=V, T=520, stream=170 + D), 0), fused=True)


@pytest.mark.parametrize("c", [0.0, 5.0, 40.0, 50.0])
def test_fused_caps(c):
    """c = 0 and c = 50 (beyond the fixed shift) take the two calls; 5 and 40 the single pass."""
    run_bwd(synth.make_inputs(workload("train_v8192", V=1500, T=400, stream=180, softcap=c), 1), softcap=c,
            fused=True)


def test_fused_stress_and_large_logits():
    """|z| up to 5c (every block leaves the series) and hidden x 8 at D = 512 (mixed blocks)."""
    run_bwd(synth.make_inputs("stress", 0), fused=True)
    run_bwd(synth.make_inputs(workload("train_v8192", T=1500, stream=181, hidden_scale=8.0), 0), fused=True)


@pytest.mark.parametrize("T", [1, 255, 257, 4097])
def test_fused_ragged_rows(T):
    run_bwd(synth.make_inputs(workload("train_v8192", V=2048, stream=182), 0, T=T), fused=True)


def test_fused_masked():
    run_bwd(synth.make_inputs("masked_stride64", 0, T=4096), fused=True)
    run_bwd(synth.make_inputs("masked_stride64", 1), fused=True)


def test_fused_grad_scale_zero_and_two():
    inp = synth.make_inputs("train_v8192", 3, T=300)
    T, D, V = inp["T"], inp["D"], inp["V"]
    d = abi.to_device(inp)
    nats, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    dH = torch.full((T, D), float("nan"), device="cuda")
    dE = torch.full((V, D), float("nan"), device="cuda")
    abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], None, inp["softcap"], 0.0, nats, lse, dH, dE)
    torch.cuda.synchronize()
    assert torch.all(dH == 0).item() and torch.all(dE == 0).item()
    run_bwd(inp, grad_scale=2.0, fused=True)


def _full_size_check(inp, rows_extra, seed, label, caps=None):
    """Both training entry points on one full-size input: sampled dH rows and dE rows against the
    oracle (computed once), the <dH, H> = <dE, E> identity, and nats / lse on sampled rows. caps:
    (c_pos, c_neg) for the asymmetric entry points."""
    from tests.gpu_helpers import oracle_forward_chunked
    T, D, V = inp["T"], inp["D"], inp["V"]
    c = inp["softcap"] if caps is None else caps
    g = 1.0 / T
    d = abi.to_device(inp)
    H, E = host_inputs(inp)
    y = inp["target"]
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(T, 256, replace=False), rows_extra]))
    vrows = np.unique(np.concatenate([[0, 1, 2, 100, V - 1], rng.choice(V, 59, replace=False)]))
    onats, olse = oracle_forward_chunked(H, E, y, c)
    odH, _ = ora.backward(H[rows], E, y[rows], c, g)
    odE = ora.embed_grad_rows(H, E, y, c, g, olse, vrows)
    for fused in (False, True):
        print(f"[case] {label} fused={fused}", flush=True)
        nats = torch.empty(T, device="cuda")
        lse = torch.empty(T, device="cuda")
        dH = torch.empty((T, D), device="cuda")
        dE = torch.empty((V, D), device="cuda")
        if caps is not None and fused:
            abi.pg_lmhead_ce_fwd_bwd_asym(d["hidden"], d["embed"], d["target"], None, c[0], c[1], g, nats, lse,
                                          dH, dE)
        elif caps is not None:
            abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], None, c[0], c[1], nats, lse)
            abi.pg_lmhead_ce_bwd_asym(d["hidden"], d["embed"], d["target"], None, lse, c[0], c[1], g, dH, dE)
        elif fused:
            abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], None, c, g, nats, lse, dH, dE)
        else:
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse)
            abi.pg_lmhead_ce_bwd(d["hidden"], d["embed"], d["target"], None, lse, c, g, dH, dE)
        torch.cuda.synchronize()
        n, l = nats.cpu().numpy(), lse.cpu().numpy()
        assert np.max(np.abs(n[rows] - onats[rows])) <= NATS_ATOL
        assert np.max(np.abs(l[rows] - olse[rows])) <= NATS_ATOL
        dHn, dEn = dH.cpu().numpy().astype(np.float64), dE.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(dHn)) and np.all(np.isfinite(dEn))
        assert rel_l2(dHn[rows], odH) <= GRAD_RL2, rel_l2(dHn[rows], odH)
        assert rel_l2(dEn[vrows], odE) <= GRAD_RL2, rel_l2(dEn[vrows], odE)
        a, b = np.sum(dHn * H), np.sum(dEn * E)
        assert abs(a - b) <= 1e-2 * abs(b), (a, b)


def test_training_full_size_sampled():
    """T = 65536, D = 512, V = 8192, mean loss (g = 1/T), in the benchmark's launch configuration,
    through both training entry points."""
    inp = synth.make_inputs("train_v8192", 0)
    T = inp["T"]
    _full_size_check(inp, [0, 255, 256, T - 1], 11, "train full size")


def test_training_full_size_sampled_asymmetric():
    """The same at caps (30, 20), through both asymmetric training entry points."""
    inp = synth.make_inputs("train_v8192", 0)
    T = inp["T"]
    _full_size_check(inp, [0, 255, 256, T - 1], 13, "train full size caps (30, 20)", caps=(30.0, 20.0))


def test_dz_beyond_2_31_elements():
    """T = 300,007 rows at V = 8192: dZ holds 2.46e9 elements (4.9 GB), so its block offsets and
    the GEMMs' reads of it pass 2^31. D = 32 keeps the oracle's full forward cheap. Both training
    entry points."""
    inp = synth.make_inputs(workload("train_v8192", T=300007, D=32, stream=60, hidden_scale=8.0), 0)
    T = inp["T"]
    _full_size_check(inp, [0, 262143, 262144, T - 1], 12, "dZ beyond 2^31")


@pytest.mark.parametrize("caps", [(30.0, 10.0), (10.0, 30.0), (30.0, 0.0), (0.0, 20.0)])
def test_asymmetric_caps(caps):
    """Gradients with separate caps for z >= 0 and z < 0; logits reach both caps' curvature."""
    w = workload("train_v8192", T=520, V=1500, stream=99, hidden_scale=40.0)
    run_bwd(synth.make_inputs(w, 1), softcap=caps)


@pytest.mark.parametrize("caps", [(30.0, 10.0), (10.0, 30.0), (30.0, 20.0), (6.0, 40.0), (30.0, 0.0), (0.0, 20.0),
                                  (50.0, 20.0)])
@pytest.mark.parametrize("scale", [1.0, 40.0])
def test_fused_asymmetric_caps(caps, scale):
    """pg_lmhead_ce_fwd_bwd_asym: one pass when both caps lie in (0, 40], with each side's slope
    stored in the common scale of the row factor; the two calls otherwise (an uncapped side, a cap
    above 40). Initialisation-scale logits (the tanh series) and hidden x 40 (both caps' curvature,
    the exact form)."""
    w = workload("train_v8192", T=520, V=1500, stream=99, hidden_scale=scale)
    run_bwd(synth.make_inputs(w, 1), softcap=caps, fused=True)


def test_fused_asymmetric_widths_masked_ragged():
    for D, V in ((32, 700), (64, 1000), (128, 777), (256, 300), (48, 200)):
        run_bwd(synth.make_inputs(workload("train_v8192", D=D, V=V, T=520, stream=190 + D, hidden_scale=8.0), 0),
                softcap=(30.0, 15.0), fused=True)
    run_bwd(synth.make_inputs("masked_stride64", 0, T=4096), softcap=(30.0, 15.0), fused=True)
    run_bwd(synth.make_inputs(workload("train_v8192", V=2048, stream=195), 0, T=257), softcap=(20.0, 30.0),
            fused=True)
    run_bwd(synth.make_inputs("stress", 0), softcap=(30.0, 10.0), fused=True)


def test_asymmetric_caps_generic_and_masked():
    run_bwd(synth.make_inputs(workload("fd", stream=100), 0), softcap=(3.0, 1.0))
    run_bwd(synth.make_inputs("masked_stride64", 0, T=4096), softcap=(30.0, 15.0))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,over", [("train_v8192", {"T": 600, "V": 1500, "stream": 140}),
                                       ("fd", {"stream": 141})])
def test_out_of_range_target_poisons_gradients(fused, name, over):
    """A scored row whose target lies outside [0, V) has NaN nats; its dH row and all of dE are NaN
    (the oracle's reading), every other dH row is as if that row were unscored. Unscored, the same
    rows change nothing. MFMA (bf16, D = 512) and vector (f32) kernels, both training paths."""
    inp = synth.make_inputs(workload(name, **over), 0)
    T, D, V, c = inp["T"], inp["D"], inp["V"], inp["softcap"]
    y = inp["target"].copy()
    bad = np.array([5, T - 3])
    y[bad[0]], y[bad[1]] = V, -1
    print(f"[case] poison {name} fused={fused} T={T} D={D} V={V}", flush=True)
    d = abi.to_device(inp)
    yt = torch.from_numpy(y).cuda()
    H, E = host_inputs(inp)
    g = 1.0 / T
    keep = np.ones(T, np.uint8)
    keep[bad] = 0
    odH, odE = ora.backward(H, E, y, c, g)
    assert np.isnan(odH[bad]).all() and np.isnan(odE).all()
    mdH, mdE = ora.backward(H, E, y, c, g, keep)
    np.testing.assert_allclose(np.delete(odH, bad, axis=0), np.delete(mdH, bad, axis=0), rtol=1e-12, atol=0)
    for mask in (None, keep):
        mask_t = None if mask is None else torch.from_numpy(mask).cuda()
        nats, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
        dH = torch.zeros((T, D), device="cuda")
        dE = torch.zeros((V, D), device="cuda")
        if fused:
            abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], yt, mask_t, c, g, nats, lse, dH, dE)
        else:
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], yt, mask_t, c, nats, lse)
            abi.pg_lmhead_ce_bwd(d["hidden"], d["embed"], yt, mask_t, lse, c, g, dH, dE)
        torch.cuda.synchronize()
        n = nats.cpu().numpy()
        dHn, dEn = dH.cpu().numpy().astype(np.float64), dE.cpu().numpy().astype(np.float64)
        good = np.delete(np.arange(T), bad)
        assert np.all(np.isfinite(dHn[good])) and np.all(np.isfinite(n[good]))
        assert rel_l2(dHn[good], mdH[good]) <= GRAD_RL2
        if mask is None:
            assert np.isnan(n[bad]).all() and np.isnan(dHn[bad]).all() and np.isnan(dEn).all()
        else:
            assert np.all(n[bad] == 0.0) and np.all(dHn[bad] == 0.0)
            assert np.all(np.isfinite(dEn)) and rel_l2(dEn, mdE) <= GRAD_RL2


@pytest.mark.parametrize("path,over,masked", [
    ("fused", {}, False), ("fused", {}, True), ("two_calls", {}, False), ("two_calls", {}, True),
    ("fused", {"D": 48}, True), ("two_calls", {"dtype": "f32", "D": 64}, False),
    ("fused_asym", {}, True), ("fused", {"softcap": 50.0}, True)])
def test_without_dhidden(path, over, masked):
    """dhidden = NULL leaves dH out (its product is not run): dE, nats and lse are those of the call
    that also computes dH, bit for bit, on the one-call path (where the forward writes dZ, and its
    fallbacks: a generic width, a cap above the fixed-shift range), the two calls, and both
    precisions, masked and not."""
    w = workload("train_v8192", T=700, V=1500, stream=140 + len(over), **over)
    inp = synth.make_inputs(w, 0)
    T, D, V = inp["T"], inp["D"], inp["V"]
    c = inp["softcap"]
    mask = (np.random.default_rng(9).random(T) < 0.4).astype(np.uint8) if masked else None
    print(f"[case] no dH {path} {over} masked={masked}", flush=True)
    d = abi.to_device(inp)
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    g = 1.0 / T
    res = []
    for with_dh in (True, False):
        nats = torch.empty(T, device="cuda")
        lse = torch.empty(T, device="cuda")
        dH = torch.full((T, D), float("nan"), device="cuda") if with_dh else None
        dE = torch.full((V, D), float("nan"), device="cuda")
        if path == "fused":
            abi.pg_lmhead_ce_fwd_bwd(d["hidden"], d["embed"], d["target"], mask_t, c, g, nats, lse, dH, dE)
        elif path == "fused_asym":
            abi.pg_lmhead_ce_fwd_bwd_asym(d["hidden"], d["embed"], d["target"], mask_t, 30.0, 20.0, g, nats, lse,
                                          dH, dE)
        else:
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask_t, c, nats, lse)
            abi.pg_lmhead_ce_bwd(d["hidden"], d["embed"], d["target"], mask_t, lse, c, g, dH, dE)
        torch.cuda.synchronize()
        res.append((nats.cpu().numpy(), lse.cpu().numpy(), dE.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        np.testing.assert_array_equal(a, b)
    assert np.all(np.isfinite(res[1][2]))


@pytest.mark.parametrize("path", ["fused", "two_calls"])
def test_no_rows_and_empty_mask(path):
    """Nothing to learn from: T = 0 rows, and 300 rows none of which is scored. dembed comes back
    exactly zero (the caller's buffer is overwritten, not left as it was), dhidden's rows too."""
    inp = synth.make_inputs(workload("train_v8192", T=300, V=1500, stream=150), 0)
    d = abi.to_device(inp)
    V, D = inp["V"], inp["D"]
    for T, mask in ((0, None), (300, torch.zeros(300, dtype=torch.uint8, device="cuda"))):
        print(f"[case] no rows {path} T={T} masked={mask is not None}", flush=True)
        H, y = d["hidden"][:T], d["target"][:T]
        nats = torch.full((T,), 5.0, device="cuda")
        lse = torch.full((T,), 5.0, device="cuda")
        dH = torch.full((T, D), 3.0, device="cuda")
        dE = torch.full((V, D), 3.0, device="cuda")
        if path == "fused":
            abi.pg_lmhead_ce_fwd_bwd(H, d["embed"], y, mask, 30.0, 1.0, nats, lse, dH, dE)
        else:
            abi.pg_lmhead_ce_fwd(H, d["embed"], y, mask, 30.0, nats, lse)
            abi.pg_lmhead_ce_bwd(H, d["embed"], y, mask, lse, 30.0, 1.0, dH, dE)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dE).item() == 0
        assert torch.count_nonzero(dH).item() == 0 and torch.count_nonzero(nats).item() == 0
