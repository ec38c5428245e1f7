"""GPU parity of the fused forward and the bits-per-byte reduction against the float64 oracle,
through the C ABI, on seeded synthetic inputs."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from oracle import oracle as ora
from tests.gpu_helpers import (BPB_RTOL, NATS_ATOL, ensure_lib, gpu_bpb, host_inputs,
                               oracle_forward_chunked)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def workload(name, **over):
    return dataclasses.replace(synth.WORKLOADS[name], **over)


def run(inp, softcap=None, mask=None, sample_rows=None, check_bpb=True, byte_per_pos=None):
    """Forward + BPB on the GPU vs the oracle; returns (nats_gpu, lse_gpu)."""
    T, D, V = inp["T"], inp["D"], inp["V"]
    c = inp["softcap"] if softcap is None else softcap
    mask = inp["mask"] if mask is None else mask
    d = abi.to_device(inp)
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    print(f"[case] {inp['workload']} seed={inp['seed']} T={T} D={D} V={V} c={c} masked={mask is not None}", flush=True)
    nats_t = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    lse_t = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    if isinstance(c, tuple):
        abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], mask_t, c[0], c[1], nats_t, lse_t)
    else:
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask_t, c, nats_t, lse_t)
    torch.cuda.synchronize()
    nats, lse = nats_t.cpu().numpy().astype(np.float64), lse_t.cpu().numpy().astype(np.float64)
    H, E = host_inputs(inp)
    y = inp["target"]
    scored = np.ones(T, bool) if mask is None else mask.astype(bool)
    if sample_rows is None:
        rows = np.nonzero(scored)[0]
    else:
        rows = np.asarray(sample_rows)
    onats = np.zeros(T)
    olse = np.zeros(T)
    if len(rows):
        onats[rows], olse[rows] = oracle_forward_chunked(H[rows], E, y[rows], c)
    err = np.max(np.abs(nats[rows] - onats[rows])) if len(rows) else 0.0
    assert err <= NATS_ATOL, f"max |nats - oracle| = {err}"
    # the target's logit is taken from the sum that forms lse, so no row can come out negative
    assert np.all(nats[rows] >= 0.0), np.min(nats[rows])
    assert np.max(np.abs(lse[rows] - olse[rows]), initial=0.0) <= NATS_ATOL
    assert np.all(nats[~scored] == 0.0) and np.all(lse[~scored] == 0.0)
    if check_bpb:
        bpp_t = None if byte_per_pos is None else torch.from_numpy(byte_per_pos).cuda()
        out = gpu_bpb(nats_t, d, V, mask_t, bpp_t)
        # the reduction itself: float64 sums of the GPU's own nats, exactly the same rows
        assert out[2] == scored.sum()
        assert out[0] == pytest.approx(np.sum(nats[scored]), rel=1e-12, abs=1e-9)
        if sample_rows is None:
            sn, sb, n, b = ora.bpb(onats, y, inp["byte_len"], mask, byte_per_pos)
            assert out[1] == sb and out[2] == n
            if math.isfinite(b):
                # (a one-entry vocabulary costs exactly nothing on both sides, so b = 0 means out = 0)
                assert abs(out[3] - b) <= BPB_RTOL * abs(b), (out[3], b)
            else:
                assert (math.isnan(b) and math.isnan(out[3])) or out[3] == b
    return nats, lse


@pytest.mark.parametrize("seed", [0, 42, 1234])
def test_tiny_f32(seed):
    run(synth.make_inputs("tiny_f32", seed))


@pytest.mark.parametrize("seed", [0, 42, 1234])
def test_baseline_vocab_full_size(seed):
    """T = 4 x 2048, D = 512, V = 1024: vocabulary split over workgroups, every row checked."""
    run(synth.make_inputs("fwd_v1024", seed))


@pytest.mark.parametrize("T", [1, 255, 1000, 4097])
def test_main_shape_ragged_rows(T):
    run(synth.make_inputs("fwd_v8192", 0, T=T))


@pytest.mark.parametrize("D,V", [(32, 128), (64, 1000), (128, 777), (256, 2048), (512, 100), (512, 1),
                                 (48, 300), (512, 65)])
def test_widths_and_ragged_vocab(D, V):
    w = workload("fwd_v8192", D=D, V=V, T=700, stream=40 + D)
    run(synth.make_inputs(w, 1))


@pytest.mark.parametrize("c", [0.0, 50.0, 5.0])
def test_other_caps(c):
    """c = 0 (no cap) and c > 40 take the running-maximum path; c = 5 bends the logits."""
    w = workload("fwd_v8192", T=600, V=3000, stream=50, softcap=c)
    run(synth.make_inputs(w, 2), softcap=c)


@pytest.mark.parametrize("seed", [0, 42])
def test_softcap_stress(seed):
    inp = synth.make_inputs("stress", seed)
    nats, _ = run(inp)
    H, E = host_inputs(inp)
    assert np.max(np.abs(H @ E.T)) > 5 * 30.0


def test_stress_f32_and_bf16_generic():
    inp = synth.make_inputs(workload("stress", dtype="f32", D=40, stream=61), 0)
    run(inp)


@pytest.mark.parametrize("seed", [0, 42, 1234])
def test_masked_stride64_small(seed):
    run(synth.make_inputs("masked_stride64", seed, T=8192))


@pytest.mark.parametrize("T", [1, 15, 16, 17, 4095, 4097, 16383, 16384, 16385, 50001])
def test_random_masks_ragged(T):
    """Scored-row selection over ragged lengths around its 16-row, 4096-row and 16 Ki-row steps:
    random masks of density 0.3, all-ones, and masks of arbitrary nonzero bytes; unscored rows
    must come out 0, scored rows as the oracle's."""
    w = workload("fwd_v1024", T=T, D=64, V=512, stream=120)
    inp = synth.make_inputs(w, 0)
    rng = np.random.default_rng(T)
    run(inp, mask=(rng.random(T) < 0.3).astype(np.uint8))
    run(inp, mask=np.ones(T, np.uint8))
    # any nonzero byte marks a scored row
    vals = np.array([0, 0, 0, 1, 2, 127, 128, 255], np.uint8)
    run(inp, mask=vals[rng.integers(0, len(vals), T)])


def test_random_mask_beyond_multi_workgroup_selection():
    """T = 1,100,000 rows (past the 2^20 rows that the multi-workgroup scored-row selection takes;
    the single-workgroup kernel runs) with a random mask of density 0.3, at D = 32, V = 128."""
    T = 1_100_000
    inp = synth.make_inputs(workload("fwd_v1024", T=T, D=32, V=128, stream=121), 0)
    run(inp, mask=(np.random.default_rng(5).random(T) < 0.3).astype(np.uint8))


def test_masked_stride64_full_size():
    run(synth.make_inputs("masked_stride64", 0))


def test_main_full_size_sampled():
    """T = 65536, D = 512, V = 8192 in the benchmark's launch configuration: sampled rows against
    the oracle, the whole BPB against the oracle's full forward."""
    inp = synth.make_inputs("fwd_v8192", 0)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(65536, 384, replace=False), [0, 1, 255, 256, 65535]]))
    nats, _ = run(inp, sample_rows=rows)
    H, E = host_inputs(inp)
    onats, _ = oracle_forward_chunked(H, E, inp["target"], 30.0)
    assert np.max(np.abs(nats - onats)) <= NATS_ATOL
    assert np.all(nats >= 0.0)
    sn, sb, n, b_ora = ora.bpb(onats, inp["target"], inp["byte_len"])
    # the GPU's own reduction of its nats: every output against the oracle's full forward
    d = abi.to_device(inp)
    out = gpu_bpb(torch.from_numpy(nats.astype(np.float32)).cuda(), d, inp["V"])
    assert out[1] == sb and out[2] == n == 65536
    assert abs(out[0] - sn) <= BPB_RTOL * sn
    assert abs(out[3] - b_ora) <= BPB_RTOL * b_ora, (out[3], b_ora)


@pytest.mark.parametrize("D,V", [(512, 65), (512, 1000), (512, 8192), (64, 300), (48, 100)])
def test_near_certain_targets(D, V):
    """p(target) -> 1: each hidden row points along its target's embedding row, so the target's
    logit (~100, capped to ~30) dwarfs the others (~N(0, (100/sqrt(D))^2)): at D = 512 nats falls
    to ~1e-9. Rows of
    the ordinary workload are mixed in. No row may come out negative, and every row stays within
    the nats tolerance of the oracle. The bits per byte of such a batch is far below what a float32
    lse resolves, so it is not compared here."""
    w = workload("fwd_v8192", T=640, D=D, V=V, stream=130 + D)
    inp = synth.make_inputs(w, 0)
    H, E = host_inputs(inp)
    y = inp["target"]
    k = 100.0 / np.sum(E[y] ** 2, axis=1)
    Hs = H.copy()
    Hs[::2] = (E[y] * k[:, None])[::2]                 # even rows near-certain, odd rows as drawn
    inp = dict(inp, hidden=synth.bf16_bits(Hs.astype(np.float32)))
    nats, _ = run(inp, check_bpb=False)
    assert np.all(nats >= 0.0)
    if D == 512:   # at smaller widths the other logits grow as 100 / sqrt(D) and p(target) stays below 1
        assert np.max(nats[::2]) < 1e-4


def test_large_logits_exact_path():
    """D = 512, V = 8192, c = 30 with hidden x 8: z has standard deviation ~3.6, so every 32 x 32
    block holds some |z| > c/8 and the epilogue takes the exact softcap instead of the series."""
    inp = synth.make_inputs(workload("fwd_v8192", T=4096, stream=97, hidden_scale=8.0), 0)
    H, E = host_inputs(inp)
    z = H[:64] @ E.T
    assert np.mean(np.abs(z) > 30.0 / 8) > 0.2
    run(inp)


@pytest.mark.parametrize("caps", [30.0, (30.0, 20.0), (20.0, 30.0), (6.0, 40.0)])
def test_series_and_exact_blocks_mixed(caps):
    """Most blocks take the tanh series; the embedding rows of a few vocabulary tiles are scaled by
    32 (exact in bf16) so that their blocks miss it. The forward then switches to the exact form
    for a run of blocks and back to the series; every row is checked against the oracle. With
    asymmetric caps the series threshold is the smaller cap / 8 and each side takes its own
    series coefficients; at caps (6, 40) the threshold is 0.75 and most blocks miss it."""
    inp = synth.make_inputs(workload("fwd_v8192", T=2048, stream=98), 0)
    E = synth.as_f64(inp["embed"], inp["dtype"]).copy()
    for tile in (3, 40, 41, 100):
        E[tile * 64:(tile + 1) * 64] *= 32.0
    inp = dict(inp, embed=synth.bf16_bits(E.astype(np.float32)))
    H, E2 = host_inputs(inp)
    assert np.array_equal(E2, E)
    z = H[:32] @ E2[3 * 64:4 * 64].T
    assert np.max(np.abs(z)) > 30.0 / 8
    run(inp, softcap=caps)


def test_ragged_full_width_direct():
    """65,436 rows: still one vocabulary split per workgroup (direct write), ragged last tile."""
    inp = synth.make_inputs("fwd_v8192", 3, T=65436)
    rows = np.array([0, 17, 30000, 65279, 65280, 65400, 65435])
    run(inp, sample_rows=rows, check_bpb=False)


def test_byte_sidecar():
    inp = synth.make_inputs("fwd_v1024", 5, T=3000)
    bpp = np.random.default_rng(1).integers(0, 9, size=3000).astype(np.int32)
    run(inp, byte_per_pos=bpp)


def test_empty_mask_zero_bytes_and_poison():
    inp = synth.make_inputs("fwd_v8192", 9, T=300)
    d = abi.to_device(inp)
    T, V = 300, 8192
    # empty mask: zero nats, BPB = 0/0
    mask = torch.zeros(T, dtype=torch.uint8, device="cuda")
    nats = torch.full((T,), 7.0, device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask, 30.0, nats, None)
    out = gpu_bpb(nats, d, V, mask)
    assert torch.all(nats == 0).item() and out[2] == 0 and math.isnan(out[3])
    # zero bytes everywhere: +inf
    abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, 30.0, nats, None)
    d0 = dict(d, byte_len=torch.zeros(V, dtype=torch.int32, device="cuda"))
    assert math.isinf(gpu_bpb(nats, d0, V)[3])
    # out-of-range targets and a NaN hidden row poison only their own rows
    y = d["target"].clone()
    y[5] = V
    y[6] = -3
    h = d["hidden"].clone()
    h[9, 3] = float("nan")
    abi.pg_lmhead_ce_fwd(h, d["embed"], y, None, 30.0, nats, None)
    n = nats.cpu().numpy()
    assert np.isnan(n[[5, 6, 9]]).all() and np.isfinite(np.delete(n, [5, 6, 9])).all()
    assert math.isnan(gpu_bpb(nats, dict(d, target=y), V)[3])


def test_zero_rows_and_zero_weights():
    inp = synth.make_inputs("fwd_v8192", 4, T=500)
    d = abi.to_device(inp)
    nats = torch.zeros(0, device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"][:0], d["embed"], d["target"][:0], None, 30.0, nats, None)
    # zero embedding: ln V exactly (up to float32), BPB = log2(V) N / bytes
    nats = torch.empty(500, device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], torch.zeros_like(d["embed"]), d["target"], None, 30.0, nats, None)
    assert np.allclose(nats.cpu().numpy(), math.log(8192), atol=1e-5)
    out = gpu_bpb(nats, d, 8192)
    exp = math.log2(8192) * 500 / inp["byte_len"][inp["target"]].sum()
    assert abs(out[3] - exp) <= 1e-5 * exp


@pytest.mark.parametrize("T", [1, 255, 256, 257, 262144, 262145, 1000003])
def test_bpb_reduction_row_counts(T):
    """The reduction alone over row counts around its workgroup sizes (256 rows per workgroup up
    to 1024 workgroups, then several rows per thread), with a mask, a few targets outside the
    vocabulary and a byte sidecar, against the oracle's ratio of sums."""
    V = 8192
    rng = np.random.default_rng([7, T])
    nats = rng.uniform(0.0, 12.0, size=T).astype(np.float32)
    y = rng.integers(-2, V + 2, size=T).astype(np.int32)
    blen = rng.integers(0, 17, size=V).astype(np.int32)
    mask = (rng.random(T) < 0.7).astype(np.uint8)
    bpp = rng.integers(0, 9, size=T).astype(np.int32)
    print(f"[case] bpb T={T}", flush=True)
    d = {"target": torch.from_numpy(y).cuda(), "byte_len": torch.from_numpy(blen).cuda()}
    nats_t = torch.from_numpy(nats).cuda()
    for m, side in ((None, None), (mask, None), (mask, bpp)):
        m_t = None if m is None else torch.from_numpy(m).cuda()
        s_t = None if side is None else torch.from_numpy(side).cuda()
        out = gpu_bpb(nats_t, d, V, m_t, s_t)
        sn, sb, n, b = ora.bpb(nats.astype(np.float64), y, blen, m, side, V=V)
        assert out[1] == sb and out[2] == n
        assert out[0] == pytest.approx(sn, rel=1e-12)
        assert out[3] == pytest.approx(b, rel=1e-12)


def test_bpb_accumulated_over_calls():
    """pg_bpb_accumulate over consecutive chunks of 1,000,003 rows (chunk sizes around the
    reduction's workgroup sizes, one without scored rows), with a mask, targets outside the
    vocabulary and a byte sidecar: the running sums after the last call are the oracle's sums over
    all rows (integers exactly), and out[3] is their ratio after every call."""
    V, T = 8192, 1000003
    rng = np.random.default_rng(17)
    nats = rng.uniform(0.0, 12.0, size=T).astype(np.float32)
    y = rng.integers(-2, V + 2, size=T).astype(np.int32)
    blen = rng.integers(0, 17, size=V).astype(np.int32)
    mask = (rng.random(T) < 0.7).astype(np.uint8)
    bpp = rng.integers(0, 9, size=T).astype(np.int32)
    # chunk starts 16-byte aligned for every array (the entry points require it); a 262,144-row
    # chunk is 1024 workgroups of 256 rows, the last one takes several rows per thread
    cuts = [0, 16, 256, 272, 608, 608 + 262144, 608 + 262144 + 16, T]
    mask[608:608 + 262144] = 0                             # a chunk with no scored row
    print("[case] bpb accumulated over calls", flush=True)
    t_y, t_n = torch.from_numpy(y).cuda(), torch.from_numpy(nats).cuda()
    t_m, t_s, t_b = torch.from_numpy(mask).cuda(), torch.from_numpy(bpp).cuda(), torch.from_numpy(blen).cuda()
    for side in (None, t_s):
        out = torch.zeros(4, dtype=torch.float64, device="cuda")
        for a, b in zip(cuts[:-1], cuts[1:]):
            abi.pg_bpb_accumulate(t_n[a:b], t_y[a:b], t_m[a:b], t_b, None if side is None else side[a:b], V, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            sn, sb, n, bb = ora.bpb(nats[:b].astype(np.float64), y[:b], blen, mask[:b],
                                    None if side is None else bpp[:b], V=V)
            assert got[1] == sb and got[2] == n
            assert got[0] == pytest.approx(sn, rel=1e-12)
            if sb:
                assert got[3] == pytest.approx(bb, rel=1e-12)


def test_bitwise_reproducible():
    inp = synth.make_inputs("fwd_v1024", 0)
    d = abi.to_device(inp)
    res = []
    for _ in range(2):
        nats = torch.empty(inp["T"], device="cuda")
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, 30.0, nats, None)
        res.append((nats.cpu().numpy().tobytes(), gpu_bpb(nats, d, inp["V"]).tobytes()))
    assert res[0] == res[1]


# ---------------------------------------------------------------- asymmetric softcap
@pytest.mark.parametrize("caps", [(30.0, 10.0), (10.0, 30.0), (30.0, 0.0), (0.0, 20.0), (8.0, 40.0)])
def test_asymmetric_caps(caps):
    """Separate caps for z >= 0 and z < 0 (fixed-shift path when both sides are capped at <= 40,
    running maximum otherwise), logits spread over both caps' curvature."""
    w = workload("fwd_v8192", T=700, V=1500, stream=95, hidden_scale=40.0)
    inp = synth.make_inputs(w, 3)
    run(inp, softcap=caps)
    H, E = host_inputs(inp)
    z = H @ E.T
    assert z.max() > 30.0 and z.min() < -30.0


def test_asymmetric_equal_caps_are_the_symmetric_path():
    inp = synth.make_inputs(workload("fwd_v8192", T=1000, V=2048, stream=96), 0)
    d = abi.to_device(inp)
    a = torch.empty(inp["T"], device="cuda")
    b = torch.empty(inp["T"], device="cuda")
    abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, 30.0, a, None)
    abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], None, 30.0, 30.0, b, None)
    assert torch.equal(a, b)


def test_asymmetric_generic_widths():
    """f32 inputs and a width without an MFMA kernel take the vector path."""
    run(synth.make_inputs(workload("stress", dtype="f32", D=40, stream=97), 0), softcap=(30.0, 10.0))
    run(synth.make_inputs(workload("stress", D=48, stream=98), 0), softcap=(12.0, 30.0))


def test_asymmetric_main_full_size_sampled():
    """The main workload (T = 65536, D = 512, V = 8192) with caps (30, 20): sampled rows and the
    whole bits per byte against the oracle."""
    inp = synth.make_inputs("fwd_v8192", 0)
    caps = (30.0, 20.0)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([rng.choice(65536, 256, replace=False), [0, 65535]]))
    nats, _ = run(inp, softcap=caps, sample_rows=rows)
    H, E = host_inputs(inp)
    onats, _ = oracle_forward_chunked(H, E, inp["target"], caps)
    assert np.max(np.abs(nats - onats)) <= NATS_ATOL
    b_gpu = ora.bpb(nats, inp["target"], inp["byte_len"])[3]
    b_ora = ora.bpb(onats, inp["target"], inp["byte_len"])[3]
    assert abs(b_gpu - b_ora) <= BPB_RTOL * b_ora
