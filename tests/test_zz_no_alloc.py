"""The allocation-free forward, pg_lmhead_ce_fwd_noalloc, through the C ABI against the workspace
entry point pg_lmhead_ce_fwd on the same inputs: two calls in a row on one GPU, the second with a
smaller input (the static scratch keeps the first call's contents), unmasked and masked, split and
unsplit vocabularies. Both run the same kernels, so the outputs must be the same bits; sampled rows
are also checked against the oracle."""
import numpy as np
import pytest
import torch

from lm_head_cross_pg_amd import abi, synth
from oracle import oracle as ora
from tests.gpu_helpers import NATS_ATOL, ensure_lib, host_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _compare(inp, mask, sample):
    T, c = inp["T"], inp["softcap"]
    print(f"[case] noalloc {inp['workload']} T={T} D={inp['D']} V={inp['V']} masked={mask is not None}", flush=True)
    d = abi.to_device(inp)
    m = None if mask is None else torch.from_numpy(mask).cuda()
    out = []
    for call in (abi.pg_lmhead_ce_fwd, abi.pg_lmhead_ce_fwd_noalloc):
        nats = torch.full((T,), float("nan"), device="cuda")
        lse = torch.full((T,), float("nan"), device="cuda")
        call(d["hidden"], d["embed"], d["target"], m, c, nats, lse)
        out.append((nats, lse))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
    H, E = host_inputs(inp)
    rows = np.asarray(sample)
    if mask is not None:
        rows = rows[mask[rows] != 0]
    onats, olse = ora.forward(H[rows], E, inp["target"][rows], c)
    assert np.max(np.abs(out[1][0].cpu().numpy()[rows] - onats)) <= NATS_ATOL
    assert np.max(np.abs(out[1][1].cpu().numpy()[rows] - olse)) <= NATS_ATOL


def test_noalloc_two_calls_second_smaller():
    rng = np.random.default_rng(3)
    big = synth.make_inputs("fwd_v8192", 0)                                  # 65,536 rows, one split
    _compare(big, None, rng.choice(big["T"], 64, replace=False))
    small = synth.make_inputs("fwd_v8192", 1, T=3000)                        # vocabulary split, masked
    mask = (rng.random(3000) < 0.4).astype(np.uint8)
    _compare(small, mask, np.arange(0, 3000, 7))
    tiny = synth.make_inputs("fwd_v1024", 2, T=300)                          # smaller again, unmasked
    _compare(tiny, None, np.arange(300))


def test_noalloc_rejects_shapes_beyond_its_scratch():
    T, D, V = (1 << 20) + 1, 32, 64
    H = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
    E = torch.zeros((V, D), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(T, dtype=torch.int32, device="cuda")
    nats = torch.zeros(T, device="cuda")
    with pytest.raises(abi.PgError, match="PG_ERR_SCRATCH"):
        abi.pg_lmhead_ce_fwd_noalloc(H, E, y, None, 30.0, nats)
    # the largest row count it takes: every row of a zero head costs ln V
    abi.pg_lmhead_ce_fwd_noalloc(H[:-1], E, y[:-1], None, 30.0, nats[:-1])
    torch.cuda.synchronize()
    assert abs(float(nats[:-1].min()) - np.log(V)) < 1e-5 and abs(float(nats[:-1].max()) - np.log(V)) < 1e-5
