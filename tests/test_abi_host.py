"""The C-ABI library on the host: it loads, exports every declared symbol, and validates arguments
before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from lm_head_cross_pg_amd import abi, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pg_lmhead.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        build.build()
    return abi.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_symbols() == sorted(abi.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert abi.abi_version() == 1
    for code in range(0, -10, -1):
        assert abi.status_str(code) and abi.status_str(code) != "unknown status"
    assert abi.status_str(-99) == "unknown status"


def test_workspace_sizes(lib):
    T, D, V = 65536, 512, 8192
    fwd = abi.workspace_bytes(abi.PG_OP_FWD, T, D, V)
    bwd = abi.workspace_bytes(abi.PG_OP_BWD, T, D, V)
    bpb = abi.workspace_bytes(abi.PG_OP_BPB, T, D, V)
    assert fwd >= 2 * T * 4 and fwd < 64 << 20
    assert bwd >= T * V * 2                       # bf16 dZ
    assert 0 < bpb <= 1 << 20
    assert abi.workspace_bytes(abi.PG_OP_FWD, -1, D, V) == 0
    assert abi.workspace_bytes(abi.PG_OP_FWD, T, 0, V) == 0
    assert abi.workspace_bytes(7, T, D, V) == 0
    assert abi.workspace_bytes(abi.PG_OP_FWD, 0, D, V) > 0


# fake, 16-byte aligned "device" addresses: validation never dereferences them
P = 0x10000
BIG = 1 << 40


def fwd(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, T=256, D=64, V=512, c=30.0,
             nats=P, lse=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["T"], a["D"],
                                a["V"], a["c"], a["nats"], a["lse"], a["ws"], a["wsb"], a["stream"])


def bwd(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, lse=P, T=256, D=64, V=512, c=30.0, g=1 / 256,
             dh=P, de=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_bwd(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["lse"], a["T"],
                                a["D"], a["V"], a["c"], a["g"], a["dh"], a["de"], a["ws"], a["wsb"], a["stream"])


def fwd_bwd(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, T=256, D=64, V=512, c=30.0, g=1 / 256,
             nats=P, lse=P, dh=P, de=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd_bwd(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["T"], a["D"],
                                    a["V"], a["c"], a["g"], a["nats"], a["lse"], a["dh"], a["de"], a["ws"],
                                    a["wsb"], a["stream"])


def fwd_asym(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, T=256, D=64, V=512, cp=30.0, cn=10.0,
             nats=P, lse=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd_asym(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["T"], a["D"],
                                     a["V"], a["cp"], a["cn"], a["nats"], a["lse"], a["ws"], a["wsb"], a["stream"])


def bwd_asym(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, lse=P, T=256, D=64, V=512, cp=30.0, cn=10.0,
             g=1 / 256, dh=P, de=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_bwd_asym(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["lse"],
                                     a["T"], a["D"], a["V"], a["cp"], a["cn"], a["g"], a["dh"], a["de"], a["ws"],
                                     a["wsb"], a["stream"])


def fwd_bwd_asym(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, T=256, D=64, V=512, cp=30.0, cn=10.0, g=1 / 256,
             nats=P, lse=P, dh=P, de=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd_bwd_asym(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["T"],
                                         a["D"], a["V"], a["cp"], a["cn"], a["g"], a["nats"], a["lse"], a["dh"],
                                         a["de"], a["ws"], a["wsb"], a["stream"])


def quant(lib, **kw):
    a = dict(embed=P, dtype=0, V=512, D=64, q=P, scale=P, stream=None)
    a.update(kw)
    return lib.pg_quantize_q8(a["embed"], a["dtype"], a["V"], a["D"], a["q"], a["scale"], a["stream"])


def fwd_q8(lib, **kw):
    a = dict(hidden=P, q=P, scale=P, target=P, mask=None, T=256, D=64, V=512, c=30.0, nats=P, lse=P, ws=P,
             wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd_q8(a["hidden"], a["q"], a["scale"], a["target"], a["mask"], a["T"], a["D"],
                                   a["V"], a["c"], a["nats"], a["lse"], a["ws"], a["wsb"], a["stream"])


def bpb(lib, **kw):
    a = dict(nats=P, target=P, mask=None, blen=P, bpp=None, T=256, V=512, out=P, ws=P, wsb=BIG, stream=None)
    a.update(kw)
    return lib.pg_bpb_reduce(a["nats"], a["target"], a["mask"], a["blen"], a["bpp"], a["T"], a["V"], a["out"],
                             a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("call", [fwd, bwd, fwd_bwd, fwd_asym, bwd_asym, fwd_bwd_asym, fwd_q8, bpb])
def test_validation_codes(lib, call):
    assert call(lib, T=-1) == -2
    assert call(lib, V=0) == -2
    assert call(lib, ws=None) == -1
    assert call(lib, ws=P + 8) == -6
    assert call(lib, wsb=16) == -5


def test_fused_training_validation(lib):
    assert fwd_bwd(lib, lse=None) == -1           # required here (the backward half needs it)
    assert fwd_bwd(lib, nats=None) == -1
    # dhidden is optional (no dH): the call gets past the pointer checks to the workspace check
    assert fwd_bwd(lib, dh=None, wsb=1) == -5
    assert fwd_bwd(lib, de=None) == -1
    assert fwd_bwd(lib, dtype=2) == -3
    assert fwd_bwd(lib, c=-1.0) == -4
    assert fwd_bwd(lib, g=float("nan")) == -4
    assert fwd_bwd(lib, dh=P + 4) == -6
    T, D, V = 65536, 512, 8192
    need = abi.workspace_bytes(abi.PG_OP_FWD_BWD, T, D, V)
    assert need >= abi.workspace_bytes(abi.PG_OP_FWD, T, D, V) + abi.workspace_bytes(abi.PG_OP_BWD, T, D, V)
    assert fwd_bwd(lib, T=T, D=D, V=V, wsb=need - 1) == -5


def test_forward_validation(lib):
    assert fwd(lib, hidden=None) == -1
    assert fwd(lib, embed=None) == -1
    assert fwd(lib, target=None) == -1
    assert fwd(lib, nats=None) == -1
    assert fwd(lib, D=0) == -2
    assert fwd(lib, D=1 << 21) == -2
    assert fwd(lib, dtype=2) == -3
    assert fwd(lib, c=-1.0) == -4
    assert fwd(lib, c=float("nan")) == -4
    assert fwd(lib, c=float("inf")) == -4
    assert fwd(lib, hidden=P + 2) == -6
    assert fwd(lib, mask=P + 1) == -6
    assert fwd(lib, lse=P + 4) == -6


def test_backward_validation(lib):
    assert bwd(lib, lse=None) == -1
    assert bwd(lib, dh=None, wsb=1) == -5      # dhidden is optional (no dH)
    assert bwd(lib, de=None) == -1
    assert bwd(lib, g=float("nan")) == -4
    assert bwd(lib, dtype=5) == -3
    assert bwd(lib, de=P + 12) == -6


@pytest.mark.parametrize("call", [fwd_asym, bwd_asym, fwd_bwd_asym])
def test_asymmetric_cap_validation(lib, call):
    assert call(lib, cp=-1.0) == -4
    assert call(lib, cn=-0.5) == -4
    assert call(lib, cn=float("nan")) == -4
    assert call(lib, cp=float("inf")) == -4
    assert call(lib, hidden=None) == -1
    assert call(lib, dtype=3) == -3


def test_fused_training_asymmetric_validation(lib):
    assert fwd_bwd_asym(lib, lse=None) == -1
    assert fwd_bwd_asym(lib, de=None) == -1
    assert fwd_bwd_asym(lib, g=float("inf")) == -4
    assert fwd_bwd_asym(lib, dh=P + 4) == -6
    need = abi.workspace_bytes(abi.PG_OP_FWD_BWD, 256, 64, 512)
    assert fwd_bwd_asym(lib, wsb=need - 1) == -5


def test_quantised_head_validation(lib):
    assert quant(lib, D=60) == -2                 # D must be a multiple of 8
    assert quant(lib, V=0) == -2
    assert quant(lib, embed=None) == -1
    assert quant(lib, q=None) == -1
    assert quant(lib, scale=None) == -1
    assert quant(lib, dtype=4) == -3
    assert quant(lib, q=P + 4) == -6
    assert fwd_q8(lib, D=36) == -2
    assert fwd_q8(lib, scale=None) == -1
    assert fwd_q8(lib, c=-3.0) == -4
    assert fwd_q8(lib, q=P + 8) == -6
    need = abi.workspace_bytes(abi.PG_OP_FWD_Q8, 256, 64, 512)
    assert need >= abi.workspace_bytes(abi.PG_OP_FWD, 256, 64, 512) + 512 * 64 * 2
    assert fwd_q8(lib, wsb=need - 1) == -5
    assert abi.workspace_bytes(abi.PG_OP_FWD_Q8, 256, 60, 512) == 0


def test_bpb_validation(lib):
    assert bpb(lib, nats=None) == -1
    assert bpb(lib, blen=None) == -1
    assert bpb(lib, out=None) == -1
    assert bpb(lib, out=P + 8) == -6


def test_valid_arguments_reach_the_device_check(lib):
    """With every argument valid, the only thing left to fail on a host without a gfx950 GPU is
    the device check; nothing is enqueued."""
    if os.environ.get("HIP_VISIBLE_DEVICES") is None and _has_gpu():
        pytest.skip("a GPU is present; the device check would pass")
    assert fwd(lib) == -7
    assert bwd(lib) == -7
    assert fwd_asym(lib) == -7
    assert bwd_asym(lib) == -7
    assert fwd_bwd_asym(lib) == -7
    assert quant(lib) == -7
    assert fwd_q8(lib) == -7
    assert bpb(lib) == -7


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_row_and_grid_limits(lib):
    """Rows up to 2^31 - 256 (the MFMA grids of one 512-thread workgroup per 256 rows stay within a
    launch's 2^32 - 1 work items); the backward also needs its dH product's grid to fit, which
    bounds T D. Both are rejected on the host, before anything is enqueued."""
    top = (1 << 31) - 256
    assert fwd(lib, T=top + 1) == -2
    assert bpb(lib, T=top + 1) == -2
    if not _has_gpu():
        assert fwd(lib, T=top) == -7               # valid: only the device check is left
        assert bwd(lib, T=1 << 30, D=32, wsb=1 << 50) == -7
    assert bwd(lib, T=1 << 30, D=512) == -2
    assert fwd_bwd(lib, T=1 << 30, D=512) == -2
    assert abi.workspace_bytes(abi.PG_OP_BWD, 1 << 30, 512, 8192) == 0
    assert abi.workspace_bytes(abi.PG_OP_FWD, top, 512, 8192) > 0


# ------------------------------------------------ the Python binding checks its tensors first
def _cpu(T=8, D=32, V=16):
    import torch
    return dict(H=torch.zeros((T, D), dtype=torch.bfloat16), E=torch.zeros((V, D), dtype=torch.bfloat16),
                y=torch.zeros(T, dtype=torch.int32), nats=torch.zeros(T), lse=torch.zeros(T),
                dH=torch.zeros((T, D)), dE=torch.zeros((V, D)), m=torch.ones(T, dtype=torch.uint8))


@pytest.fixture
def no_library(monkeypatch):
    """Any call into the library (or its loader) fails the test: the checks must come first."""
    def fail(*a, **k):
        pytest.fail("the library was called")
    monkeypatch.setattr(abi, "load", fail)


def test_binding_rejects_mismatched_tensors(no_library):
    import torch
    t = _cpu()
    H, E, y, nats, lse, dH, dE, m = t["H"], t["E"], t["y"], t["nats"], t["lse"], t["dH"], t["dE"], t["m"]
    fwd_ = abi.pg_lmhead_ce_fwd
    cases = [
        (lambda: fwd_(H, E.float(), y, None, 30.0, nats), "embed has dtype"),
        (lambda: fwd_(H, E[:, :16].contiguous(), y, None, 30.0, nats), "embed has 16 columns"),
        (lambda: fwd_(H, E, y.long(), None, 30.0, nats), "target has dtype torch.int64"),
        (lambda: fwd_(H, E, y[:7], None, 30.0, nats), "target has 7 elements"),
        (lambda: fwd_(H, E, y, m.float(), 30.0, nats), "score_mask has dtype"),
        (lambda: fwd_(H, E, y, m[:3], 30.0, nats), "score_mask has 3 elements"),
        (lambda: fwd_(H, E, y, None, 30.0, nats.double()), "nats has dtype"),
        (lambda: fwd_(H, E, y, None, 30.0, nats, lse[:5]), "lse has 5 elements"),
        (lambda: fwd_(H.t(), E, y, None, 30.0, nats), "hidden must be contiguous"),
        (lambda: fwd_(H[0], E, y, None, 30.0, nats), "hidden must be 2-D"),
        (lambda: fwd_(H.double(), E, y, None, 30.0, nats), "hidden has dtype"),
        (lambda: fwd_(H, E, y, None, 30.0, nats), "is on cpu"),
        (lambda: abi.pg_lmhead_ce_bwd(H, E, y, None, lse, 30.0, 0.1, dH[:4], dE), "dhidden has 128 elements"),
        (lambda: abi.pg_lmhead_ce_bwd(H, E, y, None, lse, 30.0, 0.1, dH, dE[:, :8].contiguous()), "dembed has"),
        (lambda: abi.pg_lmhead_ce_bwd(H, E, y, None, None, 30.0, 0.1, dH, dE), "lse is required"),
        (lambda: abi.pg_lmhead_ce_fwd_bwd(H, E, y, None, 30.0, 0.1, nats, None, dH, dE), "lse is required"),
        (lambda: abi.pg_lmhead_ce_fwd_bwd_asym(H, E, y, None, 30.0, 20.0, 0.1, nats, lse, dH.double(), dE),
         "dhidden has dtype"),
        (lambda: abi.pg_lmhead_ce_bwd_asym(H, E, y, None, lse, 30.0, 20.0, 0.1, dH, dE), "is on cpu"),
        (lambda: abi.pg_lmhead_ce_fwd_asym(H, E, y.long(), None, 30.0, 20.0, nats), "target has dtype"),
        (lambda: abi.pg_quantize_q8(E, torch.zeros((16, 32), dtype=torch.int16), torch.zeros(16)),
         "embed_q8 has dtype"),
        (lambda: abi.pg_quantize_q8(E, torch.zeros((16, 32), dtype=torch.int8), torch.zeros(15)),
         "embed_scale has 15 elements"),
        (lambda: abi.pg_lmhead_ce_fwd_q8(H.float(), torch.zeros((16, 32), dtype=torch.int8), torch.zeros(16), y,
                                         None, 30.0, nats), "hidden has dtype"),
        (lambda: abi.pg_lmhead_ce_fwd_q8(H, torch.zeros((16, 24), dtype=torch.int8), torch.zeros(16), y,
                                         None, 30.0, nats), "embed_q8 has 24 columns"),
        (lambda: abi.pg_bpb_reduce(nats, y, None, torch.zeros(15, dtype=torch.int32), None, 16,
                                   torch.zeros(4, dtype=torch.float64)), "at least 16"),
        (lambda: abi.pg_bpb_reduce(nats, None, None, torch.zeros(16, dtype=torch.int32), None, 16,
                                   torch.zeros(4, dtype=torch.float64)), "target is required"),
        (lambda: abi.pg_bpb_reduce(nats, y, None, torch.zeros(16, dtype=torch.int32), None, 16,
                                   torch.zeros(4)), "out has dtype"),
        (lambda: abi.pg_bpb_reduce(nats, y, None, torch.zeros(16, dtype=torch.int32), y.long(), 16,
                                   torch.zeros(4, dtype=torch.float64)), "byte_per_pos has dtype"),
    ]
    for call, msg in cases:
        with pytest.raises(ValueError, match=msg):
            call()


def fwd_noalloc(lib, **kw):
    a = dict(hidden=P, embed=P, dtype=0, target=P, mask=None, T=256, D=64, V=512, c=30.0, nats=P, lse=P,
             stream=None)
    a.update(kw)
    return lib.pg_lmhead_ce_fwd_noalloc(a["hidden"], a["embed"], a["dtype"], a["target"], a["mask"], a["T"],
                                        a["D"], a["V"], a["c"], a["nats"], a["lse"], a["stream"])


def test_noalloc_forward_validation(lib):
    """The allocation-free forward validates like pg_lmhead_ce_fwd, and rejects a shape whose scratch
    would not fit its static buffer (T > 2^20 rows) with PG_ERR_SCRATCH before anything else runs."""
    assert fwd_noalloc(lib, T=-1) == -2
    assert fwd_noalloc(lib, nats=None) == -1
    assert fwd_noalloc(lib, dtype=2) == -3
    assert fwd_noalloc(lib, c=-1.0) == -4
    assert fwd_noalloc(lib, lse=P + 4) == -6
    assert fwd_noalloc(lib, T=(1 << 20) + 1) == -9
    assert abi.status_str(-9) != "unknown status"
    if not _has_gpu():
        assert fwd_noalloc(lib, T=1 << 20) == -7        # fits: only the device check is left
        assert fwd_noalloc(lib) == -7
