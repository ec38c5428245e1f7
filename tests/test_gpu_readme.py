"""The README's Python examples run as written (on small stand-in hidden states)."""
import os
import re

import pytest
import torch

from tests.gpu_helpers import ensure_lib

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _blocks():
    text = open(README, encoding="utf-8").read()
    usage = text[text.index("## Usage"):text.index("## Commands")]
    return re.findall(r"```python\n(.*?)```", usage, flags=re.S)


def test_readme_examples_run():
    ensure_lib()
    blocks = _blocks()
    assert len(blocks) == 2
    ns = {}
    print("[case] README example 1", flush=True)
    exec(compile(blocks[0], "README.md example 1", "exec"), ns)
    assert torch.isfinite(ns["out"]).all() and ns["out"][3].item() > 0
    assert torch.isfinite(ns["dhidden"]).all() and torch.isfinite(ns["dembed"]).all()

    def hidden_of(w0, nw):
        g = torch.Generator(device="cuda").manual_seed(1000 + w0)
        return torch.randn(nw * 2048, ns["D"], device="cuda", generator=g).to(torch.bfloat16)
    ns["hidden_of"] = hidden_of
    embed0 = ns["embed"].clone()
    print("[case] README example 2", flush=True)
    exec(compile(blocks[1], "README.md example 2", "exec"), ns)
    torch.cuda.synchronize()
    assert ns["n_scored"] == ns["tokens"].numel() - 1
    assert ns["bpb"] > 0
    assert abs(ns["bpb_int8"] - ns["bpb"]) < 1e-2 * ns["bpb"]   # the int8 head scores close to the bf16 one
    assert not torch.equal(ns["embed"], embed0)        # the test-time steps moved the embedding
