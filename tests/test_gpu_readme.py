"""The Python example in README.md, run as written on the GPU, with its prefill and decode outputs checked against
the float64 oracle (the cache read back after each call's store)."""
import os
import re

import numpy as np
import pytest
import torch

from harness import assert_close
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example() -> str:
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has no python example"
    return blocks[0]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.gpu
def test_readme_example_matches_the_oracle():
    src = _example()
    # the prefill half first, then the cache as the decode call finds it
    split = src.index("# one decode step")
    ns: dict = {}
    exec(compile(src[:split], "README.md example (prefill)", "exec"), ns)
    torch.cuda.synchronize()
    kc, vc, bt = _bits(ns["k_cache"]), _bits(ns["v_cache"]), ns["block_table"].cpu().numpy()
    meta = {k: t.cpu().numpy() for k, t in ns["meta"].items()}
    scale = ns["D"] ** -0.5
    ref = oracle.prefill_varlen(_bits(ns["q"]), kc, vc, meta["cu_seqlens_q"], meta["cu_seqlens_k"], bt, scale, "bf16")
    assert tuple(ns["out"].shape) == (144, ns["Hq"], ns["D"])
    assert_close(ns["out"], ref, what="README prefill")

    exec(compile(src[split:], "README.md example (decode)", "exec"), ns)
    torch.cuda.synchronize()
    kc, vc = _bits(ns["k_cache"]), _bits(ns["v_cache"])
    ctx = ns["num_cached"].cpu().numpy() + 1
    ref1 = oracle.decode(_bits(ns["q1"]), kc, vc, ctx, bt, scale, "bf16")
    assert tuple(ns["out1"].shape) == (2, ns["Hq"], ns["D"])
    assert_close(ns["out1"], ref1, what="README decode")
    # the decode call stored the new rows where the block table puts position num_cached[s]
    bs = ns["bs"]
    for s, pos in enumerate(ns["num_cached"].cpu().numpy()):
        slot = int(bt[s][pos // bs]) * bs + int(pos) % bs
        flat_k = kc.reshape(-1, ns["Hkv"], ns["D"])
        np.testing.assert_array_equal(flat_k[slot], _bits(ns["k1"][s]))
