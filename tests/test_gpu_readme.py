"""The README's usage examples, run as written.

The first example steps one layer once from an empty cache; the second
continues it, with names the README leaves to the reader (layers, budgets, d
and the incoming rows) set up here.  Each example must run unchanged, and its
results must be what the example says.
"""
from __future__ import annotations

import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _python_blocks() -> list[str]:
    text = open(os.path.join(ROOT, "README.md")).read()
    return re.findall(r"```python\n(.*?)```", text, re.S)


def test_readme_has_two_python_examples():
    assert len(_python_blocks()) == 2


@pytest.mark.gpu
def test_readme_examples_run():
    first, second = _python_blocks()
    ns: dict = {}
    exec(compile(first, "README.md (first example)", "exec"), ns)
    torch.cuda.synchronize()
    assert ns["ctr"].n_kept == 1 and ns["ctr"].next_pos == 1
    assert tuple(ns["keys"].shape) == (8, 1, 128) and tuple(ns["values"].shape) == (8, 1, 128)
    assert torch.equal(ns["values"][:, 0], ns["v"])      # the appended row, stored as given
    assert bool((ns["ev"] == -1).all())                   # under budget: nothing evicted

    import kv_cache_eviction_step_amd as kve
    d, bh, budgets = 128, 256, [300, 200, 100]
    layers = [kve.Layer.empty(bh, b + 1, d, "cuda") for b in budgets]
    new_k = torch.randn(len(budgets), bh, d, device="cuda").half()
    new_v = torch.randn(len(budgets), bh, d, device="cuda").half()
    evicted = torch.empty(len(budgets), bh, dtype=torch.int32, device="cuda")
    ns.update({"layers": layers, "budgets": budgets, "d": d, "new_k": new_k, "new_v": new_v,
               "evicted": evicted})                # the second example continues the first
    exec(compile(second, "README.md (second example)", "exec"), ns)
    torch.cuda.synchronize()
    batch = ns["batch"]
    for l in range(len(budgets)):                         # two calls: two rows appended
        assert batch.ctrs[l].n_kept == 2
        keys, values = layers[l].get_kv(batch.ctrs[l].n_kept)
        assert torch.equal(values[:, 1], new_v[l])
