"""The usage example of README.md runs as written and its output matches the
CPU oracle (so the documentation cannot drift from the library)."""
import os
import re

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs_and_matches_oracle():
    text = open(os.path.join(ROOT, "README.md")).read()
    block = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    env: dict = {}
    exec(compile(block, "README.md", "exec"), env)
    torch.cuda.synchronize()
    q = env["q_bf16"].cpu()
    kv = env["kv_bf16"].cpu()
    qs, ks = oracle.fp8_absmax_scale(q), oracle.fp8_absmax_scale(kv)
    q8, k8 = oracle.fp8_quantize(q, qs), oracle.fp8_quantize(kv, ks)
    qo = np.asarray(env["qo"], dtype=np.int32)
    kvp = np.asarray(env["kvp"], dtype=np.int32)
    ref, _ = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, workloads.SM_SCALE)
    got = env["out"].float().cpu().numpy()
    assert np.array_equal(env["q8"].cpu().numpy(), q8)
    assert np.all(np.abs(got - ref) <= 1e-2 + 2e-2 * np.abs(ref))
