"""GPU: the README's Python usage example runs as printed, and its result
matches the float64 oracle (a history of zeros but the appended token)."""

import os
import re

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_usage_example(gpu):
    text = open(README, encoding="utf-8").read()
    code = re.search(r"Usage from Python.*?```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    q = ns["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    kn = ns["k_new"].view(torch.int16).cpu().numpy().view(np.uint16)
    vn = ns["v_new"].view(torch.int16).cpu().numpy().view(np.uint16)
    Hkv, D = ns["Hkv"], ns["D"]
    for b, n in enumerate(ns["ctx"]):
        k = np.zeros((Hkv, n, D))
        v = np.zeros((Hkv, n, D))
        k[:, n - 1] = oracle.widen_bf16(kn[b])
        v[:, n - 1] = oracle.widen_bf16(vn[b])
        eo, el = oracle.decode_one_pass(oracle.widen_bf16(q[b]), k, v, n, D ** -0.5, Hkv)
        assert_out_close(ns["out"][b].cpu().numpy(), eo, what=f"request {b} out")
        assert_lse_close(ns["lse"][b].cpu().numpy(), el, what=f"request {b} lse")
