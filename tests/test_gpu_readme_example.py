"""The README's Python example runs as written and agrees with the oracle."""
import os
import re

import numpy as np
import pytest
import torch

from gpu_cases import bits, orc, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_readme_example_matches_oracle():
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    torch.manual_seed(0)
    env = {}
    say("[gpu] README example")
    exec(compile(code, "README.md example", "exec"), env)
    torch.cuda.synchronize()
    q, out, bt, ctx, d = env["q"], env["out"], env["block_tables"], env["ctx"], env["d"]
    # host pools: the example's zero pools with the new tokens stored by the
    # oracle; the GPU pools must hold the same bits
    host_k = np.zeros(tuple(env["k_cache"].shape), np.uint16)
    host_v = np.zeros_like(host_k)
    orc().store(bits(env["k_new"]), bits(env["v_new"]), env["slots"].numpy(), host_k, host_v)
    assert np.array_equal(bits(env["k_cache"]), host_k) and np.array_equal(bits(env["v_cache"]), host_v)
    ref = orc().decode(bits(q), host_k, host_v, bt.numpy(), ctx.numpy(), d ** -0.5)
    got = out.float().cpu().numpy()
    err = np.abs(got - ref)
    say(f"    max |err| {err.max():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
