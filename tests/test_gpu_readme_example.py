"""The README's decode-step example runs as written, and its output is the
attention over each sequence's prompt rows plus its new row (plain fp32
attention in PyTorch on the gathered rows, GQA head h reading KV head
h // (Hq / Hkv))."""
import os
import re

import pytest
import torch

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_decode_step_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    m = re.search(r"<!-- example -->\s*```python\n(.*?)```", text, re.S)
    assert m, "README example block not found"
    env = {}
    torch.manual_seed(0)
    print("README example", flush=True)
    exec(compile(m.group(1), "README.md", "exec"), env)
    torch.cuda.synchronize()
    Hq, Hkv, d = env["Hq"], env["Hkv"], env["d"]
    k_rows, v_rows, k_new, v_new, q, out = (env[n] for n in ("k_rows", "v_rows", "k_new", "v_new", "q", "out"))
    spans = [(0, 40), (40, 340)]  # the two prompts' rows
    G = Hq // Hkv
    for s, (a, b) in enumerate(spans):
        k = torch.cat([k_rows[a:b], k_new[s:s + 1]]).float().view(-1, Hkv, d)
        v = torch.cat([v_rows[a:b], v_new[s:s + 1]]).float().view(-1, Hkv, d)
        for h in range(Hq):
            g = h // G
            w = torch.softmax((k[:, g] @ q[s, h].float()) / d ** 0.5, dim=0)
            ref = w @ v[:, g]
            assert torch.allclose(out[s, h], ref, atol=2e-3, rtol=2e-3), (s, h, (out[s, h] - ref).abs().max())
