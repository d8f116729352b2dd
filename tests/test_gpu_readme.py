"""The README's Python usage example runs as written, and its two results are
what the example says: relu(a + b) * 0.5 exactly (one correctly rounded fp32
add, an exact max and an exact halving), and h = x + r, y = RMSNorm(h) * w
with h bit-exact and y within 2 bf16 ulps of a float64 evaluation on the GPU."""
import os
import re

import numpy as np
import pytest
import torch

from gpu_util import need_gpu
from tolerance import check_half

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example():
    need_gpu()
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, flags=re.S).group(1)
    env = {}
    exec(compile(code, "README.md", "exec"), env)  # noqa: S102 - the repository's own example
    torch.cuda.synchronize()
    a, b, out = env["a"], env["b"], env["out"]
    assert torch.equal(out, torch.relu(a + b) * 0.5)
    x, r, w, h, y = env["x"], env["r"], env["w"], env["h"], env["y"]
    assert torch.equal(h, (x.float() + r.float()).to(torch.bfloat16))
    hd = h.double()
    ref = (hd * torch.rsqrt((hd * hd).mean(1, keepdim=True) + 1e-6) * w.double()).to(torch.bfloat16)
    sel = torch.arange(0, x.shape[0], 97, device="cuda")
    got = y[sel].cpu().view(torch.int16).numpy().view(np.uint16)
    want = ref[sel].cpu().view(torch.int16).numpy().view(np.uint16)
    check_half(got, want, "bf16", max_ulp=2, what="README RMSNorm example")
    env["npa"].np_shutdown()
