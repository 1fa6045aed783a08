"""The README's usage example runs as written and produces outputs of the shapes and dtypes it states."""

import os
import re

import pytest
import torch

from tests.helpers import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_usage_example_runs():
    require_gpu()
    text = open(os.path.join(ROOT, "README.md")).read()
    block = re.search(r"## Use\n\n```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(block, "README.md (Use)", "exec"), ns)
    torch.cuda.synchronize()
    expect = {"y": ((8192, 18432), torch.bfloat16), "dx": ((8192, 7168), torch.bfloat16),
              "dw": ((18432, 7168), torch.float32), "ye": ((512, 2048), torch.bfloat16),
              "yp": ((8192, 18432), torch.bfloat16), "qpt": ((7168, 8192), torch.uint8),
              "spt": ((64, 7168), torch.float32)}
    for name, (shape, dtype) in expect.items():
        t = ns[name]
        assert tuple(t.shape) == shape and t.dtype == dtype, name
        if t.dtype != torch.uint8:
            assert bool(torch.isfinite(t.float()).all()), name
