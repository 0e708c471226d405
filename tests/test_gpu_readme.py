"""The README's usage example runs as written on the GPU (its Python block is
executed unchanged), and its two steps leave finite state and a 16-bit copy
that rounds the master weights."""
import os
import re

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    torch.cuda.synchronize()
    sh, p16 = ns["sh"], ns["p16"]
    assert ns["updated"] is True and ns["coef"] == 1.0  # zero gradients: nothing to clip
    assert bool(torch.isfinite(sh.master).all()) and bool(torch.isfinite(sh.exp_avg_sq).all())
    # zero weights and zero gradients stay zero; the copy is exactly zero too
    assert int(torch.count_nonzero(sh.master)) == 0 and int(torch.count_nonzero(p16.view(torch.int16))) == 0
    del ns
    torch.cuda.empty_cache()
