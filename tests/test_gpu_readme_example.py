"""The usage example in README.md runs as written: two steps (gathered, then
read in place), each a real update whose 16-bit params are the
round-to-nearest-even of the new fp32 master."""
import os
import re

import pytest
import torch

import zero_sharded_mixed_grads_amd as z

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example() -> str:
    text = open(os.path.join(ROOT, "README.md")).read()
    part = text.split("## Using it from PyTorch", 1)[1]
    return re.search(r"```python\n(.*?)```", part, re.S).group(1)


def test_readme_example_runs(capsys):
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    st = z.read_adam_state(ns["state"])
    assert st.step == 2 and st.skip == 0
    master, p16 = ns["master"], ns["param_slice"]
    assert torch.equal(p16, master.half())
    start = ns["flat"][ns["begin"]:ns["end"]].float()
    assert (master != start).float().mean().item() > 0.99
    assert z.read_loss_scale(ns["scale"]).scale == 2.0 ** 16  # no overflow, no growth yet
