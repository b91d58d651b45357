"""Runs the Python example of README.md on the GPU and checks its results:
every node is accepted along the deepest path, the new prefix lengths grow
by the accepted length plus one, and the tree's committed KV is what the
attention appended."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    print("[gpu] README example", flush=True)
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    assert env["err"].tolist() == [0, 0]
    # depth 3 (nodes 0 -> 1 -> 3 -> 5) is the deepest path of the example tree
    assert env["accept_len"].tolist() == [3, 3]
    assert env["path"][:, :4].tolist() == [[0, 1, 3, 5]] * 2
    assert env["prefix_len"].tolist() == [504, 704]
    assert torch.equal(env["bonus"], env["tgt_argmax"][:, 5])
