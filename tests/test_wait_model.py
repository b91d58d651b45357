"""The bf16 attention kernel's hand-counted s_waitcnt vmcnt values.

The kernel (tv_attn_bf16.hip) issues its tile copies into LDS and several
register loads from inline asm, so the compiler inserts no waits for them;
every count is instantiated from the issue-order model in
csrc/tv_attn_waits.h. tests/wait_model_check.cpp replays, on the host, the
operations one thread issues and the waits it executes for every
instantiation (paged or not, tree built in the kernel or given), tile count,
tree-tile count and pass, and checks that each
wait covers what it guards, exactly, and that the counter never overflows.
Compiled with the host compiler; no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tree_attention_verification_tv_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("waits") / "wait_model_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{CSRC}", "-o", exe,
                    os.path.join(HERE, "wait_model_check.cpp")], check=True)
    return exe


def test_every_wait_covers_exactly_what_it_guards(checker):
    r = subprocess.run([checker], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    ok, cases, waits = r.stdout.split()
    assert ok == "ok" and int(cases) == 1152 and int(waits) > 5000


def test_the_earlier_tree_tile_wait_is_caught(checker):
    # the tree-tile wait once counted as for the last tree tile at the top of
    # an iteration (two later tiles), while only one tile follows the second
    # tree tile when the tree spans two tiles: the fill could read a stage
    # still being copied
    r = subprocess.run([checker, "--legacy-tree"], capture_output=True, text=True)
    assert r.returncode == 1
    assert "wait tree tiles" in r.stdout and "leaves tile1 in flight" in r.stdout
    assert "n_masked=2" in r.stdout and "n_masked=1 " not in r.stdout
