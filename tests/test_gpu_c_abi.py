"""The C ABI from a plain C program (tests/native/c_abi_example.c, built next to the library by
the build script): plan, reassign and forward on a layer whose keys and values are constant
within each cluster, where the result must be dense attention, with exact assignments, sizes
and counts. The program runs in its own process and reports through its exit status."""
import os
import subprocess

import pytest

from parity_util import say, torch_mod

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXAMPLE = os.path.join(ROOT, "sparse_attention_video_da_amd", "lib", "c_abi_example")


def test_c_program_through_the_abi():
    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXAMPLE), "build the library first (it builds the C example too)"
    say("[case] C program: cluster-constant layer through da_plan_create/da_reassign/da_forward")
    r = subprocess.run([EXAMPLE], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr
