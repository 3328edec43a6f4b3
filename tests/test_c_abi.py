"""The boundary from plain C: tests/c_abi/c_abi_check.c includes only
include/rar.h and the HIP runtime header, links librar.so, and checks host
calls (CPU) and integer-exact collectives on device memory it allocates
itself (GPU).  The program is built by __graft_entry__.build()."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "_build", "c_abi_check")


def _run(*args):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    return subprocess.run([EXE, *args], capture_output=True, text=True, timeout=120)


def test_c_program_host_calls():
    p = _run("--cpu")
    assert p.returncode == 0, p.stderr
    assert "c_abi_check OK" in p.stdout


@pytest.mark.gpu
def test_c_program_collectives_on_device():
    p = _run()
    assert p.returncode == 0, p.stderr
    assert "c_abi_check OK" in p.stdout


@pytest.mark.gpu
def test_c_program_with_debug_sync():
    """RAR_DEBUG_SYNC=1 synchronises after every launch; results are unchanged."""
    env = dict(os.environ, RAR_DEBUG_SYNC="1")
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    p = subprocess.run([EXE], capture_output=True, text=True, timeout=120, env=env)
    assert p.returncode == 0, p.stderr
    assert "c_abi_check OK" in p.stdout
