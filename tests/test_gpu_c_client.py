"""The C ABI driven from plain C on the device (tests/c/abi_device.c, built by
__graft_entry__.build()): hipMalloc'd rank buffers, AllReduce and the ring's
reduce-scatter on the null stream in several launch forms, compared in C with
exact integer references (wrapping int32 sum, int8 max)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_device")


def test_plain_c_client_on_the_device():
    if not os.path.exists(EXE):
        import __graft_entry__
        __graft_entry__.build_c_client()
    print("case: tests/c/abi_device", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=180)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert lines[-1] == "ok"
    assert sum(line.endswith("-> exact") for line in lines) == 6
