"""The C ABI from plain C (no GPU): a C99 program compiled against
include/hbmcoll.h and linked against the library makes host-only calls, and
its view must match the Python binding's (same library, same plans)."""
import os
import shutil
import subprocess

import pytest

import allreduce_reduction_amd as hc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_plain_c_client(tmp_path):
    lib = hc.LIB_PATH
    exe = tmp_path / "abi_host"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
                    lib, "-Wl,-rpath," + os.path.dirname(lib), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=120).stdout.splitlines()
    facts = dict(line.split(" -> ") for line in out if " -> " in line)
    with hc.Comm(8, "ring") as c:
        info = c.plan_info("allreduce", 1 << 20, "fp32")
        assert out[0] == f"ring8 allreduce steps {info['nsteps']} hbm {info['hbm_bytes']} recv {info['max_recv_bytes']}"
        assert info["nsteps"] == 14
        si = c.step_info("reduce_scatter", 1000, "int32", 0)
        assert out[2] == f"ring8 reduce_scatter step0 items {si['nitems']} hbm {si['hbm_bytes']}"
        form = c.exec_choice("allreduce", 4096, "fp16")
        assert out[3] == f"ring8 allreduce 4096 fp16 form {hc.EXEC[form]}"
        assert out[4] == f"ring8 allreduce 4096 fp16 regs bytes {c.exec_bytes('allreduce', 4096, 'fp16', 'regs')}"
    with hc.Comm(5, "rhd") as c:
        info = c.plan_info("allreduce", 4096, "bf16")
        assert out[1] == f"rhd5 allreduce steps {info['nsteps']} hbm {info['hbm_bytes']}"
    assert facts["create P=0"] == "1" and facts["pipeline S*M != P"] == "1"
    assert facts["set_exec_mode 99"] == "1" and facts["allreduce null bufs"] == "1"
    assert out[-2] == "status 1 " + hc.load_library().hbmc_status_string(1).decode()
    assert out[-1] == "done"
