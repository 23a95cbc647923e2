"""The C-ABI from C: tests/c_abi_client.c, a C99 program that includes include/mhc.h only,
is compiled with gcc (-std=c99 -pedantic, warnings as errors), linked against the in-tree
libmhc.so and run. It calls the entry points that answer on the host (version, status
strings, workspace and packed sizes, validation errors), so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "mhc_hyper_connection_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the C client")
def test_c_client_builds_links_and_runs(tmp_path):
    from mhc_hyper_connection_amd import _binding as B
    B.load()   # builds libmhc.so in the tree if it is not there yet
    lib = os.path.join(LIB_DIR, "libmhc.so")
    assert os.path.exists(lib)
    exe = str(tmp_path / "c_abi_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"),
           "-o", exe, lib, "-Wl,-rpath," + LIB_DIR]
    rocm_lib = "/opt/rocm/lib"
    if os.path.isdir(rocm_lib):
        cmd += ["-Wl,-rpath-link," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = ":".join(p for p in (LIB_DIR, rocm_lib, env.get("LD_LIBRARY_PATH", "")) if p)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
