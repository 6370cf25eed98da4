"""The header is plain C: a C99 client (tests/c_abi_client.c) compiles against include/ with
-Wall -Wextra -pedantic -Werror, links libdecode_attn.so and runs its host-side checks (planning
and argument validation; no device work)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from paged_gqa_kv_attn_amd import binding

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_client_builds_and_runs(tmp_path):
    lib = binding.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    exe = str(tmp_path / "c_abi_client")
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_client.c"),
           "-L", libdir, "-ldecode_attn", "-Wl,-rpath," + libdir, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(
        [libdir, "/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")])
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c client ok" in run.stdout
