"""The batch-1 streaming kernel's weight loader, replayed on the CPU.

Compiles tests/stream_plan_check.cpp against the loader header the kernel
uses (qd_stream_plan.h) and runs it: for every wave of every workgroup of
several shapes and grid sizes, each issued tile must be the wave's next
expected tile (so inside its matrix), land in the slot it is read from, be
issued before it is read, never overfill the ring, and no tile may be
issued past the end of the stream."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)


def test_stream_loader_replay(tmp_path):
    exe = str(tmp_path / "stream_plan_check")
    cmd = ["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(REPO, "include"),
           "-I", os.path.join(REPO, "paged_kv_gqa_qwen3_amd", "csrc"),
           "-I", "/opt/rocm/include",
           os.path.join(HERE, "stream_plan_check.cpp"), "-o", exe]
    try:
        subprocess.run(cmd, check=True, capture_output=True, text=True)
    except FileNotFoundError:
        pytest.skip("g++ not available")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
