"""The C ABI from a plain C program (tests/c/abi_example.c): no Python, no
torch, buffers from the HIP runtime.  The CPU tier checks that it compiles
against the public header; the GPU tier runs the binary that build() made."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_example.c")
EXE = os.path.join(ROOT, "tests", "c", "abi_example")


def test_c_example_compiles_against_the_header():
    r = subprocess.run(["gcc", "-fsyntax-only", "-std=c11", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I" + os.path.join(ROOT, "include"), SRC],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout


@pytest.mark.gpu
def test_plain_c_caller_moves_bytes_and_reads_state():
    if not os.path.exists(EXE):  # build() makes it; build it only if nothing did
        import __graft_entry__
        __graft_entry__.build_c_example()
    r = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=120)
    assert r.returncode == 0 and "abi_example: ok" in r.stdout, r.stdout
