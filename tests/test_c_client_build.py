"""The C ABI from plain C: include/ep.h compiles as strict C99, and the C
client (tests/c_client/ep_c_client.c, built by build()) links against the
in-tree libep.so and the HIP runtime.  The GPU test runs it."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "ep_c_client")


def test_header_is_strict_c99():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-x", "c",
                    os.path.join(ROOT, "include", "ep.h")], check=True)


def test_client_source_compiles_as_c99():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), CLIENT + ".c"], check=True)


def test_client_links_the_in_tree_library():
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client/ep_c_client is missing: run __graft_entry__.build()")
    out = subprocess.run(["ldd", CLIENT], capture_output=True, text=True, check=True).stdout
    lib = [l for l in out.splitlines() if "libep.so" in l]
    assert lib and "not found" not in lib[0]
    assert os.path.realpath(lib[0].split("=>")[1].split("(")[0].strip()) == \
        os.path.realpath(os.path.join(ROOT, "combine_ep_route_amd", "libep.so"))
