"""The boundary from plain C: tests/c/abi_host_calls.c includes include/beamattn.h under
gcc -std=c99 -pedantic -Werror, links libbeamattn.so and runs its host-only calls and
argument checks (no GPU work is launched)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "nope_gqa_attention_amd")


def test_plain_c_consumer_compiles_links_and_runs(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libbeamattn.so")):
        pytest.fail("libbeamattn.so is not built (python -m nope_gqa_attention_amd.build)")
    exe = str(tmp_path / "abi_host_calls")
    src = os.path.join(ROOT, "tests", "c", "abi_host_calls.c")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), src, "-L", LIBDIR, "-lbeamattn",
                    f"-Wl,-rpath,{LIBDIR}", "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
