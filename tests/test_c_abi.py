"""The C-ABI from plain C: include/pmoe.h compiles as C99 and C++17 with warnings
as errors, and a C program linked against the library runs its host-only entry
points and argument checks (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import precision_moe_amd as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
SRC = os.path.join(ROOT, "tests", "c", "abi_smoke.c")


@pytest.fixture(scope="module")
def libdir():
    if not os.path.exists(pm.LIB_PATH):
        pytest.fail(f"{pm.LIB_PATH} is missing: build it first")
    return os.path.dirname(os.path.abspath(pm.LIB_PATH))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_header_compiles(tmp_path, lang):
    cc = "gcc" if lang == "c99" else "g++"
    x = "c" if lang == "c99" else "c++"
    src = tmp_path / "h.c"
    src.write_text('#include "pmoe.h"\nint main(void) { return pmoe_version() < 0; }\n')
    subprocess.run([cc, f"-std={lang}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INC,
                    "-x", x, "-c", str(src), "-o", str(tmp_path / "h.o")], check=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_calls_the_library(tmp_path, libdir):
    exe = tmp_path / "abi_smoke"
    lib = os.path.basename(pm.LIB_PATH)
    assert lib.startswith("lib") and lib.endswith(".so")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", INC, SRC, "-o", str(exe),
                    "-L", libdir, f"-l{lib[3:-3]}", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_smoke: ok" in r.stdout
