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


LLVM_BIN = "/opt/rocm/llvm/bin"
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not (os.path.exists(os.path.join(LLVM_BIN, "clang")) and os.path.exists(HIPCC)),
                    reason="needs the ROCm clang toolchain")
def test_c_program_under_host_sanitizers(tmp_path, libdir):
    """The host layer of the library (argument checks, layouts, error strings) built with
    AddressSanitizer and UndefinedBehaviorSanitizer on the host side only, linked with the
    other objects of the normal build, driven by the same C program."""
    from precision_moe_amd import build as pb
    objs = sorted(os.path.join(pb.BUILD, f) for f in os.listdir(pb.BUILD)
                  if f.endswith(".o") and f != "api.o") if os.path.isdir(pb.BUILD) else []
    if len(objs) != len(pb.SOURCES) - 1:
        pytest.fail("the library's objects are missing: build it first")
    api = tmp_path / "api_san.o"
    lib = tmp_path / "libpmoe_san.so"
    exe = tmp_path / "abi_smoke_san"
    rt = os.path.dirname(subprocess.run(
        [os.path.join(LLVM_BIN, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
        capture_output=True, text=True, check=True).stdout.strip())
    subprocess.run([HIPCC, *pb.FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(pb.CSRC, "api.hip"), "-o", str(api)],
                   check=True, capture_output=True)
    san = "-fsanitize=" + "address,undefined"
    subprocess.run([os.path.join(LLVM_BIN, "clang++"), "-shared", "-fPIC", san, "-shared-libsan",
                    "-o", str(lib), str(api), *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    subprocess.run([os.path.join(LLVM_BIN, "clang"), "-std=c99", san, "-shared-libsan", "-I", INC,
                    SRC, "-o", str(exe), "-L", str(tmp_path), "-lpmoe_san",
                    f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{rt}"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_smoke: ok" in r.stdout and "runtime error" not in r.stderr
