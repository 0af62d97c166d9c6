"""The CPU oracle and the library's host-side paths under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The oracle (plain C) is built with gcc -fsanitize=address,undefined and
  driven through every export on small inputs (tests/sanitize/oracle_driver.c).
* The library's host logic (argument checks, size arithmetic, configuration
  choice, the fault-injection hook, the scratch-array path) is compiled with
  the sanitizers on the host side only (-Xarch_host) and linked with the
  kernel-table objects of the regular build; tests/sanitize/abi_driver.c
  calls every entry point with invalid arguments, extreme sizes and, under
  FS_FAULT_INJECT=launch, valid ones -- nothing is launched.
Any sanitizer report fails the run (halt on the first error).
"""
import os
import shutil
import subprocess

import pytest

from lm_head_exact_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_TUS = ["fs_api", "fs_fused", "fs_unfused", "fs_online", "fs_pack"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    return r


def _env(**kw):
    env = dict(os.environ)
    env.pop("FS_FAULT_INJECT", None)
    env.update(kw)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1",
                             OMP_NUM_THREADS="4"))
    assert "all exports ran clean" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm hipcc")
def test_library_host_paths_under_asan_and_ubsan(tmp_path):
    # the configuration tables' objects of the current library build (by the
    # build's own source list: stale objects of removed units are not linked)
    kernels = [os.path.join(ROOT, "_build", os.path.splitext(src)[0] + ".o")
               for src in lib_build.SOURCES if src.startswith("fs_configs_")]
    if not kernels or not all(os.path.exists(k) for k in kernels):
        pytest.skip("kernel-table objects missing: run the library build first")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-w", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-ffp-contract=off", f"-I{os.path.join(ROOT, 'include')}"]
    procs, objs = [], []
    for tu in HOST_TUS:
        obj = str(tmp_path / f"{tu}.o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, *flags, "-c", os.path.join(ROOT, "lm_head_exact_amd", "csrc", f"{tu}.hip"),
             "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for tu, p in zip(HOST_TUS, procs):
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, f"{tu}: {out}"
    lib = str(tmp_path / "libflashsample_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", *objs, *kernels, "-o", lib])
    exe = str(tmp_path / "abi_san")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "abi_driver.c"), "-o", exe,
          f"-L{tmp_path}", "-lflashsample_san", f"-Wl,-rpath,{tmp_path}"])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1"))
    assert "all host paths ran clean" in r.stdout
