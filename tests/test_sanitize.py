"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

- The C ABI's host side (argument checks, workspace planning, error paths of every entry
  point) is compiled with the sanitizers on the host pass only and driven by
  tests/sanitize/host_driver.cpp; the kernel launchers are replaced by stand-ins that report
  "no device", so no call reaches a kernel.
- The fp64 oracle is compiled with the sanitizers and run by tests/sanitize/oracle_driver.c;
  its checksums must equal those of a plain build (same arithmetic, any thread count).
- The key-major launch shape (which workgroup computes which head group, live item, column
  slice and row part; where the parts' sums go) is checked on the host by
  tests/sanitize/kv_shape_check.cpp.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_DIR = os.path.join(HERE, "sanitize")
CSRC = os.path.join(ROOT, "sparse_mla_flash_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# sanitizer flags for the host pass of a HIP compile (the device pass is left alone)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# sanitizer flags of the host-only link and of the gcc build of the oracle
LINK_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, cwd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout, r.stderr


def _checked(cmd, cwd):
    rc, out, err = _run(cmd, cwd)
    assert rc == 0, f"{' '.join(cmd)} failed:\n{out}\n{err}"


def _env(extra):
    env = dict(os.environ)
    env.update(extra)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    src = [os.path.join(SAN_DIR, "oracle_driver.c"), os.path.join(ROOT, "oracle", "sfag_oracle.c")]
    inc = ["-I", os.path.join(ROOT, "oracle")]
    plain = str(tmp_path / "oracle_plain")
    san = str(tmp_path / "oracle_san")
    _checked(["gcc", "-O2", "-std=c99", "-fopenmp", *inc, "-o", plain, *src, "-lm"], str(tmp_path))
    _checked(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fno-omit-frame-pointer", "-static-libasan",
              *LINK_SAN, *inc, "-o", san, *src, "-lm"], str(tmp_path))
    rc, ref, err = _run([plain], str(tmp_path), env=_env({"OMP_NUM_THREADS": "1"}))
    assert rc == 0, err
    # libgomp keeps its thread pool until exit: leak checks stay on for everything else
    rc, got, err = _run([san], str(tmp_path), env=_env({**ENV_SAN, "OMP_NUM_THREADS": "3"}))
    assert rc == 0 and "runtime error" not in err and "AddressSanitizer" not in err, f"{got}\n{err}"
    ref_lines, got_lines = ref.splitlines(), got.splitlines()
    assert len(ref_lines) == len(got_lines) and len(ref_lines) > 40
    for a, b in zip(ref_lines, got_lines):
        fa, fb = a.split(), b.split()
        assert fa[0] == fb[0]
        for x, y in zip(fa[1:], fb[1:]):
            if fa[0] == "==":
                continue
            x, y = float(x), float(y)
            assert abs(x - y) <= 1e-13 * max(1.0, abs(x)), (a, b)


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not available")
def test_host_library_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    hip_common = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *inc]
    objs = []
    for src in (os.path.join(CSRC, "sfag_api.cpp"), os.path.join(SAN_DIR, "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        _checked([HIPCC, *hip_common, *HOST_SAN, "-c", src, "-o", obj], str(tmp_path))
        objs.append(obj)
    drv = str(tmp_path / "host_driver.o")
    _checked([CLANGXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *LINK_SAN, *inc, "-c",
              os.path.join(SAN_DIR, "host_driver.cpp"), "-o", drv], str(tmp_path))
    exe = str(tmp_path / "host_san")
    _checked([CLANGXX, *LINK_SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
              "-Wl,-rpath,/opt/rocm/lib"], str(tmp_path))
    # the HIP runtime keeps allocations until exit: leaks are not checked in this process
    env = _env({**ENV_SAN, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
    rc, out, err = _run([exe], str(tmp_path), env=env, timeout=300)
    assert rc == 0 and "runtime error" not in err and "AddressSanitizer" not in err, f"{out}\n{err}"
    assert "ok: 0 failed expectations" in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="ROCm compilers not available")
def test_key_major_launch_shape(tmp_path):
    exe = str(tmp_path / "kv_shape")
    _checked([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", CSRC, *HOST_SAN,
              os.path.join(SAN_DIR, "kv_shape_check.cpp"), "-o", exe], str(tmp_path))
    rc, out, err = _run([exe], str(tmp_path), env=_env({**ENV_SAN, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"}))
    assert rc == 0 and out.startswith("ok"), f"{out}\n{err}"
