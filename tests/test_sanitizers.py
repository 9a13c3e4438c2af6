"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code (CPU only).

- The fp64 oracle (oracle/ssm_oracle.c) is built with gcc and both sanitizers
  and run by tests/sanitize/oracle_driver.c over every entry point, with the
  optional arguments present and absent, lengths and resets.
- The C-ABI layer (selective_state_space_66_amd/csrc/ssm_api.hip: argument
  validation, kernel choice, size queries) is built with hipcc, the
  sanitizers applied to its host code only, and linked ahead of the built
  library; tests/sanitize/abi_driver.cpp then calls every entry point on
  arguments the library must refuse and the host-only queries on shapes up to
  the int64 limits.  None of those calls reaches a HIP call, so no GPU is
  needed.

Either run aborts on the first report (halt_on_error, no recovery), so a
non-zero exit status is a finding.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")

ENV = dict(os.environ,
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           ASAN_OPTIONS="halt_on_error=1:verify_asan_link_order=0")


def _run(exe, env):
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"{os.path.basename(exe)} failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


SAN_C = ["-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]


def test_sanitizers_catch_a_planted_overrun(tmp_path):
    """The toolchain's sanitizers are live here: a read one past a heap array
    and a signed overflow each abort their program."""
    for name, body in (("overrun", "double* p = malloc(4 * sizeof(double)); "
                                   "volatile double v = p[argc + 3]; (void)v; free(p);"),
                       ("overflow", "volatile long long v = 0x7fffffffffffffffLL; v = v + argc;")):
        src = tmp_path / f"{name}.c"
        src.write_text("#include <stdlib.h>\nint main(int argc, char** argv) { (void)argv; "
                       + body + " return 0; }\n")
        exe = str(tmp_path / name)
        subprocess.run(["gcc", *SAN_C, "-o", exe, str(src)], check=True)
        r = subprocess.run([exe], env=ENV, capture_output=True, text=True, timeout=60)
        assert r.returncode != 0, f"the {name} went unreported"


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", *SAN_C, "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-lm", "-pthread"], check=True)
    env = dict(ENV, ASAN_OPTIONS=ENV["ASAN_OPTIONS"] + ":detect_leaks=1")
    assert "done" in _run(exe, env)


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    from selective_state_space_66_amd import build
    hipcc = build.hipcc()
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    if not os.path.exists(build.LIB):
        build.build()
    libdir = os.path.dirname(build.LIB)
    exe = str(tmp_path / "abi_driver")
    host = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", flag]
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", *host,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(build.CSRC, "ssm_api.hip"), os.path.join(HERE, "abi_driver.cpp"),
           f"-L{libdir}", "-lssm66_hip", f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # the HIP runtime keeps allocations until exit: leak checking is for the oracle
    env = dict(ENV, ASAN_OPTIONS=ENV["ASAN_OPTIONS"] + ":detect_leaks=0")
    assert "done" in _run(exe, env)
