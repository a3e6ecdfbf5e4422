"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU-side code
(no GPU): the oracle (plain C, gcc) and the decode library's host-side entry
points and argument checks (csrc/api.hip compiled for the host with hipcc,
sanitizers on the host pass only, kernel launchers stubbed to abort).  Each
harness in tests/sanitize/ must exit 0 with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return r.returncode, r.stdout, err


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_asan")
    rc, out, err = _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                         os.path.join(HERE, "oracle_main.c"), os.path.join(ROOT, "oracle", "mla_oracle.c"),
                         "-o", exe, "-lm"])
    assert rc == 0, err
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    rc, out, err = _run([exe], env=env)
    assert rc == 0 and "0 failures" in out, out + err
    assert "runtime error" not in err and "AddressSanitizer" not in err, err


def test_host_abi_checks_under_asan_ubsan(tmp_path):
    if not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_asan")
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", f]
    rc, out, err = _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host,
                         os.path.join(HERE, "abi_main.cpp"),
                         os.path.join(ROOT, "mla_decode_attention_split_amd", "csrc", "api.hip"),
                         "-o", exe])
    assert rc == 0, err
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out, err = _run([exe], env=env)
    assert rc == 0 and "0 failures" in out, out + err
    assert "runtime error" not in err and "AddressSanitizer" not in err, err
