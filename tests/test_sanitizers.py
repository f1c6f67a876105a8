"""The CPU oracle and the host side of the HIP library under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU (no GPU is touched).

* oracle: oracle.c linked into tests/sanitize/oracle_driver.c, which drives
  every oracle function on small inputs (leak checking on);
* library host code: the library's sources compiled host-only, linked into
  tests/sanitize/api_driver.cpp, which drives argument validation,
  workspace sizing and the no-op paths.  Host-only objects refer to the
  device code bundles by symbol; the driver launches no kernel, so those
  symbols are given zero-filled stand-ins generated from the objects'
  undefined-symbol list.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
# the same for hipcc, host side only
HOST_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[:3], r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc"] + FLAGS + ["-fopenmp", "-ffp-contract=off", os.path.join(SAN, "oracle_driver.c"),
                            os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    r = _run([exe], env=env)
    assert r.stdout.startswith("OK")


@pytest.mark.skipif(shutil.which("hipcc") is None or shutil.which("nm") is None, reason="needs hipcc and nm")
def test_library_host_code_under_asan_ubsan(tmp_path):
    objs = []
    for src in sorted(glob.glob(os.path.join(ROOT, "quantized_moe_amd", "csrc", "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        objs.append((src, obj))
    procs = [subprocess.Popen(["hipcc", "--cuda-host-only", "-c", "-std=c++17", "-I", os.path.join(ROOT, "include")]
                              + HOST_FLAGS + [src, "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.PIPE)
             for src, obj in objs]
    for p, (src, _) in zip(procs, objs):
        out, err = p.communicate()
        assert p.returncode == 0, (src, err.decode()[-3000:])
    undef = _run(["nm", "-u"] + [o for _, o in objs]).stdout.split()
    names = sorted({s for s in undef if s.startswith("__hip_fatbin_")})
    stub = tmp_path / "fatbin_stubs.cpp"
    stub.write_text("".join(f'extern "C" {{ char {n}[4096] __attribute__((aligned(4096))); }}\n' for n in names))
    exe = str(tmp_path / "api_driver")
    _run(["hipcc", "-std=c++17", "-I", os.path.join(ROOT, "include")] + HOST_FLAGS +
         ["-x", "c++", os.path.join(SAN, "api_driver.cpp"), str(stub), "-x", "none"] +
         [o for _, o in objs] + ["-L/opt/rocm/lib", "-lhipblaslt", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")  # (the HIP runtime keeps allocations to exit)
    r = _run([exe], env=env)
    assert r.stdout.strip().endswith("OK")
