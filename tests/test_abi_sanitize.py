"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU needed).

api.hip's host code is rebuilt with both sanitizers (device code untouched)
and linked with the library's other objects and the driver
`abi_host_checks.c`.  The driver calls every entry point with valid, edge and
invalid arguments that fail validation before any HIP call (int32 extremes,
NaN and infinite scales, sizes whose products overflow 32 bits, NULL and
misaligned pointers, undersized workspaces, bad chunk lists), checks the
status codes, and the sanitizers stop the run on any finding."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "column_sparse_masked_amd")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["address", "undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


def test_validation_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from column_sparse_masked_amd import build as B
    objs = [os.path.join(B.BUILD_DIR, s.replace(".hip", ".o")) for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "api_san.o")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([HIPCC, *flags, *host_san, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o])
    drv_o = str(tmp_path / "checks.o")
    san = "-fsanitize=" + ",".join(SAN)
    _run([CLANG, "-O1", "-g", san, "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", drv_o])
    exe = str(tmp_path / "abi_host_checks")
    _run([CLANGXX, san, drv_o, api_o, *objs, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failures" in r.stdout, out[-4000:]
