"""The library's host code (argument checks, work planning, workspace sizing,
status and error strings, the checked-mode switch) under AddressSanitizer
and UndefinedBehaviorSanitizer: a build whose host half is instrumented (the
device code is the same) runs the host-only ABI tests (tests/test_abi.py) in
a child process with the sanitizer runtime preloaded; any report fails the
test. No GPU is needed: those tests never launch a kernel."""
import glob
import hashlib
import os
import subprocess
import sys

from query_aware_sparse_page_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources_sha():
    h = hashlib.sha256()
    for f in B.sources() + [os.path.join(ROOT, "include", "qsa.h")] + glob.glob(os.path.join(B.PKG, "csrc", "*.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _sanitized_lib():
    stamp = B.SAN_LIB + ".sha"
    sha = _sources_sha()
    if os.path.exists(B.SAN_LIB) and os.path.exists(stamp) and open(stamp).read() == sha:
        return B.SAN_LIB
    B.build(sanitize=True)
    with open(stamp, "w") as f:
        f.write(sha)
    return B.SAN_LIB


def test_abi_under_host_sanitizers(tmp_path):
    lib = _sanitized_lib()
    rt = B.sanitizer_runtime()
    logs = str(tmp_path / "san")
    env = dict(os.environ)
    env.update({
        "QSA_LIBRARY": lib,
        "LD_PRELOAD": rt,
        "LD_LIBRARY_PATH": os.path.dirname(rt) + ":" + env.get("LD_LIBRARY_PATH", ""),
        # leaks of the Python interpreter and the ROCm runtime are not the library's
        "ASAN_OPTIONS": f"detect_leaks=0:halt_on_error=1:log_path={logs}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={logs}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + reports[:6000])
    assert "passed" in r.stdout
