"""The host control plane (block tables and work plan, block lifecycle,
persistent-pool files) under AddressSanitizer and UndefinedBehaviorSanitizer:
the library built with shared_paged_kv_amd.build --host-sanitized, loaded in a
child process (KVPOOL_LIB, sanitizer runtimes preloaded), runs the CPU tests of
those three parts, the file reader's mutation test included.  Any sanitizer
report fails the run (UBSan halts on its first finding)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(not (_runtime("libasan.so") and _runtime("libubsan.so")), reason="no sanitizer runtimes")
def test_control_plane_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from shared_paged_kv_amd import build
    lib = build.build_host_sanitized()
    pre = [_runtime("libasan.so"), _runtime("libubsan.so")]
    if os.environ.get("LD_PRELOAD"):
        pre.append(os.environ["LD_PRELOAD"])   # keep what is already preloaded, after the sanitizer runtime
    env = dict(os.environ, KVPOOL_LIB=lib, LD_PRELOAD=":".join(pre),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from shared_paged_kv_amd import _lib as K\n"
            "K.lib(); assert K.LIB_PATH == %r, K.LIB_PATH\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
            "    'tests/test_tables_cpu.py', 'tests/test_lifecycle_cpu.py', 'tests/test_persist_cpu.py']))\n"
            % (ROOT, lib))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
