"""The host side of the library (every argument check, the state and workspace
bookkeeping that runs before a kernel is enqueued) built with a sanitizer and driven by the
ABI tests in a subprocess: undefined behaviour (as traps) and invalid memory accesses (with
the address sanitizer's runtime preloaded) in those paths stop it."""
import os
import subprocess
import sys

import pytest

import weight_sequence_layers_amd.build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("kind", ["ubsan", "asan"])
def test_abi_checks_under_sanitizer(tmp_path, kind):
    if not all(os.path.exists(os.path.join(B.PKG, "_build", s.replace(".", "_") + ".o"))
               for s in B.SOURCES):
        pytest.skip("no kernel objects: run the build first")
    lib = B.build_host_sanitized(str(tmp_path / f"libttt_{kind}.so"), kind)
    env = dict(os.environ, LIBTTT_PATH=lib)
    if kind == "asan":
        rt = B.asan_runtime()
        if not os.path.exists(rt):
            pytest.skip("no address-sanitizer runtime")
        env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    assert " passed" in r.stdout
