"""The host side of libdf11.so under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is built again with every host
compilation sanitized (the codec, which parses caller headers and buffers,
and the argument checks and launch arithmetic of the device entry points),
and the host-library tests run against that build in a child process with
the sanitizer runtime preloaded.  Any report ends the child with an error."""

import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_library_under_asan_and_ubsan(tmp_path):
    from entropy_decoding_df11_amd import _build
    try:
        runtime = _build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = _build.build_sanitized(str(tmp_path / "libdf11_sanitized.so"))
    env = dict(os.environ, DF11_LIB_PATH=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # The profile check compares committed files with the sources: nothing of the library runs in it.
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(REPO, "tests", "test_host_library.py"),
                          "-k", "not committed_profiles"],
                         cwd=REPO, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert " passed" in res.stdout and "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
