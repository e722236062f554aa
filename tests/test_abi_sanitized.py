"""The C ABI's host logic (argument checks, shape planners, workspace layout, status strings)
under AddressSanitizer and UBSan: the host-sanitized build of the library runs the whole of
test_abi.py in a child process with the sanitizer runtime preloaded.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_under_host_sanitizers(tmp_path):
    from draft_selection_position_amd import build

    lib = build.build_host_sanitized()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm  # the host code really is instrumented
    env = dict(os.environ)
    rt = build.sanitizer_runtime()
    env["LD_PRELOAD"] = rt + (" " + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={tmp_path / 'asan'}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:log_path={tmp_path / 'ubsan'}"
    env["DFS_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    reports = sorted(tmp_path.glob("*san*"))
    detail = "".join(f"\n--- {p.name}\n" + p.read_text()[:4000] for p in reports)
    assert r.returncode == 0 and not reports, r.stdout[-4000:] + r.stderr[-4000:] + detail
    assert " passed" in r.stdout and "skipped" not in r.stdout, r.stdout[-2000:]
