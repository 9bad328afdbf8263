"""The fp64 oracle under the host sanitizers: AddressSanitizer with
UndefinedBehaviorSanitizer, and ThreadSanitizer for its threaded forward
pass.  A C driver (tests/oracle_sanitize_driver.c) calls oracle_gdn_forward
on exact-size heap buffers; any report fails the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                                   ["-fsanitize=thread"]], ids=["asan-ubsan", "tsan"])
def test_oracle_runs_clean_under_sanitizers(tmp_path, flags):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "drv"
    build = subprocess.run([cc, "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", *flags,
                            os.path.join(HERE, "oracle_sanitize_driver.c"),
                            os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", str(exe), "-lm", "-lpthread"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "Sanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.stdout.count("rc 0") == 7
