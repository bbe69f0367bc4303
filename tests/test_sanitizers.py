"""The host-side boundary checks and the oracle under the address and undefined-
behaviour sanitizers: the ABI tests (every validation path of every entry point, with
no GPU) and the oracle's pins run in a child process against the sanitizer builds
(tests/sanitize.py); any sanitizer report fails it."""
import os
import subprocess
import sys

import sanitize

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_oracle_pins_under_sanitizers():
    env = dict(os.environ, **sanitize.build())
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_loss_pins.py",
           "tests/test_oracle_backward_pins.py"]
    out = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (out.stdout + out.stderr)[-3000:]
    assert out.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
