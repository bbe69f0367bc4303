"""Host sanitizers over the CPU test suite.

Builds the HIP library with its host code under -fsanitize=address,undefined
(chunk_level_activation_amd/build_lib.py --sanitize) and the oracle's sanitizer build
(oracle.build_sanitized), then runs pytest with BLOCKFFN_SANITIZE=1 (both loaders pick
the sanitizer builds) and the sanitizer runtime preloaded; any report aborts the run.

    python tests/sanitize.py [pytest arguments]     (default: tests -m "not gpu")
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def build():
    from chunk_level_activation_amd import build_lib
    import oracle
    build_lib.build(sanitize=True)
    oracle.build_sanitized()
    return build_lib.sanitizer_env()


def run(pytest_args):
    env = dict(os.environ, **build())
    cmd = [sys.executable, "-m", "pytest", *pytest_args]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(run(sys.argv[1:] or ["tests", "-m", "not gpu", "-q"]))
