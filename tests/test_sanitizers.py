"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no
GPU): the oracle's whole pin suite against a sanitized build of the oracle;
the host ABI tests against a sanitized host-only build of the library (the
kernel launcher stubbed); and a fuzz of the checkpoint-stream loader.  Each
runs in a child interpreter with the sanitizer runtimes preloaded, so that a
memory error or undefined behaviour ends it with a failure."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "sanitize"))
import build_sanitized as S  # noqa: E402

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc/g++")

ORACLE_TESTS = ["tests/test_oracle_encodings.py", "tests/test_oracle_quant.py",
                "tests/test_oracle_adam.py", "tests/test_oracle_static.py",
                "tests/test_oracle_amsgrad.py"]


def _run(cmd, env, timeout=900):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    return r.stdout


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitized"))


def test_oracle_pins_under_sanitizers(san_dir):
    env = S.env_with_sanitizers()
    env["ORACLE_LIBRARY"] = S.build_oracle(san_dir)
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
                "not gpu", *ORACLE_TESTS], env)
    assert " passed" in out


def _with_library(lib, code):
    return ("import sys; sys.path[:0] = [%r, %r]; "
            "import memory_efficient_adam_amd._binding as B; B._LIB_PATH = %r; " % (ROOT, HERE, lib)
            + code)


def test_host_abi_under_sanitizers(san_dir):
    lib = S.build_host_runtime(san_dir)
    code = _with_library(lib, "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', "
                              "'no:cacheprovider', 'tests/test_abi_host.py']))")
    out = _run([sys.executable, "-c", code], S.env_with_sanitizers())
    assert " passed" in out


def test_checkpoint_loader_fuzz_under_sanitizers(san_dir):
    lib = S.build_host_runtime(san_dir)
    out = _run([sys.executable, os.path.join(HERE, "sanitize", "fuzz_load.py"), lib, "1234", "3000"],
               S.env_with_sanitizers())
    assert "0 unexpected results" in out
