"""Host code under the address and undefined-behaviour sanitizers.

The CPU oracle (oracle/stepq_oracle.cpp) and the host side of the library
(layout creation, argument checks and status strings of stepq_api.cpp, with
the kernel launchers replaced by host stand-ins from tests/sanitize/) are
built with g++ -fsanitize=address,undefined, and the oracle pins and the ABI
checks run against those builds in a child process with the sanitizer
runtimes preloaded; any report aborts the child.  A deliberate heap overflow
built the same way confirms that the instrumentation is live."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def _runtime(name: str) -> str:
    return subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    out = tmp_path_factory.mktemp("sanitized")
    from oracle import oracle as O
    ora = out / "libstepq_oracle_san.so"
    subprocess.run(["g++", *SAN, *O.COMPILE_FLAGS, str(O.SRC), "-o", str(ora)], check=True)
    host = out / "libstepq_host_san.so"
    subprocess.run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT / 'include'}", str(ROOT / "quantized_recurrent_state_packed_amd" / "csrc" / "stepq_api.cpp"),
                    str(ROOT / "tests" / "sanitize" / "launch_stub.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(host)], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               STEPQ_ORACLE_LIB=str(ora), STEPQ_LIBRARY=str(host))
    return out, env


def test_instrumentation_reports_a_heap_overflow(builds):
    out, env = builds
    src = out / "overflow.cpp"
    src.write_text("#include <cstdlib>\nint main(int c, char**) { int* p = (int*)std::malloc(4 * sizeof(int));"
                   " int v = p[c + 3]; std::free(p); return v == 12345; }\n")
    exe = out / "overflow"
    subprocess.run(["g++", *SAN, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env={k: v for k, v in env.items() if k != "LD_PRELOAD"})
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr), r.stderr


def test_oracle_pins_and_abi_checks_run_clean_under_the_sanitizers(builds):
    _, env = builds
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
