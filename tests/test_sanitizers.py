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


def test_layout_tables_under_the_sanitizers(tmp_path):
    """The host side's layout tables for the workload layouts and for random
    mixed ones (tests/sanitize/layout_tables.cpp recomputes the storage order,
    bit offsets, head words and the D = 128 group table from each layout's
    widths alone), built and run with the sanitizers and host-memory stand-ins
    for the HIP runtime calls of layout creation."""
    import numpy as np
    from quantized_recurrent_state_packed_amd import workloads as W
    exe = tmp_path / "layout_tables"
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT / 'include'}", str(ROOT / "tests" / "sanitize" / "layout_tables.cpp"),
                    str(ROOT / "tests" / "sanitize" / "launch_stub.cpp"), "-o", str(exe)], check=True)
    g = np.random.default_rng(23)
    cases = {f"config{c}": (W.make_layout(c).H, W.make_layout(c).D, W.make_layout(c).gate_mode,
                            W.make_layout(c).unit_bits) for c in (1, 2, 3, 4)}
    for n, D in enumerate((128, 128, 128, 64, 32)):
        H = int(g.integers(1, 5))
        p = g.dirichlet(np.ones(6))
        cases[f"random{n}-d{D}"] = (H, D, 1, g.choice([2, 4, 6, 8, 16, 32], size=H * D, p=p))
    # a head whose every block holds float rows, and one of 8-row runs of all widths
    cases["floats-and-runs"] = (2, 128, 1, np.r_[np.full(128, 16), np.repeat([2, 4, 6, 8, 16, 32, 8, 6], 16)])
    for name, (H, D, gate, ub) in cases.items():
        for cal in (0, 1):
            f = tmp_path / f"{name}-{cal}.txt"
            f.write_text(f"{H} {D} {gate} {cal}\n" + " ".join(str(int(x)) for x in np.asarray(ub).ravel()) + "\n")
            r = subprocess.run([str(exe), str(f)], capture_output=True, text=True)
            assert r.returncode == 0 and r.stdout.startswith("ok"), (name, cal, r.stdout, r.stderr[-2000:])
