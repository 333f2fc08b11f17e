"""Full-size step-locked parity: every tile of a workload at its stated batch,
over its whole step sequence, against the oracle.

The default suite step-locks every tile on slices of the workloads and samples
tiles at the full batches; these runs take minutes each (the oracle steps
every tile on the host, and the pool crosses to the host every step), so they
run only with STEPQ_FULL_PARITY=1 in the environment:

    STEPQ_FULL_PARITY=1 python -m pytest tests/test_gpu_full_parity.py -m gpu -s

The bounds are those of every step-locked test (tests/parity.py)."""
import os

import pytest

from test_gpu_parity import _locked

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("STEPQ_FULL_PARITY") != "1",
                                 reason="full-size runs take minutes; set STEPQ_FULL_PARITY=1")]


@pytest.mark.parametrize("mode", ["calibrated", "refit"])
@pytest.mark.parametrize("cfg,B,T", [(1, 32, 256), (2, 64, 512), (4, 16, 2048), (3, 64, 128)])
def test_full_size_step_locked(cfg, B, T, mode):
    """Configs 1, 2 and 4 at their stated batches and step counts; the serving
    workload (config 3) on its first 64 requests (3,072 tiles) for its 128
    steps."""
    print(f"config {cfg} {mode} B={B} T={T}, every tile", flush=True)
    st_pack, st = _locked(cfg, B, T, B, mode, seed=100 + cfg, progress=16)
    print(f"config {cfg} {mode} full size: pack {st_pack.as_dict()}")
    print(f"config {cfg} {mode} full size: steps {st.as_dict()}")
    st_pack.check()
    st.check()


@pytest.mark.parametrize("mode", ["calibrated", "refit"])
@pytest.mark.parametrize("first", [64, 128, 192, 256, 320, 384, 448])
def test_serving_workload_rest_step_locked(first, mode):
    """The serving workload's other 448 requests in slices of 64 (requests are
    independent, and each regenerates its own seeded state and inputs), so
    that with the first slice above every tile of the 512 requests is
    step-locked over the 128 steps."""
    print(f"config 3 {mode} requests {first}..{first + 63}, every tile", flush=True)
    st_pack, st = _locked(3, 64, 128, 64, mode, seed=103, progress=32, first=first)
    print(f"config 3 {mode} requests {first}..{first + 63}: steps {st.as_dict()}")
    st_pack.check()
    st.check()
