"""Free-running HIP path vs oracle (tests/free_running.py): a short run per
gate mode.  The comparison is reported rather than gated: once a near-tie
rounds differently the two histories differ, codes by more than one step and
column scales by many ulps in the odd column.  The bounds here are loose
sanity limits on what matters downstream: the readouts stay close and both
paths carry the same quantisation error against the dense recurrence."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
pytest.importorskip("torch")


@pytest.mark.parametrize("cfg,n_req", [(1, 4), (2, 2)])
def test_free_running_short(cfg, n_req):
    import free_running as F
    rows = F.run(cfg, n_req, 32)
    print(F.report(rows, cfg, n_req, "calibrated"))
    for r in rows:
        assert r["code_diff_share"] <= 1e-2
        assert r["o_gpu_vs_oracle"] <= 1e-2
        assert abs(r["o_gpu_vs_dense"] - r["o_oracle_vs_dense"]) <= 0.05 * r["o_oracle_vs_dense"] + 1e-6
        assert np.isfinite(r["o_gpu_vs_dense"])
