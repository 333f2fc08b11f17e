"""The oracle-side drift / lifetime study runs end to end on a small slice.

Properties checked (none depends on tuning): a finer uniform grid drifts less
(INT8 below INT4 at every checkpoint of a short run), and the per-unit
statistics are well formed.
"""
import numpy as np

from oracle import drift_study as DS


def test_drift_study_small_slice():
    r = DS.run(1, ["stepq", "stepq-refit", "int4", "int8"], n_req=1, T=8)
    m = r["modes"]
    for p in r["checkpoints"]:
        assert m["int8"]["state_rel"][p] < m["int4"]["state_rel"][p]
        for mode in m:
            assert np.isfinite(m[mode]["state_rel"][p])
    assert np.all(m["int8"]["o_rel"] < m["int4"]["o_rel"])
    for mode in m:
        s = DS.lifetime_stats(r["layout"], m[mode]["unit_sq"])
        assert s["units"] == 48 and -1 <= s["spearman"] <= 1 and 0 <= s["top_quarter_share"] <= 1
    text = DS.drift_report(r, 1, 1)
    assert "Spearman" in text and "int8" in text


def test_calibrated_row_magnitudes_come_from_the_fp32_trajectory():
    """The study's own calibration is the RMS of the dense float64 trajectory's
    rows: positive, and ordered like the generator's outlier rows."""
    from quantized_recurrent_state_packed_amd import workloads as W
    lay = W.make_layout(2)
    m = DS.calibrate_row_magnitude(2, lay, 4).reshape(lay.H, lay.D)
    assert np.all(m > 0)
    for h in range(lay.H):
        rows = lay.outlier_rows[h]
        others = np.setdiff1d(np.arange(lay.D), rows)
        assert m[h, rows].min() > 5 * np.median(m[h, others])


def test_lifetime_impact_weights():
    """Row impact times lifetime capped at the horizon, mean 1: one factor per
    head under the per-head gate; under the KDA gate the factor follows each
    row's lifetime until the cap, and a horizon below every lifetime leaves
    the per-step weights unchanged."""
    from quantized_recurrent_state_packed_amd import workloads as W
    lay1 = W.make_layout(1)
    w = DS.lifetime_impact(lay1, 256)
    assert abs(w.mean() - 1) < 1e-6
    r = (w / lay1.row_impact).reshape(lay1.H, lay1.D)
    assert np.allclose(r, r[:, :1], rtol=1e-5)
    lay2 = W.make_layout(2)
    tau = np.asarray(lay2.lifetime, np.float64)
    assert tau.shape == (lay2.H * lay2.D,)
    w_inf = DS.lifetime_impact(lay2, 10 ** 12).astype(np.float64)
    r = w_inf / lay2.row_impact / tau
    assert np.allclose(r, r[0], rtol=1e-5)
    w_one = DS.lifetime_impact(lay2, tau.min()).astype(np.float64)
    base = lay2.row_impact / lay2.row_impact.mean()
    assert np.allclose(w_one, base, rtol=1e-5)
