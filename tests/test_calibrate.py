"""Offline calibration and lifetime-aware allocation.

CPU: the exact allocator against brute force, the pivot rule and the budget.
GPU: the statistics of the FP32-state trajectories against the dense float64
recurrence of the oracle side, and the measured distortion table against the
oracle's own pack / unpack of the same states.
"""
import itertools

import numpy as np
import pytest

from quantized_recurrent_state_packed_amd import calibrate as C


def _brute(life, dist, widths, avg, n_piv):
    n = life.size
    risk = life * dist[min(widths)]
    piv = sorted(range(n), key=lambda u: (-risk[u], u))[:n_piv]
    free = [u for u in range(n) if u not in piv]
    budget = avg * n - 16 * n_piv
    best, arg = np.inf, None
    for bb in itertools.product(widths, repeat=len(free)):
        if sum(bb) != budget:
            continue
        c = sum(life[u] * dist[b][u] for u, b in zip(free, bb))
        if c < best:
            best, arg = c, bb
    return best, set(piv)


@pytest.mark.parametrize("trial", range(12))
def test_allocation_is_the_exact_optimum(trial):
    """Brute force over every width assignment meeting the budget exactly."""
    g = np.random.default_rng(100 + trial)
    n_piv = trial % 3 == 0
    n = 8 if n_piv else 6          # room for a 16-bit pivot inside the budget
    widths = (2, 4, 6) if trial % 2 else (4, 6, 8)
    avg = 4 if trial % 2 else 6
    life = np.exp(g.normal(2, 1.5, n))
    base = np.exp(g.normal(0, 1, n))
    # measured tables need not be convex in the width: perturb a 4^-b law
    dist = {b: base * 4.0 ** (-b) * np.exp(g.normal(0, 0.3, n)) for b in widths}
    dist[16] = base * 4.0 ** -16
    bits = C.allocate(life, dist, widths, avg, int(n_piv))
    assert bits.sum() == avg * n
    best, piv = _brute(life, dist, widths, avg, int(n_piv))
    assert set(np.flatnonzero(bits == 16)) == piv
    cost = sum(life[u] * dist[int(b)][u] for u, b in enumerate(bits) if b != 16)
    assert cost <= best * (1 + 1e-12)


def test_allocation_follows_lifetime_when_distortion_is_equal():
    """Same distortion everywhere: the longer-lived unit never gets fewer bits,
    and the pivots are the longest-lived units."""
    n = 12
    life = np.linspace(1, 100, n)
    dist = {b: np.full(n, 4.0 ** -b) for b in (4, 6, 8, 16)}
    bits = C.allocate(life, dist, (4, 6, 8), 6, 2)
    assert set(np.flatnonzero(bits == 16)) == {n - 1, n - 2}
    ints = bits[bits != 16].astype(int)
    assert np.all(np.diff(ints) >= 0)
    assert bits.sum() == 6 * n


def test_unreachable_budget_is_rejected():
    dist = {b: np.ones(3) for b in (4, 6, 8, 16)}
    with pytest.raises(ValueError):
        C.allocate(np.ones(3), dist, (4, 6, 8), 9, 0)


# ------------------------------------------------------------------ GPU
def _calib_inputs(cfg, n_req, T):
    import torch
    from quantized_recurrent_state_packed_amd import workloads as W
    lay = W.make_layout(cfg)
    req = list(range(1000, 1000 + n_req))
    S0 = W.make_initial_state(cfg, req, lay)
    steps = [W.make_step_inputs(cfg, t, req, lay, q_law="impact") for t in range(T)]
    dev = [{k: torch.from_numpy(v).cuda() for k, v in s.items()} for s in steps]
    return lay, S0, steps, dev


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [1, 2])
def test_statistics_follow_the_dense_recurrence(cfg):
    """Row magnitudes of the GPU's FP32-state trajectories against the float64
    dense recurrence over the same inputs; impact weights and lifetimes from
    the inputs."""
    import time
    import torch
    from oracle import dense_ref
    lay, S0, steps, dev = _calib_inputs(cfg, 4, 64)
    t0 = time.perf_counter()
    st = C.collect_statistics(lay.H, lay.D, lay.gate_mode, torch.from_numpy(S0).cuda(), dev, snapshot_every=8)
    torch.cuda.synchronize()
    print(f"config {cfg}: statistics of 4 requests x 64 steps in {1e3 * (time.perf_counter() - t0):.1f} ms")
    S = np.swapaxes(S0.astype(np.float64), -1, -2)
    acc = np.zeros((lay.H, lay.D))
    q2 = np.zeros((lay.H, lay.D))
    for t, inp in enumerate(steps, start=1):
        S, _ = dense_ref.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"])
        q2 += (inp["q"].astype(np.float64) ** 2).sum(axis=0)
        if t % 8 == 0:
            acc += (S * S).mean(axis=2).sum(axis=0)   # S is value x key: mean over value columns
    m_ref = np.sqrt(acc / (8 * S0.shape[0])).reshape(-1)
    assert np.allclose(st.row_magnitude, m_ref, rtol=1e-4)
    w_ref = (q2 / q2.mean()).reshape(-1)
    assert np.allclose(st.row_impact, w_ref, rtol=1e-5)
    a = lay.fixed_gate.astype(np.float64)
    assert np.allclose(st.lifetime, -1.0 / np.log(a), rtol=1e-9)
    assert len(st.snapshots) == 8
    assert np.array_equal(st.scale_impact, st.row_impact)
    # scale impact with lifetimes capped at a 32-step horizon: per-step weight
    # times min(lifetime, 32), mean 1; the other statistics do not move
    st32 = C.collect_statistics(lay.H, lay.D, lay.gate_mode, torch.from_numpy(S0).cuda(), dev, snapshot_every=8,
                                horizon=32)
    assert np.array_equal(st32.row_impact, st.row_impact)
    assert np.array_equal(st32.row_magnitude, st.row_magnitude)
    tau = -1.0 / np.log(a)
    tau_rows = np.repeat(tau, lay.D) if lay.gate_mode == 0 else tau.reshape(-1)
    si_ref = w_ref * np.minimum(tau_rows, 32.0)
    assert np.allclose(st32.scale_impact, si_ref / si_ref.mean(), rtol=1e-5)
    ratio = (st32.scale_impact / st32.row_impact).reshape(lay.H, lay.D)
    if lay.gate_mode == 0:      # one factor per head: it cancels against the column scales
        assert np.allclose(ratio, ratio[:, :1], rtol=1e-5)
    else:                       # rows of one head differ in lifetime, so their factors differ
        assert np.ptp(ratio, axis=1).max() > 0.1 * ratio.mean()


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,horizon", [(1, None), (2, None), (2, 32)])
def test_distortion_table_matches_the_oracle_codec(cfg, horizon):
    """Impact-weighted distortion per unit and width, measured through the
    library, against the oracle's pack / unpack of the same sampled states
    (row scales from the scale impact, errors weighed by the per-step one)."""
    import torch
    from oracle import oracle as O
    lay, S0, steps, dev = _calib_inputs(cfg, 2, 32)
    st = C.collect_statistics(lay.H, lay.D, lay.gate_mode, torch.from_numpy(S0).cuda(), dev, snapshot_every=16,
                              horizon=horizon)
    widths = (4, 6, 8)
    dist = C.measure_distortion(lay.H, lay.D, lay.gate_mode, st, widths)
    n_units = C.units_of(lay.H, lay.D, lay.gate_mode)
    w = st.row_impact.astype(np.float64).reshape(lay.H, lay.D)
    for b in widths + (16,):
        ol = O.OracleLayout(lay.H, lay.D, lay.gate_mode, np.full(n_units, b, np.uint8), st.scale_impact,
                            st.row_magnitude)
        acc = np.zeros((lay.H, lay.D))
        n = 0
        for snap in st.snapshots:
            x = snap.cpu().numpy()
            slots = np.arange(x.shape[0], dtype=np.int32)
            pool, scales = ol.new_pool(x.shape[0])
            ol.pack(slots, x, pool, scales)
            rec = ol.unpack(slots, pool, scales)
            acc += ((rec.astype(np.float64) - x) ** 2).sum(axis=(0, 3))
            n += x.shape[0]
        per_row = acc / n * w
        ref = per_row.sum(axis=1) if lay.gate_mode == 0 else per_row.reshape(-1)
        # A rounding tie decided differently moves one code and, through the
        # column fit, that column's binary16 scale by one ulp (2^-11), which
        # shifts every reconstruction of the column by up to |q| 2^-11 grid
        # steps: visible in a 128-element key-row unit, averaged out in a head
        # or over all units.
        rel = np.abs(dist[b] - ref) / np.maximum(ref, 1e-300)
        agg = abs(dist[b].sum() - ref.sum()) / ref.sum()
        print(f"config {cfg} horizon {horizon} width {b}: per-unit max rel {rel.max():.2e}, "
              f"aggregate rel {agg:.2e}")
        assert rel.max() <= (2e-3 if lay.gate_mode == 0 else 3e-2), b
        assert agg <= 1e-3, b
    # wider codes never do worse on average
    assert dist[8].sum() < dist[6].sum() < dist[4].sum()


@pytest.mark.gpu
def test_calibrated_allocation_meets_the_budget():
    import time
    import torch
    lay, S0, steps, dev = _calib_inputs(4, 2, 64)
    t0 = time.perf_counter()
    cal = C.calibrate(lay.H, lay.D, lay.gate_mode, torch.from_numpy(S0).cuda(), dev, (2, 4, 6), 4, 1,
                      snapshot_every=16)
    print(f"long-4bit layout: calibration of 2 requests x 64 steps in {time.perf_counter() - t0:.2f} s")
    assert cal.unit_bits.sum() == 4 * lay.H
    assert (cal.unit_bits == 16).sum() == 1
    assert np.all(cal.stats.row_magnitude > 0)


@pytest.mark.gpu
def test_lifetime_capped_impact_lowers_kda_drift_on_the_gpu():
    """End to end through the library: statistics of calibration requests
    with a 64-step horizon, then 64 decode steps of other requests in the KDA
    layout (the workload's widths, calibrated magnitudes) with the row scales
    and column fit weighted by the lifetime-capped impact or by the per-step
    one.  The state error against the FP32-state trajectory of the same kernel
    (every row binary32) is much lower with the lifetime-capped impact, as in
    the oracle-side study."""
    import torch
    from quantized_recurrent_state_packed_amd import stepq as S
    from quantized_recurrent_state_packed_amd import workloads as W
    T, B = 64, 4
    lay, S0c, _, devc = _calib_inputs(2, 4, T)
    st = C.collect_statistics(lay.H, lay.D, lay.gate_mode, torch.from_numpy(S0c).cuda(), devc,
                              snapshot_every=8, horizon=T)
    req = list(range(B))
    S0 = torch.from_numpy(W.make_initial_state(2, req, lay)).cuda()
    steps = [{k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in W.make_step_inputs(2, t, req, lay, q_law="impact").items()}
             for t in range(T)]
    slots = torch.arange(B, dtype=torch.int32, device="cuda")

    def final_state(unit_bits, impact):
        L = S.Layout(lay.H, lay.D, lay.gate_mode, unit_bits, impact, S.ROW_SCALES_CALIBRATED, st.row_magnitude)
        pool, scales = L.alloc(B, device="cuda")
        S.stepq_pack(L.handle, B, slots, B, S0, pool, scales)
        o = torch.empty(B, lay.H, lay.D, device="cuda")
        for d in steps:
            S.stepq_decode_step(L.handle, B, slots, B, d["q"], d["k"], d["v"], d["beta"], d["gate"], pool, scales, o)
        out = torch.empty_like(S0)
        S.stepq_unpack(L.handle, B, slots, B, pool, scales, out)
        return out.double().cpu()

    ref = final_state(np.full_like(lay.unit_bits, 32), st.row_impact)
    err = {}
    for name, impact in (("lifetime-capped", st.scale_impact), ("per-step", st.row_impact)):
        x = final_state(lay.unit_bits, impact)
        err[name] = float(torch.linalg.vector_norm(x - ref) / torch.linalg.vector_norm(ref))
    print(f"KDA layout, 4 requests x {T} steps, state error against FP32 state: {err}")
    assert err["lifetime-capped"] < 0.75 * err["per-step"]


@pytest.mark.gpu
def test_command_line_writes_a_usable_layout(tmp_path):
    """The calibration command on the KDA workload: the saved widths meet the
    budget with the pivot count, and the saved layout builds in the library."""
    from quantized_recurrent_state_packed_amd import stepq as S
    out = tmp_path / "kda.npz"
    assert C.main(["--workload", "kimi-kda-b64", "--requests", "2", "--steps", "32", "--horizon", "64",
                   "--pivots", "41", "--out", str(out)]) == 0
    z = np.load(out)
    ub = z["unit_bits"]
    assert ub.size == int(z["H"]) * int(z["D"]) and ub.sum() == 6 * ub.size
    assert (ub == 16).sum() == 41 and set(np.unique(ub)) <= {4, 6, 8, 16}
    assert abs(float(z["row_impact"].mean()) - 1.0) < 1e-5 and np.all(z["row_magnitude"] > 0)
    L = S.Layout(int(z["H"]), int(z["D"]), int(z["gate_mode"]), ub, z["row_impact"], S.ROW_SCALES_CALIBRATED,
                 z["row_magnitude"])
    assert L.handle
