"""Offline calibration and lifetime-aware bit allocation for the packed state.

STEPQuant fixes its configuration once, offline, on calibration data, and
uses it for every request (ai-papers.net "STEPQuantの仕組み"; ai-trend.me
"방법"; ai-feeds.com key modules 1-3).  This module computes that configuration
on the GPU, through the library's own kernels:

  1. statistics of FP32-state trajectories of the calibration requests (every
     row stored as binary32, i.e. the unquantised decode step):
       - calibrated row magnitude m_i: RMS of key row i over requests, sampled
         steps and value columns;
       - row-impact weight w_i = E[q_i^2] (the readout o = M'^T q weighs row
         i's error by q_i; ai.info "Methodology in Plain English"), scaled to
         mean 1 (the rule is invariant to a common factor);
       - unit lifetime tau_u = -1 / E[ln a_u] from the mean log retention of
         the unit's gate (ai.info "Key Contributions" 2);
       - the impact the layout's row scales and column fit use: w_i itself,
         or, given a horizon T (the decode length the state must serve),
         w_i min(tau_i, T) scaled to mean 1.  An error written into a row
         persists for about the row's lifetime, so its cost to later readouts
         grows with it (ai-papers.net "誤差が効く時と場所": where and when errors
         matter).  Under the per-head gate the factor is constant within a tile
         and cancels against the column scales; under the per-key-channel gate
         it moves resolution toward long-lived rows;
  2. the impact-weighted distortion D_u(b) = E sum_{i in u} w_i ||M_i - M^_i||^2
     of every unit at every candidate width, measured by packing and unpacking
     sampled states with the library's quantiser (calibrated row scales, the
     scale impact above); the weight is the per-step w_i, since the allocation
     multiplies by the lifetime itself;
  3. the allocation: the n_pivots units of highest risk tau_u D_u(b_min) become
     FP16 pivots (ai.info "Key Contributions" 2: a few highest-risk units kept
     in FP16), and the others take the widths minimising
     sum_u tau_u D_u(b_u) under the exact average budget, pivots counted inside
     it (ai-papers.net "STEPQuantの仕組み": lifetime-weighted reconstruction
     error minimised under the average bit budget).

A unit is a head under the per-head gate and a key row under the per-key-channel
(KDA) gate.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PIVOT_BITS = 16


@dataclass
class Statistics:
    row_magnitude: np.ndarray          # float32 [H*D]
    row_impact: np.ndarray             # float32 [H*D], mean 1: per-step readout weight E[q_i^2]
    lifetime: np.ndarray               # float64 [units]
    scale_impact: np.ndarray           # float32 [H*D], mean 1: the layout's row impact
    snapshots: list = field(default_factory=list)   # device float32 [B, H, D, D] states
    steps: int = 0
    requests: int = 0


@dataclass
class Calibration:
    stats: Statistics
    widths: tuple
    distortion: dict                   # width -> float64 [units]
    unit_bits: np.ndarray              # uint8 [units]


def units_of(H: int, D: int, gate_mode: int) -> int:
    return H if gate_mode == 0 else H * D


def collect_statistics(H: int, D: int, gate_mode: int, S0, step_inputs, snapshot_every: int = 16,
                       max_snapshots: int = 8, horizon: int | None = None) -> Statistics:
    """FP32-state trajectories of the calibration requests on the GPU.

    S0: device float32 [B, H, D, D] initial states; step_inputs: iterable of
    dicts of device tensors q, k, v [B, H, D], beta [B, H], gate [B, H] or
    [B, H, D] (the decode step's inputs).  Row statistics are sampled after
    every snapshot_every-th step; the last max_snapshots sampled states are
    kept for the distortion measurement.  horizon: None, or the decode
    length (>= 1) that caps the lifetimes in the scale impact."""
    if horizon is not None and horizon < 1:
        raise ValueError("horizon must be at least 1 step")
    import torch
    from . import stepq as S
    B = S0.shape[0]
    dev = S0.device
    ub = np.full(H if gate_mode == 0 else H * D, 32, np.uint8)
    L = S.Layout(H, D, gate_mode, ub, np.ones(H * D, np.float32), S.ROW_SCALES_REFIT)   # binary32 rows: no scales
    pool, scales = L.alloc(B, device=dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    S.stepq_pack(L.handle, B, slots, B, S0.contiguous(), pool, scales)
    o = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    state = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    row_sq = torch.zeros(H, D, dtype=torch.float64, device=dev)
    q_sq = torch.zeros(H, D, dtype=torch.float64, device=dev)
    log_a = torch.zeros(H if gate_mode == 0 else H * D, dtype=torch.float64, device=dev)
    snaps = []
    n_samples = 0
    t = 0
    for t, d in enumerate(step_inputs, start=1):
        S.stepq_decode_step(L.handle, B, slots, B, d["q"], d["k"], d["v"], d["beta"], d["gate"], pool, scales, o)
        q_sq += (d["q"].double() ** 2).sum(dim=0)
        la = torch.log(d["gate"].double())
        log_a += la.sum(dim=0) if gate_mode == 0 else la.sum(dim=0).reshape(-1)
        if t % snapshot_every == 0:
            S.stepq_unpack(L.handle, B, slots, B, pool, scales, state)
            row_sq += (state.double() ** 2).mean(dim=3).sum(dim=0)
            n_samples += 1
            snaps.append(state.clone())
            if len(snaps) > max_snapshots:
                snaps.pop(0)
    if n_samples == 0 or t == 0:
        raise ValueError("calibration needs at least snapshot_every steps")
    m = torch.sqrt(row_sq / (n_samples * B)).cpu().numpy().reshape(-1)
    w = (q_sq / (t * B)).cpu().numpy().reshape(-1)
    w = w / w.mean()
    mean_log_a = (log_a / (t * B)).cpu().numpy()
    life = np.where(mean_log_a < 0, -1.0 / np.minimum(mean_log_a, -1e-300), np.inf)
    # a zero magnitude (a row no step ever wrote) gets the smallest positive one
    pos = m[m > 0]
    m = np.where(m > 0, m, pos.min() if pos.size else 1.0)
    if horizon is None:
        si = w
    else:
        life_rows = np.repeat(life, D) if gate_mode == 0 else life
        si = w * np.minimum(life_rows, float(horizon))
        si = si / si.mean()
    return Statistics(row_magnitude=m.astype(np.float32), row_impact=w.astype(np.float32), lifetime=life,
                      scale_impact=si.astype(np.float32), snapshots=snaps, steps=t, requests=B)


def measure_distortion(H: int, D: int, gate_mode: int, stats: Statistics, widths) -> dict:
    """Impact-weighted squared reconstruction error per unit at every width,
    averaged over the sampled states: pack with every unit at that width
    (calibrated row scales from the scale impact), unpack, compare, weigh
    each row's error by its per-step readout weight."""
    import torch
    from . import stepq as S
    out = {}
    n_units = units_of(H, D, gate_mode)
    w = torch.from_numpy(stats.row_impact.astype(np.float64).reshape(H, D))
    for b in sorted(set(int(x) for x in widths) | {PIVOT_BITS}):
        L = S.Layout(H, D, gate_mode, np.full(n_units, b, np.uint8), stats.scale_impact,
                     S.ROW_SCALES_CALIBRATED, stats.row_magnitude)
        acc = torch.zeros(H, D, dtype=torch.float64)
        n = 0
        for snap in stats.snapshots:
            B = snap.shape[0]
            dev = snap.device
            pool, scales = L.alloc(B, device=dev)
            slots = torch.arange(B, dtype=torch.int32, device=dev)
            S.stepq_pack(L.handle, B, slots, B, snap, pool, scales)
            rec = torch.empty_like(snap)
            S.stepq_unpack(L.handle, B, slots, B, pool, scales, rec)
            acc += ((rec.double() - snap.double()) ** 2).sum(dim=(0, 3)).cpu()
            n += B
        per_row = (acc / max(n, 1)) * w
        per_row = per_row.numpy()
        out[b] = per_row.sum(axis=1) if gate_mode == 0 else per_row.reshape(-1)
    return out


def allocate(lifetime, distortion: dict, widths, avg_bits: int, n_pivots: int) -> np.ndarray:
    """Exact lifetime-aware allocation.

    Pivots: the n_pivots units with the largest risk tau_u D_u(b_min) (ties to
    the lower index).  The remaining units choose widths from `widths`
    minimising sum_u tau_u D_u(b_u) subject to sum_u b_u = avg_bits * units
    (pivots counted at 16 bits), solved exactly by dynamic programming over the
    budget (all widths share the unit's row count, so the budget is a count of
    bits per row)."""
    life = np.asarray(lifetime, np.float64)
    n = life.size
    ws = sorted(int(x) for x in widths)
    life = np.where(np.isfinite(life), life, np.finfo(np.float64).max / 1e6)
    risk = life * np.asarray(distortion[ws[0]], np.float64)
    order = sorted(range(n), key=lambda u: (-risk[u], u))
    pivots = set(order[:n_pivots])
    free = [u for u in range(n) if u not in pivots]
    budget = avg_bits * n - PIVOT_BITS * len(pivots)
    g = int(np.gcd.reduce(ws + [budget]))
    cap = budget // g
    if budget < ws[0] * len(free) or budget > ws[-1] * len(free):
        raise ValueError("bit budget not reachable with these widths")
    cost = {b: life * np.asarray(distortion[b], np.float64) for b in ws}
    INF = np.inf
    # dp over units: best[c] = minimal cost using exactly c*g bits so far
    best = np.full(cap + 1, INF)
    best[0] = 0.0
    choice = np.zeros((len(free), cap + 1), np.int8)
    for k, u in enumerate(free):
        nxt = np.full(cap + 1, INF)
        arg = np.zeros(cap + 1, np.int8)
        for bi, b in enumerate(ws):
            s = b // g
            cand = np.full(cap + 1, INF)
            cand[s:] = best[: cap + 1 - s] + cost[b][u]
            better = cand < nxt
            nxt = np.where(better, cand, nxt)
            arg = np.where(better, bi, arg)
        best = nxt
        choice[k] = arg
    if not np.isfinite(best[cap]):
        raise ValueError("bit budget not reachable with these widths")
    bits = np.zeros(n, np.int64)
    for u in pivots:
        bits[u] = PIVOT_BITS
    c = cap
    for k in range(len(free) - 1, -1, -1):
        b = ws[choice[k, c]]
        bits[free[k]] = b
        c -= b // g
    assert c == 0
    return bits.astype(np.uint8)


def calibrate(H: int, D: int, gate_mode: int, S0, step_inputs, widths, avg_bits: int, n_pivots: int,
              snapshot_every: int = 16, max_snapshots: int = 8, horizon: int | None = None) -> Calibration:
    """Statistics, distortion table and allocation in one pass (see module doc).
    The layout to serve with takes stats.scale_impact as its row impact,
    stats.row_magnitude as its row magnitudes and unit_bits as its widths."""
    stats = collect_statistics(H, D, gate_mode, S0, step_inputs, snapshot_every, max_snapshots, horizon)
    dist = measure_distortion(H, D, gate_mode, stats, widths)
    bits = allocate(stats.lifetime, dist, widths, avg_bits, n_pivots)
    return Calibration(stats=stats, widths=tuple(widths), distortion=dist, unit_bits=bits)


def main(argv=None) -> int:
    """Calibrates a layout for one of the synthetic workloads on the GPU and
    saves it: widths (unit_bits), the row impact the layout should use
    (row_impact: the scale impact), row magnitudes, lifetimes, the per-step
    readout weights and the distortion table (npz).

        python -m quantized_recurrent_state_packed_amd.calibrate --workload kimi-kda-b64 --horizon 512 --out kda.npz
    """
    import argparse
    import time

    import torch

    from . import workloads as W
    ap = argparse.ArgumentParser(description="offline calibration and lifetime-aware allocation")
    ap.add_argument("--workload", "--config", dest="config", metavar="NAME", type=W.workload_id, default="kimi-kda-b64",
                    help="workload name or index (workloads.CONFIGS)")
    ap.add_argument("--requests", type=int, default=4, help="calibration requests (ids 1000, 1001, ...)")
    ap.add_argument("--steps", type=int, default=64, help="decode steps of the FP32-state trajectories")
    ap.add_argument("--widths", type=str, default="4,6,8", help="candidate integer widths")
    ap.add_argument("--avg-bits", type=int, default=6, help="average bits per element, pivots included")
    ap.add_argument("--pivots", type=int, default=None,
                    help="binary16 pivot units (default: the workload's own count)")
    ap.add_argument("--horizon", type=int, default=None,
                    help="decode length capping the lifetimes in the scale impact (default: per-step impact)")
    ap.add_argument("--snapshot-every", type=int, default=16)
    ap.add_argument("--out", type=str, required=True)
    a = ap.parse_args(argv)
    lay = W.make_layout(a.config)
    req = list(range(1000, 1000 + a.requests))
    S0 = torch.from_numpy(W.make_initial_state(a.config, req, lay)).cuda()
    steps = ({k: torch.from_numpy(v).cuda() for k, v in W.make_step_inputs(a.config, t, req, lay, q_law="impact").items()}
             for t in range(a.steps))
    widths = tuple(int(x) for x in a.widths.split(","))
    n_piv = a.pivots if a.pivots is not None else int((lay.unit_bits == PIVOT_BITS).sum())
    t0 = time.perf_counter()
    cal = calibrate(lay.H, lay.D, lay.gate_mode, S0, steps, widths, a.avg_bits, n_piv,
                    snapshot_every=a.snapshot_every, horizon=a.horizon)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = cal.stats
    np.savez(a.out, H=lay.H, D=lay.D, gate_mode=lay.gate_mode, unit_bits=cal.unit_bits,
             row_impact=st.scale_impact, row_magnitude=st.row_magnitude, lifetime=st.lifetime,
             readout_weight=st.row_impact, widths=np.array(widths),
             **{f"distortion_{b}": d for b, d in cal.distortion.items()})
    hist = {int(b): int((cal.unit_bits == b).sum()) for b in np.unique(cal.unit_bits)}
    print(f"{W.CONFIGS[a.config]['name']}: {cal.unit_bits.size} units, widths {hist}, "
          f"{cal.unit_bits.mean():.2f} bits average, horizon {a.horizon}, {dt:.2f} s -> {a.out}")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
