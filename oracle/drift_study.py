"""Drift and lifetime study of quantised recurrent states.

TEST INFRASTRUCTURE: it runs only the CPU oracle; nothing in the product
imports it.  Two measurements on the seeded synthetic workloads:

drift     From one initial state and one input sequence, the state is carried
          (a) in binary32 (the FP32-state trajectory), (b) in the workload's
          STEPQuant layout with row scales from the workload's row magnitudes
          ("stepq"), from row magnitudes calibrated on FP32 trajectories of other
          requests ("stepq-cal"; "stepq-cal-log" and "stepq-cal-med" combine
          the per-step row RMS by geometric mean and median instead), and
          refitted from the row RMS at every step ("stepq-refit"); and with the
          row-impact weights also multiplied by each row's lifetime capped at
          the run length ("stepq-life" on the workload's magnitudes,
          "stepq-cal-life" on the calibrated ones), (c) as
          uniform INT4 and INT8 with one absmax scale per tile, each
          requantised after every step.  Reported: how far the
          readout and the state of each quantised trajectory drift from the
          FP32-state one.  The pages compare these storage modes by task
          accuracy (ai.info summary, "Main Findings": uniform quantisation
          degrades sharply as bits drop; 4-bit STEPQuant beats uniform INT8);
          trajectory drift on synthetic dynamics is the measurable analog.

lifetime  For every unit (a head under the per-head gate, a key row under the
          per-channel KDA gate), its accumulated state error after T steps of a
          quantised trajectory against its lifetime: Spearman's rank
          correlation, and the share of the total error held by the
          longest-lived quarter of units.  The pages report rho of about 0.80
          over Qwen heads under uniform INT6 (ai.info summary, "Main Findings";
          ai-trend.me review, "결과"), and a longest-lived quarter holding
          52.5 % (Qwen) and 78.8 % (KDA) of the INT6 error (ai-papers.net
          article, "誤差が効く時と場所").

    python -m oracle.drift_study drift --workload long-4bit-b16 [--requests 16] [--steps 2048] [--out report.md] [--csv steps.csv]
    python -m oracle.drift_study lifetime --workload qwen-gdn-b32 [--bits 6] [--requests 8] [--modes int6,stepq,stepq-cal-life]
(--workload names a workload of quantized_recurrent_state_packed_amd/workloads.py, or gives its
index: tiny-sanity (0), qwen-gdn-b32 (1, Qwen-like heads), kimi-kda-b64 (2, Kimi-like KDA rows),
serving-b512-h48-d128 (3, the serving shape), long-4bit-b16 (4, the long 4-bit run).  The
default is long-4bit-b16 for the drift study and qwen-gdn-b32 for the lifetime study.)
"""
from __future__ import annotations

import argparse
import dataclasses
import math
import sys
import time
from pathlib import Path

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, str(Path(__file__).resolve().parent.parent))

from oracle import dense_ref                                      # noqa: E402
from oracle import oracle as O                                   # noqa: E402
from quantized_recurrent_state_packed_amd import workloads as W  # noqa: E402


# ------------------------------------------------------------ trajectories
class PackedTrajectory:
    """State carried in an oracle pool under a layout (binary32 rows = FP32 state)."""

    def __init__(self, lay, unit_bits, S0: np.ndarray, row_mag=None):
        self.ol = O.OracleLayout(lay.H, lay.D, lay.gate_mode, unit_bits, lay.row_impact, row_mag)
        n = S0.shape[0]
        self.slots = np.arange(n, dtype=np.int32)
        self.pool, self.scales = self.ol.new_pool(n)
        self.ol.pack(self.slots, S0, self.pool, self.scales)

    def step(self, inp: dict) -> np.ndarray:
        return self.ol.step(self.slots, inp, self.pool, self.scales)

    def state(self) -> np.ndarray:
        return self.ol.unpack(self.slots, self.pool, self.scales).astype(np.float64)


class UniformTrajectory:
    """State carried as uniform INT-b codes with one binary32 absmax scale per tile."""

    def __init__(self, lay, bits: int, S0: np.ndarray):
        self.bits, self.gate_mode = bits, lay.gate_mode
        self.codes, self.scale = O.uniform_pack(S0, bits)

    def step(self, inp: dict) -> np.ndarray:
        return O.uniform_step(self.codes, self.scale, inp, self.bits, self.gate_mode)

    def state(self) -> np.ndarray:
        return self.codes.astype(np.float64) * self.scale.astype(np.float64)[..., None, None]


CALIBRATION_REQUESTS = range(1000, 1004)   # disjoint from the evaluated requests


CAL_STATS = {"stepq-cal": "rms", "stepq-cal-log": "logmean", "stepq-cal-med": "median"}


def calibrate_row_magnitude(cfg: int, lay, steps: int, stat: str = "rms") -> np.ndarray:
    """Offline calibration of the row magnitudes from the FP32-state trajectory
    (dense float64 recurrence) of the calibration requests ([H*D] float32).
    Per step, a key row's RMS over requests and value columns; over the steps:
      rms      the RMS over all steps (the mean square, then the root);
      logmean  the geometric mean of the per-step RMS;
      median   the median of the per-step RMS.
    A row whose magnitude grows over the trajectory is weighted toward its late
    values by rms, evenly by logmean and median."""
    req = list(CALIBRATION_REQUESTS)
    S = np.swapaxes(W.make_initial_state(cfg, req, lay).astype(np.float64), -1, -2)
    per_step = np.zeros((steps, lay.H, lay.D))
    for t in range(steps):
        inp = W.make_step_inputs(cfg, t, req, lay, q_law="impact")
        S, _ = dense_ref.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"])
        per_step[t] = (S * S).mean(axis=(0, 2))   # S is value x key: mean over requests, columns
    if stat == "rms":
        m = np.sqrt(per_step.mean(axis=0))
    elif stat == "logmean":
        m = np.exp(0.5 * np.log(np.maximum(per_step, 1e-300)).mean(axis=0))
    elif stat == "median":
        m = np.sqrt(np.median(per_step, axis=0))
    else:
        raise ValueError(stat)
    return m.reshape(-1).astype(np.float32)


def lifetime_impact(lay, horizon: int) -> np.ndarray:
    """Row-impact weights that also count how long an error persists: w_i times
    the row's lifetime capped at the run length, normalised to mean 1
    ([H*D] float32).  An error injected into a row with retention a decays as
    a^t, so its summed squared effect on later readouts grows with the lifetime
    until the run ends first."""
    tau = np.asarray(lay.lifetime, np.float64)
    tau_rows = np.repeat(tau, lay.D) if lay.gate_mode == 0 else tau
    w = lay.row_impact.astype(np.float64) * np.minimum(tau_rows, horizon)
    return (w / w.mean()).astype(np.float32)


def make_trajectory(mode: str, lay, S0):
    if mode == "fp32":
        return PackedTrajectory(lay, np.full_like(lay.unit_bits, 32), S0)
    if mode == "stepq":
        return PackedTrajectory(lay, lay.unit_bits, S0, lay.row_magnitude)
    if mode in CAL_STATS:
        return PackedTrajectory(lay, lay.unit_bits, S0, lay.extra["row_magnitude_" + CAL_STATS[mode]])
    if mode in ("stepq-life", "stepq-cal-life"):
        lay_w = dataclasses.replace(lay, row_impact=lay.extra["lifetime_impact"])
        m = lay.row_magnitude if mode == "stepq-life" else lay.extra["row_magnitude_rms"]
        return PackedTrajectory(lay_w, lay.unit_bits, S0, m)
    if mode == "stepq-refit":
        return PackedTrajectory(lay, lay.unit_bits, S0, None)
    if mode.startswith("int"):
        return UniformTrajectory(lay, int(mode[3:]), S0)
    raise ValueError(mode)


def unit_errors(dM: np.ndarray, gate_mode: int) -> np.ndarray:
    """Squared state error per request and unit: [n, H] (per-head gate) or
    [n, H*D] (per-key-row gate)."""
    sq = dM * dM
    if gate_mode == 0:
        return sq.sum(axis=(-1, -2))
    return sq.sum(axis=-1).reshape(sq.shape[0], -1)


def checkpoints(T: int) -> list[int]:
    pts = [1]
    while pts[-1] * 2 < T:
        pts.append(pts[-1] * 2)
    return sorted(set(pts + [T]))


def run(cfg: int, modes: list[str], n_req: int, T: int, log=None) -> dict:
    """Run the FP32-state trajectory and every mode in lock-step on the same
    inputs.  Returns per-mode readout errors of every step, state errors at
    the checkpoints, and the final per-unit squared state error."""
    lay = W.make_layout(cfg)
    for m in modes:
        if m in CAL_STATS:
            lay.extra["row_magnitude_" + CAL_STATS[m]] = calibrate_row_magnitude(cfg, lay, min(T, 256), CAL_STATS[m])
    if "stepq-cal-life" in modes and "row_magnitude_rms" not in lay.extra:
        lay.extra["row_magnitude_rms"] = calibrate_row_magnitude(cfg, lay, min(T, 256), "rms")
    lay.extra["lifetime_impact"] = lifetime_impact(lay, T)
    req = list(range(n_req))
    S0 = W.make_initial_state(cfg, req, lay)
    ref = make_trajectory("fp32", lay, S0)
    trajs = {m: make_trajectory(m, lay, S0) for m in modes}
    pts = checkpoints(T)
    res = {m: dict(o_rel=np.zeros(T), state_rel={}, unit_sq=None) for m in modes}
    t0 = time.perf_counter()
    for t in range(T):
        inp = W.make_step_inputs(cfg, t, req, lay, q_law="impact")
        o_ref = ref.step(inp).astype(np.float64)
        o_norm = np.linalg.norm(o_ref)
        outs = {m: tr.step(inp).astype(np.float64) for m, tr in trajs.items()}
        for m in modes:
            res[m]["o_rel"][t] = np.linalg.norm(outs[m] - o_ref) / o_norm
        if t + 1 in pts:
            Mr = ref.state()
            mnorm = np.linalg.norm(Mr)
            for m, tr in trajs.items():
                dM = tr.state() - Mr
                res[m]["state_rel"][t + 1] = float(np.linalg.norm(dM) / mnorm)
                if t + 1 == T:
                    res[m]["unit_sq"] = unit_errors(dM, lay.gate_mode)
            if log:
                log(f"step {t + 1}/{T}  {time.perf_counter() - t0:.1f} s  " +
                    "  ".join(f"{m} {res[m]['state_rel'][t + 1]:.3e}" for m in modes))
    return dict(layout=lay, checkpoints=pts, modes=res, seconds=time.perf_counter() - t0)


def spearman(x: np.ndarray, y: np.ndarray) -> float:
    from scipy.stats import spearmanr
    return float(spearmanr(x, y).statistic)


def lifetime_stats(lay, unit_sq: np.ndarray) -> dict:
    """Spearman of the mean accumulated squared state error per unit against
    the unit's lifetime, and the longest-lived quarter's share of the error."""
    err = unit_sq.mean(axis=0)
    life = np.asarray(lay.lifetime, np.float64)
    order = np.argsort(-life, kind="stable")
    top = order[: int(math.ceil(life.size / 4))]
    return dict(units=int(life.size), spearman=spearman(life, err),
                top_quarter_share=float(err[top].sum() / err.sum()))


# ------------------------------------------------------------------ report
def drift_report(r: dict, cfg: int, n_req: int) -> str:
    lay, pts, modes = r["layout"], r["checkpoints"], r["modes"]
    c = W.CONFIGS[cfg]
    avg = lay.row_bits().mean()
    lines = [f"# Drift against the FP32-state trajectory: {c['name']}",
             "",
             f"Workload: requests 0..{n_req - 1} of `{c['name']}` (H={lay.H}, D={lay.D}, "
             f"gate mode {lay.gate_mode}), {pts[-1]} steps; STEPQuant layout at {avg:.2f} bits per "
             f"element including pivots; uniform INT-b with one absmax scale per tile.  Queries follow "
             f"the impact-shaped law q ~ N(0, diag w) (the layout's weights are each key row's true "
             f"readout weight).  Oracle run time {r['seconds']:.0f} s on {O.num_threads()} threads.",
             "",
             "Relative state error ||M - M_fp32||_F / ||M_fp32||_F (all tiles):",
             "",
             "| step | " + " | ".join(modes) + " |",
             "|---|" + "---|" * len(modes)]
    for p in pts:
        lines.append(f"| {p} | " + " | ".join(f"{modes[m]['state_rel'][p]:.3e}" for m in modes) + " |")
    lines += ["",
              "Relative readout error ||o - o_fp32|| / ||o_fp32|| (all tiles), at the step and averaged "
              "over steps 1..t:",
              "",
              "| step | " + " | ".join(f"{m} (step) | {m} (mean)" for m in modes) + " |",
              "|---|" + "---|---|" * len(modes)]
    for p in pts:
        cells = []
        for m in modes:
            o = modes[m]["o_rel"]
            cells += [f"{o[p - 1]:.3e}", f"{o[:p].mean():.3e}"]
        lines.append(f"| {p} | " + " | ".join(cells) + " |")
    lines += ["", "Accumulated state error per unit against lifetime (final step):", "",
              "| mode | units | Spearman rho | longest-lived quarter's share |", "|---|---|---|---|"]
    for m in modes:
        s = lifetime_stats(lay, modes[m]["unit_sq"])
        lines.append(f"| {m} | {s['units']} | {s['spearman']:.3f} | {100 * s['top_quarter_share']:.1f} % |")
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("study", choices=["drift", "lifetime"])
    ap.add_argument("--workload", "--config", dest="config", metavar="NAME", type=W.workload_id, default=None,
                    help="workload name or index (workloads.CONFIGS)")
    ap.add_argument("--requests", type=int, default=None)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--bits", type=int, default=6, help="uniform width of the lifetime study")
    ap.add_argument("--modes", type=str, default=None,
                    help="comma-separated modes (default: the study's own set); calibration statistics: "
                         + ", ".join(f"{k} ({v})" for k, v in CAL_STATS.items()))
    ap.add_argument("--out", type=Path, default=None)
    ap.add_argument("--csv", type=Path, default=None,
                    help="per-step relative readout error of every mode (one row per step)")
    args = ap.parse_args(argv)
    cfg = args.config if args.config is not None else (4 if args.study == "drift" else 1)
    c = W.CONFIGS[cfg]
    n_req = min(args.requests or c["B"], c["B"])
    T = min(args.steps or c["T"], c["T"])
    modes = (["stepq", "stepq-cal", "stepq-refit", "int4", "int8"] if args.study == "drift"
             else [f"int{args.bits}", "stepq", "stepq-cal", "stepq-refit"])
    if args.modes:
        modes = args.modes.split(",")
    r = run(cfg, modes, n_req, T, log=lambda s: print(s, file=sys.stderr, flush=True))
    text = drift_report(r, cfg, n_req)
    text += "\nCommand: python -m oracle.drift_study " + " ".join(argv if argv is not None else sys.argv[1:]) + "\n"
    if args.out:
        args.out.parent.mkdir(parents=True, exist_ok=True)
        args.out.write_text(text)
    if args.csv:
        args.csv.parent.mkdir(parents=True, exist_ok=True)
        names = list(r["modes"])
        with args.csv.open("w") as f:
            f.write("step," + ",".join(f"{m}_readout_rel" for m in names) + "\n")
            for t in range(T):
                f.write(f"{t + 1}," + ",".join(f"{r['modes'][m]['o_rel'][t]:.6e}" for m in names) + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
