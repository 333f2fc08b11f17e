"""Free-running comparison of the HIP path and the oracle (reported, not gated).

Both start from the same packed initial state: the oracle packs S0, and its
pool and scales are uploaded as the GPU's.  Each then steps its own pool with
the same seeded inputs for T steps, so differences accumulate: a code that
rounds differently at a near-tie in one step changes every later step of that
tile.  Per step the report gives:
  - the share of integer codes that differ between the two pools and the
    largest |code difference|;
  - the share of binary16 column scales that differ and the largest ulp gap;
  - the readout relative L2 between the two paths, over all (b, h, j);
  - each path's readout relative L2 against the float64 dense recurrence
    from the same unquantised S0 (oracle/dense_ref.py), i.e. the
    quantisation error itself, which the first two should not move.

Run on a GPU, from the repository root (--workload: a workload name or index of
quantized_recurrent_state_packed_amd/workloads.py):
    python tests/free_running.py --workload qwen-gdn-b32 --requests 8 --steps 256 \
        --out tests/reports/free_running_qwen_gdn.md --csv tests/reports/free_running_qwen_gdn.csv
"""
from __future__ import annotations

import argparse
import dataclasses
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

from oracle import dense_ref                                        # noqa: E402
from oracle import oracle as O                                      # noqa: E402
from quantized_recurrent_state_packed_amd import workloads as W     # noqa: E402


def _rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _signed(fields, bits):
    f = fields.astype(np.int64)
    b = bits[:, None].astype(np.int64)
    return np.where(f >= (1 << (b - 1)), f - (1 << b), f)


def compare(ol, slots, pg, sg, po, so):
    """Code and column-scale differences between two pools of the same layout."""
    rb = ol.row_bits()
    D = ol.D
    n_int = n_diff = 0
    max_d = 0
    n_sc = n_sc_diff = 0
    max_ulp = 0
    sg16 = sg.reshape(-1, ol.H, 2 * D)
    so16 = so.reshape(-1, ol.H, 2 * D)
    for s_ in slots:
        for h in range(ol.H):
            is_int = rb[h] <= 8
            if not is_int.any():
                continue
            fg = ol.decode_tile(h, ol.tile_words(pg, int(s_), h))
            fo = ol.decode_tile(h, ol.tile_words(po, int(s_), h))
            cg = _signed(fg[is_int], rb[h][is_int])
            co = _signed(fo[is_int], rb[h][is_int])
            d = np.abs(cg - co)
            n_int += d.size
            n_diff += int(np.count_nonzero(d))
            max_d = max(max_d, int(d.max()))
            a = sg16[s_, h, D:].astype(np.int64)
            b = so16[s_, h, D:].astype(np.int64)
            u = np.abs(a - b)          # positive binary16 values: bit-pattern distance = ulps
            n_sc += u.size
            n_sc_diff += int(np.count_nonzero(u))
            max_ulp = max(max_ulp, int(u.max()))
    return dict(code_diff_share=n_diff / max(n_int, 1), max_code_diff=max_d,
                scale_diff_share=n_sc_diff / max(n_sc, 1), max_scale_ulp=max_ulp)


def run(cfg: int, n_req: int, steps: int, calibrated: bool = True, log=print) -> list:
    import torch
    from quantized_recurrent_state_packed_amd import stepq as S
    lay = W.make_layout(cfg)
    if not calibrated:
        lay = dataclasses.replace(lay, row_mode=0)
    ol = O.OracleLayout.from_workload(lay)
    L = S.Layout.from_workload(lay)
    req = list(range(n_req))
    slots = np.arange(n_req, dtype=np.int32)
    S0 = W.make_initial_state(cfg, req, lay)
    po, so = ol.new_pool(n_req)
    ol.pack(slots, S0, po, so)
    pool = torch.from_numpy(po.copy()).cuda()
    scales = torch.from_numpy(so.copy().view(np.int16)).cuda()
    sd = torch.from_numpy(slots).cuda()
    Sd = np.swapaxes(S0.astype(np.float64), -1, -2)          # dense recurrence: value x key
    rows = []
    for t in range(steps):
        inp = W.make_step_inputs(cfg, t, req, lay, q_law="impact")
        dv = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
        o_g = torch.empty(n_req, lay.H, lay.D, dtype=torch.float32, device="cuda")
        S.stepq_decode_step(L.handle, n_req, sd, n_req, dv["q"], dv["k"], dv["v"], dv["beta"], dv["gate"],
                            pool, scales, o_g)
        torch.cuda.synchronize()
        o_o = ol.step(slots, inp, po, so)
        Sd, o_d = dense_ref.dense_step(Sd, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"])
        og = o_g.cpu().numpy()
        pg, sg = pool.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
        row = dict(step=t + 1, **compare(ol, slots, pg, sg, po, so),
                   o_gpu_vs_oracle=_rel(og, o_o), o_gpu_vs_dense=_rel(og, o_d), o_oracle_vs_dense=_rel(o_o, o_d))
        rows.append(row)
        if (t + 1) & t == 0 or (t + 1) % 64 == 0 or t + 1 == steps:
            log(f"step {t + 1}: " + ", ".join(f"{k} {v:.3g}" for k, v in row.items() if k != "step"))
    return rows


def report(rows, cfg, n_req, mode) -> str:
    keys = ["code_diff_share", "max_code_diff", "scale_diff_share", "max_scale_ulp", "o_gpu_vs_oracle",
            "o_gpu_vs_dense", "o_oracle_vs_dense"]
    marks = sorted({r["step"] for r in rows if r["step"] & (r["step"] - 1) == 0} | {rows[-1]["step"]})
    lines = [f"# Free-running HIP path vs oracle — {W.CONFIGS[cfg]['name']} ({n_req} requests, {len(rows)} steps, "
             f"{mode} row scales)", "",
             "Both paths start from the oracle's packing of the same initial state and then step their own "
             "pools with the same inputs (tests/free_running.py).  Code and scale columns compare the two "
             "pools; readout columns are relative L2 over all (b, h, j); \"dense\" is the float64 recurrence "
             "from the unquantised initial state.  Queries follow the impact-shaped law q ~ N(0, diag w).", "",
             "| step | " + " | ".join(keys) + " |", "|" + "---|" * (len(keys) + 1)]
    by_step = {r["step"]: r for r in rows}
    for s_ in marks:
        r = by_step[s_]
        lines.append(f"| {s_} | " + " | ".join(f"{r[k]:.3g}" if isinstance(r[k], float) else str(r[k])
                                                for k in keys) + " |")
    worst = max(r["o_gpu_vs_oracle"] for r in rows)
    gap = max(abs(r["o_gpu_vs_dense"] - r["o_oracle_vs_dense"]) / max(r["o_oracle_vs_dense"], 1e-300) for r in rows)
    lines += ["", f"Largest readout gap between the two paths over the run: {worst:.3g} (relative L2).  "
              f"Largest relative difference between their errors against the dense recurrence: {gap:.3g}.", ""]
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", "--config", dest="config", metavar="NAME", type=W.workload_id, default="qwen-gdn-b32",
                    help="workload name or index (workloads.CONFIGS)")
    ap.add_argument("--requests", type=int, default=8)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--refit", action="store_true", help="per-step row refit instead of calibrated row scales")
    ap.add_argument("--out", type=Path)
    ap.add_argument("--csv", type=Path)
    a = ap.parse_args(argv)
    rows = run(a.config, a.requests, a.steps, calibrated=not a.refit)
    text = report(rows, a.config, a.requests, "refit" if a.refit else "calibrated")
    text += "Command: python tests/free_running.py " + " ".join(argv if argv is not None else sys.argv[1:]) + "\n"
    print(text)
    if a.out:
        a.out.parent.mkdir(parents=True, exist_ok=True)
        a.out.write_text(text)
    if a.csv:
        a.csv.parent.mkdir(parents=True, exist_ok=True)
        keys = list(rows[0])
        a.csv.write_text(",".join(keys) + "\n" + "\n".join(",".join(f"{r[k]:.6e}" if isinstance(r[k], float)
                                                                     else str(r[k]) for k in keys) for r in rows) + "\n")


if __name__ == "__main__":
    main()
