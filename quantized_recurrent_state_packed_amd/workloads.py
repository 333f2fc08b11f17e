"""Seeded synthetic workloads for the STEPQuant packed-state decode step.

This module draws inputs only.  It holds none of the step's arithmetic (no
reconstruction, no update, no quantisation); both the HIP path and the oracle
consume what it returns, so it is the one piece of code they share.

What it produces, per workload:
  * a layout: per-unit bit widths (a whole head under the scalar gate, a key row
    under the per-key-channel gate), fixed row-impact weights, calibrated row
    magnitudes, and the fixed gates from which unit lifetimes are read;
  * the initial recurrent state of each request;
  * per decode step: q, k (L2-normalised), v, beta and the gate.

Row-impact weights are the expected squared query weight of a key row (the
readout o = M'^T q weighs row i's error by q_i).  Queries follow one of two
laws: "isotropic" (the default: q ~ N(0, I), L2-normalised, as the workload
recipes state it) or "impact" (q ~ N(0, diag w), L2-normalised, so that the
layout's weights are the true impact of each key row: the calibration and
drift studies use it).  Outlier key rows and value columns are channels of a
head, the same for every request.  The calibrated row magnitude
of a row is the RMS the row's initial-state law gives it: a synthetic stand-in
for the offline calibration statistic, handed in like the impact weights.

The bit widths come from a small greedy stand-in for the offline lifetime-aware
allocator (STEPQuant summary pages: "Lifetime-aware Bit Allocation" -- widths
spent where errors are large and long-lived under a fixed average budget, the
riskiest units kept as FP16 pivots counted inside the budget).  The library
itself never allocates bits; the allocation is an input, like the random draws.

Random numbers: numpy PCG64 streams keyed by SeedSequence([base, stream, ...]),
drawn in float64 and rounded once to float32.  Per-step inputs are keyed per
(step, request), so any slice of requests can be regenerated on its own.
For the full-size serving shape a device-side generator (torch Philox) follows
the same recipe with different values; its outputs are copied to the host when
the oracle needs them.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260000

STREAM_LAYOUT = 0
STREAM_STATE = 1
STREAM_STEP = 2

# Workload recipes.  Shapes, lifetimes, bit budgets, pivot fractions, impact
# weight spreads and outlier structure follow the serving workloads the pages
# describe (Qwen-style gated DeltaNet with a per-head gate, Kimi-style KDA with
# a per-key-channel gate, a batch-512 serving shape, a long 4-bit stress run).
CONFIGS = {
    0: dict(name="tiny-sanity", B=1, H=1, D=16, T=64, gate_mode=0,
            gate="per_step", gate_logit=(-3.0, 1.0),
            bits="uniform", uniform_bits=6, pivot_frac=0.0,
            omega="uniform", omega_range=(0.5, 2.0), outliers=False),
    1: dict(name="qwen-gdn-b32", B=32, H=48, D=128, T=256, gate_mode=0,
            gate="halflife", halflife=(1.0, 1000.0),
            bits="alloc", widths=(4, 6, 8), avg_bits=6, pivot_frac=0.02,
            omega="lognormal", omega_sigma=0.5, outliers=False),
    2: dict(name="kimi-kda-b64", B=64, H=32, D=128, T=512, gate_mode=1,
            gate="kda", kda_logit=(-4.0, 1.5),
            bits="alloc", widths=(4, 6, 8), avg_bits=6, pivot_frac=0.01,
            omega="lognormal", omega_sigma=0.5, outliers=True),
    3: dict(name="serving-b512-h48-d128", B=512, H=48, D=128, T=128, gate_mode=0,
            gate="halflife", halflife=(1.0, 1000.0),
            bits="alloc", widths=(4, 6, 8), avg_bits=6, pivot_frac=0.02,
            omega="lognormal", omega_sigma=0.5, outliers=False),
    4: dict(name="long-4bit-b16", B=16, H=48, D=128, T=2048, gate_mode=0,
            gate="halflife", halflife=(100.0, 5000.0),
            bits="alloc", widths=(2, 4, 6), avg_bits=4, pivot_frac=0.02,
            omega="lognormal", omega_sigma=1.0, outliers=True),
}



def workload_id(key: str | int) -> int:
    """Index of a workload given by name ("kimi-kda-b64") or by index ("2").

    The index is also the workload's seed offset.  Used as an argparse type;
    an unknown key raises ValueError, which argparse reports as a usage error.
    """
    s = str(key).strip()
    for i, c in CONFIGS.items():
        if s == c["name"] or s == str(i):
            return i
    names = ", ".join(f"{c['name']} ({i})" for i, c in CONFIGS.items())
    raise ValueError(f"unknown workload {key!r}; known: {names}")


STATE_STD = 0.1          # S0 ~ N(0, 0.1^2)
OUTLIER_FRAC = 0.02      # 2 % of a head's key rows and 2 % of its value columns
OUTLIER_GAIN = 30.0


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _round_count(frac: float, n: int) -> int:
    """A fraction of a small count: nearest integer, at least one (if frac > 0)."""
    if frac <= 0.0:
        return 0
    return max(1, int(math.floor(frac * n + 0.5)))


@dataclass
class Layout:
    cfg: int
    H: int
    D: int
    gate_mode: int                 # 0 scalar per (request, head); 1 per key channel
    unit_bits: np.ndarray          # uint8, [H] (mode 0) or [H*D] (mode 1)
    row_impact: np.ndarray         # float32, [H*D]
    lifetime: np.ndarray           # float64, one per unit (e-folding steps)
    fixed_gate: np.ndarray | None  # float32 [H] or [H*D]; None when drawn per step
    row_magnitude: np.ndarray | None = None   # float32 [H*D], calibrated row RMS
    row_mode: int = 1              # 1: calibrated row scales; 0: refitted every step
    outlier_rows: np.ndarray | None = None    # int [H, n] outlier key rows per head
    outlier_cols: np.ndarray | None = None    # int [H, n] outlier value columns per head
    extra: dict = field(default_factory=dict)

    @property
    def n_units(self) -> int:
        return int(self.unit_bits.size)

    def row_bits(self) -> np.ndarray:
        """Width of every key row, [H, D]."""
        if self.gate_mode == 0:
            return np.repeat(self.unit_bits.reshape(self.H, 1), self.D, axis=1)
        return self.unit_bits.reshape(self.H, self.D).copy()


def allocate_bits(lifetime: np.ndarray, widths, avg_bits: int, n_pivots: int) -> np.ndarray:
    """Synthetic stand-in for the offline lifetime-aware allocator.

    1. The n_pivots units with the longest lifetime become FP16 pivots (16 bits).
    2. Every other unit starts at the smallest width.
    3. Repeatedly widen (+2 bits) the unit with the largest lifetime-weighted
       distortion drop tau * (2^-2b - 2^-2(b+2)) until the average, pivots
       included, is exactly avg_bits.  Ties go to the lower unit index.
    """
    widths = sorted(int(w) for w in widths)
    wmin, wmax = widths[0], widths[-1]
    n = lifetime.size
    order = sorted(range(n), key=lambda u: (-float(lifetime[u]), u))
    bits = np.full(n, wmin, dtype=np.int64)
    pivots = set(order[:n_pivots])
    for u in pivots:
        bits[u] = 16
    remaining = avg_bits * n - int(bits.sum())
    if remaining < 0 or remaining % 2:
        raise ValueError("bit budget not reachable with +2 steps")
    heap = []
    for u in range(n):
        if u in pivots or bits[u] >= wmax:
            continue
        gain = float(lifetime[u]) * (2.0 ** (-2 * int(bits[u])) - 2.0 ** (-2 * (int(bits[u]) + 2)))
        heap.append((-gain, u))
    heapq.heapify(heap)
    while remaining > 0:
        if not heap:
            raise ValueError("bit budget exceeds the widest allocation")
        _, u = heapq.heappop(heap)
        bits[u] += 2
        remaining -= 2
        if bits[u] < wmax:
            b = int(bits[u])
            gain = float(lifetime[u]) * (2.0 ** (-2 * b) - 2.0 ** (-2 * (b + 2)))
            heapq.heappush(heap, (-gain, u))
    return bits.astype(np.uint8)


def make_layout(cfg: int) -> Layout:
    c = CONFIGS[cfg]
    H, D = c["H"], c["D"]
    g = _rng(SEED_BASE + cfg, STREAM_LAYOUT)
    fixed_gate = None
    if c["gate"] == "halflife":
        lo, hi = c["halflife"]
        hl = 10.0 ** g.uniform(math.log10(lo), math.log10(hi), size=H)
        a = 2.0 ** (-1.0 / hl)
        fixed_gate = a.astype(np.float32)
        lifetime = hl / math.log(2.0)
    elif c["gate"] == "kda":
        mu, sd = c["kda_logit"]
        x = g.normal(mu, sd, size=H * D)
        a = np.exp(-_softplus(x))
        fixed_gate = a.astype(np.float32)
        lifetime = -1.0 / np.log(a.astype(np.float32).astype(np.float64))
    else:  # per-step gate: lifetime from the mean log retention of its law
        mu, sd = c["gate_logit"]
        lifetime = np.full(H, 1.0 / float(np.mean(_softplus(g.normal(mu, sd, size=4096)))))
    if c["omega"] == "uniform":
        lo, hi = c["omega_range"]
        omega = g.uniform(lo, hi, size=H * D)
    else:
        omega = g.lognormal(0.0, c["omega_sigma"], size=H * D)
    n_units = H if c["gate_mode"] == 0 else H * D
    # outlier channels of each head, and the row RMS the initial-state law gives
    go = _rng(SEED_BASE + cfg, STREAM_LAYOUT, 1)
    n_out = _round_count(OUTLIER_FRAC, D) if c["outliers"] else 0
    out_rows = np.stack([go.choice(D, size=n_out, replace=False) for _ in range(H)]) if n_out else None
    out_cols = np.stack([go.choice(D, size=n_out, replace=False) for _ in range(H)]) if n_out else None
    row_gain, col_gain = _outlier_gains(H, D, out_rows, out_cols)
    row_mag = STATE_STD * row_gain * np.sqrt((col_gain ** 2).mean(axis=1, keepdims=True))
    if c["bits"] == "uniform":
        unit_bits = np.full(n_units, c["uniform_bits"], dtype=np.uint8)
    else:
        n_piv = _round_count(c["pivot_frac"], n_units)
        unit_bits = allocate_bits(np.asarray(lifetime, dtype=np.float64), c["widths"],
                                  c["avg_bits"], n_piv)
    return Layout(cfg=cfg, H=H, D=D, gate_mode=c["gate_mode"], unit_bits=unit_bits,
                  row_impact=omega.astype(np.float32), lifetime=np.asarray(lifetime, np.float64),
                  fixed_gate=fixed_gate, row_magnitude=row_mag.reshape(-1).astype(np.float32),
                  outlier_rows=out_rows, outlier_cols=out_cols)


def _outlier_gains(H: int, D: int, rows, cols):
    """Per-head row and column gain vectors ([H, D] each, 1 or OUTLIER_GAIN)."""
    rg = np.ones((H, D))
    cg = np.ones((H, D))
    if rows is not None:
        for h in range(H):
            rg[h, rows[h]] = OUTLIER_GAIN
            cg[h, cols[h]] = OUTLIER_GAIN
    return rg, cg


def make_initial_state(cfg: int, requests, layout: Layout | None = None) -> np.ndarray:
    """float32 [len(requests), H, D, D]; row index = key channel, column = value channel.
    N(0, STATE_STD^2), times OUTLIER_GAIN on the head's outlier rows and columns."""
    c = CONFIGS[cfg]
    H, D = c["H"], c["D"]
    if layout is None:
        layout = make_layout(cfg)
    rg, cg = _outlier_gains(H, D, layout.outlier_rows, layout.outlier_cols)
    gain = rg[:, :, None] * cg[:, None, :]
    out = np.empty((len(requests), H, D, D), dtype=np.float32)
    for n, b in enumerate(requests):
        g = _rng(SEED_BASE + cfg, STREAM_STATE, int(b))
        out[n] = (g.normal(0.0, STATE_STD, size=(H, D, D)) * gain).astype(np.float32)
    return out


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


Q_LAWS = ("isotropic", "impact")


def _q_scale(layout: Layout, q_law: str) -> np.ndarray:
    """Per-row standard deviation of the query draw before normalisation, [H, D]."""
    if q_law == "isotropic":
        return np.ones((layout.H, layout.D))
    if q_law == "impact":
        return np.sqrt(layout.row_impact.astype(np.float64)).reshape(layout.H, layout.D)
    raise ValueError(f"unknown query law {q_law!r}; known: {Q_LAWS}")


def make_step_inputs(cfg: int, t: int, requests, layout: Layout | None = None, q_law: str = "isotropic") -> dict:
    """Inputs of decode step t for the given requests (float32 arrays).

    q: [n, H, D] = normalise(N(0, I)) ("isotropic") or normalise(N(0, diag(w)))
    with w the row-impact weights ("impact"); k: [n, H, D] unit L2 norm,
    isotropic; v: [n, H, D]; beta: [n, H] = sigmoid(N(0,1)); gate (linear
    retention a in (0,1]): [n, H] (scalar gate) or [n, H, D] (KDA).  Both query
    laws use the same normal draws.
    """
    c = CONFIGS[cfg]
    H, D = c["H"], c["D"]
    if layout is None:
        layout = make_layout(cfg)
    n = len(requests)
    q = np.empty((n, H, D), np.float32)
    k = np.empty((n, H, D), np.float32)
    v = np.empty((n, H, D), np.float32)
    beta = np.empty((n, H), np.float32)
    gshape = (n, H) if c["gate_mode"] == 0 else (n, H, D)
    gate = np.empty(gshape, np.float32)
    qs = _q_scale(layout, q_law)
    for m, b in enumerate(requests):
        g = _rng(SEED_BASE + cfg, STREAM_STEP, int(t), int(b))
        q[m] = _unit(g.standard_normal((H, D)) * qs).astype(np.float32)
        k[m] = _unit(g.standard_normal((H, D))).astype(np.float32)
        v[m] = g.standard_normal((H, D)).astype(np.float32)
        beta[m] = _sigmoid(g.standard_normal(H)).astype(np.float32)
        if c["gate"] == "per_step":
            mu, sd = c["gate_logit"]
            gate[m] = np.exp(-_softplus(g.normal(mu, sd, size=H))).astype(np.float32)
        elif c["gate_mode"] == 0:
            gate[m] = layout.fixed_gate
        else:
            gate[m] = layout.fixed_gate.reshape(H, D)
    return dict(q=q, k=k, v=v, beta=beta, gate=gate)


def make_step_inputs_torch(cfg: int, t: int, B: int, device, layout: Layout | None = None,
                           q_law: str = "isotropic") -> dict:
    """Same recipe as make_step_inputs, drawn on a torch device (Philox).

    Used for the full-size serving shape, where host generation would dominate
    the run.  Values differ from the host generator; the distributions do not.
    """
    import torch
    c = CONFIGS[cfg]
    H, D = c["H"], c["D"]
    if layout is None:
        layout = make_layout(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed((SEED_BASE + cfg) * 1_000_003 + 7919 * int(t) + 1)
    f64 = torch.float64

    def nrm(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=f64)

    qs = torch.from_numpy(_q_scale(layout, q_law).reshape(1, H, D)).to(device)
    q = nrm(B, H, D) * qs
    q = (q / q.norm(dim=-1, keepdim=True)).float()
    k = nrm(B, H, D)
    k = (k / k.norm(dim=-1, keepdim=True)).float()
    v = nrm(B, H, D).float()
    beta = torch.sigmoid(nrm(B, H)).float()
    if c["gate"] == "per_step":
        mu, sd = c["gate_logit"]
        gate = torch.exp(-torch.nn.functional.softplus(nrm(B, H) * sd + mu)).float()
    elif c["gate_mode"] == 0:
        gate = torch.from_numpy(layout.fixed_gate).to(device).reshape(1, H).expand(B, H).contiguous()
    else:
        gate = torch.from_numpy(layout.fixed_gate).to(device).reshape(1, H, D).expand(B, H, D).contiguous()
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), beta=beta.contiguous(), gate=gate)


def make_initial_state_torch(cfg: int, B: int, device, layout: Layout | None = None) -> "torch.Tensor":
    """Device-side S0 with the same recipe as make_initial_state (values differ)."""
    import torch
    c = CONFIGS[cfg]
    H, D = c["H"], c["D"]
    if layout is None:
        layout = make_layout(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed((SEED_BASE + cfg) * 1_000_003 + 3)
    s = torch.randn(B, H, D, D, generator=gen, device=device, dtype=torch.float32) * STATE_STD
    if layout.outlier_rows is not None:
        rg, cg = _outlier_gains(H, D, layout.outlier_rows, layout.outlier_cols)
        gain = torch.from_numpy((rg[:, :, None] * cg[:, None, :]).astype(np.float32)).to(device)
        s = s * gain.unsqueeze(0)
    return s.contiguous()


def make_slot_ids(B: int, num_slots: int, seed: int = 0) -> np.ndarray:
    """Distinct pool slots for B requests, drawn from [0, num_slots)."""
    if num_slots < B:
        raise ValueError("need at least one slot per request")
    g = _rng(SEED_BASE, 99, int(seed))
    return g.permutation(num_slots)[:B].astype(np.int32)
