"""Dense float64 gated Delta-rule recurrence (a second, independent CPU reference).

TEST INFRASTRUCTURE ONLY.  Written in the value-by-key orientation of the
update as usually stated for gated DeltaNet / KDA (ai-trend.me review,
"핵심 용어: Gated Delta Rule"; ai.info summary, "Methodology in Plain English"):

    S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

with S of shape (d_v, d_k); a scalar gate is Diag(a) = a I.  It uses plain
matrix products and shares nothing with the oracle's element loops, whose state
is the transpose M = S^T.
"""
from __future__ import annotations

import numpy as np


def dense_step(S: np.ndarray, q, k, v, beta, gate) -> tuple[np.ndarray, np.ndarray]:
    """One step for a batch of tiles.  S: (..., D, D) value-by-key, float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)[..., None, None]
    gate = np.asarray(gate, np.float64)
    D = k.shape[-1]
    eye = np.eye(D)
    if gate.ndim == k.ndim - 1:                      # one retention per tile
        decay = gate[..., None, None] * eye
    else:                                            # one retention per key channel
        decay = gate[..., None, :] * eye
    transition = decay @ (eye - beta * (k[..., :, None] * k[..., None, :]))
    S_new = S @ transition + beta * (v[..., :, None] * k[..., None, :])
    o = (S_new @ q[..., :, None])[..., 0]
    return S_new, o


def run(S0_keyrow: np.ndarray, steps) -> tuple[np.ndarray, list[np.ndarray]]:
    """Run from a key-row-oriented state M0 (..., d_k, d_v); returns the final
    key-row state and the readouts of every step."""
    S = np.swapaxes(np.asarray(S0_keyrow, np.float64), -1, -2).copy()
    outs = []
    for inp in steps:
        S, o = dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"])
        outs.append(o)
    return np.swapaxes(S, -1, -2), outs
