"""Step-locked parity between the HIP path (through the C ABI) and the oracle.

At every step the oracle starts from the pool and scales the GPU left after
the previous step, applies the same inputs, and the two results are compared
tile by tile:
  * integer codes: equal, except +-1 flips (the kernel decides in binary32,
    the oracle rounds the float64 quotient: values within a few binary32 ulps
    of a rounding tie may go either way), counted over the run;
  * binary16 pivots and binary16 row scales: within one unit in the last place,
    plus the binary32 forward-error bound of the update where a row is ill
    conditioned (see allowed_ulps); calibrated row scales (a layout constant):
    bit-exact;
  * binary16 column scales: the same bound, against the oracle's
    least-squares fit for the GPU's own codes of that column (the fit is
    defined for fixed codes, so a column holding a tie flip is fitted to the
    codes the GPU actually stored);
  * binary32 (zero-loss) rows: within 1e-5 of the row's largest magnitude;
  * readout o: relative L2 error <= 1e-4 at every step, for the fused step
    and, where a test asks for it, for the split-phase readout (stepq_readout)
    taken from the same pool before the step;
  * the GPU words re-encode exactly from their own fields (layout, zero padding).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

O_TOL = 1e-4
FLIP_BUDGET = 1e-4
EPS32 = 2.0 ** -24
HALF_ULP_REL = 2.0 ** -11     # relative spacing of binary16 values (upper bound 2^-10)


def update_error_scale(ctx: dict) -> np.ndarray:
    """Per element A_ij such that the binary32 kernel's updated state obeys
    |M'_gpu - M'| <= D * eps32 * A_ij (standard forward error bound of
    M' = M~ + beta k (v - sum_i k_i M~_i), with the D-term sum accumulated in
    binary32; D * eps32 bounds the accumulation, the few remaining roundings
    are absorbed in the same factor).  ctx: float64 M~ (decayed state), k, v,
    beta of the tile."""
    Mt, k, v, beta = ctx["Mt"], np.abs(ctx["k"]), np.abs(ctx["v"]), abs(float(ctx["beta"]))
    col = (k[:, None] * np.abs(Mt)).sum(axis=0)
    return np.abs(Mt) + beta * k[:, None] * (v[None, :] + col[None, :])


def allowed_ulps(rel: np.ndarray) -> np.ndarray:
    """1 ulp, plus the ulps a relative error bound rel can move a binary16 value."""
    return 1 + np.ceil(rel / HALF_ULP_REL).astype(np.int64)


def half_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(x):
        x = x.astype(np.int64) & 0xFFFF
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


def sign_extend(f: np.ndarray, bits: np.ndarray) -> np.ndarray:
    f = f.astype(np.int64)
    b = bits.astype(np.int64)[:, None]
    half = np.left_shift(1, b - 1)
    return np.where(f >= half, f - np.left_shift(1, b), f)


class Stats:
    def __init__(self):
        self.int_elems = 0
        self.flips = 0
        self.max_code_diff = 0
        self.piv_elems = 0
        self.piv_ulp1 = 0
        self.max_piv_ulp = 0
        self.max_scale_ulp = 0
        self.scale_ulp1 = 0
        self.scale_elems = 0
        self.max_rhat_ulp = 0
        self.max_chat_ulp = 0
        self.refit_columns = 0
        self.max_excess_ulp = 0       # ulps beyond the allowance (must stay <= 0)
        self.conditioned = 0          # scales/pivots that needed more than 1 ulp
        self.max_f32_err = 0.0
        self.o_rel = []
        self.readout_rel = []         # split-phase readout (stepq_readout) against the oracle
        self.layout_mismatch = 0
        self.rhat_mismatch = 0        # calibrated row scales that differ at all

    @property
    def flip_rate(self) -> float:
        return self.flips / max(1, self.int_elems)

    def as_dict(self) -> dict:
        return dict(int_elems=self.int_elems, flips=self.flips, flip_rate=self.flip_rate,
                    max_code_diff=self.max_code_diff, piv_elems=self.piv_elems, piv_ulp1=self.piv_ulp1,
                    max_piv_ulp=self.max_piv_ulp, scale_elems=self.scale_elems, scale_ulp1=self.scale_ulp1,
                    max_scale_ulp=self.max_scale_ulp, max_rhat_ulp=self.max_rhat_ulp,
                    max_chat_ulp=self.max_chat_ulp, refit_columns=self.refit_columns,
                    max_excess_ulp=self.max_excess_ulp, conditioned=self.conditioned,
                    max_f32_err=self.max_f32_err,
                    max_o_rel=max(self.o_rel) if self.o_rel else 0.0,
                    max_readout_rel=max(self.readout_rel) if self.readout_rel else None,
                    layout_mismatch=self.layout_mismatch,
                    rhat_mismatch=self.rhat_mismatch)

    def check(self) -> None:
        d = self.as_dict()
        assert self.layout_mismatch == 0, d
        assert self.rhat_mismatch == 0, d
        assert self.max_code_diff <= 1, d
        assert self.flip_rate <= FLIP_BUDGET, d
        assert self.max_excess_ulp <= 0, d
        assert self.max_scale_ulp < 99, d
        assert self.max_f32_err <= 1e-5, d
        assert not self.o_rel or max(self.o_rel) <= O_TOL, d
        assert not self.readout_rel or max(self.readout_rel) <= O_TOL, d


def compare_tile(ol: O.OracleLayout, h: int, wg, rg, cg, wo, ro, co, st: Stats, ctx_for=None) -> None:
    """ctx_for(): dict with the tile's float64 M' (before requantisation) and,
    for a decode step, M~, k, v, beta; needed only when a code differs (to
    refit column scales for the GPU's codes) or a value differs by more
    than one ulp (to bound the binary32 error of the update)."""
    rb = ol.row_bits()[h]
    D = ol.D
    fg = ol.decode_tile(h, wg)
    fo = ol.decode_tile(h, wo)
    if not np.array_equal(ol.encode_tile(h, fg), wg):
        st.layout_mismatch += 1
    is_int = rb <= 8
    piv = rb == 16
    ctx = None

    def get_ctx():
        nonlocal ctx
        if ctx is None:
            ctx = ctx_for() if ctx_for is not None else {}
        return ctx

    def row_rel():
        c = get_ctx()
        if "Mt" not in c:
            return np.zeros(D)
        A = update_error_scale(c)
        num = D * EPS32 * np.linalg.norm(A, axis=1)
        return num / np.maximum(np.linalg.norm(c["Mp"], axis=1), 1e-300)

    def account(u, allowed):
        st.max_excess_ulp = max(st.max_excess_ulp, int((u - allowed).max()))
        st.conditioned += int(np.count_nonzero(u > 1))

    if is_int.any():
        qg = sign_extend(fg[is_int], rb[is_int])
        qo = sign_extend(fo[is_int], rb[is_int])
        d = np.abs(qg - qo)
        st.int_elems += d.size
        st.flips += int(np.count_nonzero(d))
        st.max_code_diff = max(st.max_code_diff, int(d.max()))
        ur = half_ulp_distance(rg[is_int], ro[is_int])
        if ol.row_mag is not None:
            st.rhat_mismatch += int(np.count_nonzero(ur))
        ref = co
        if d.any() and ctx_for is not None:
            codes = np.zeros((D, D), np.int32)
            codes[is_int] = qg
            ref = ol.fit_columns_for_codes(h, get_ctx()["Mp"], codes)
            st.refit_columns += int(np.count_nonzero(d.max(axis=0)))
        uc = half_ulp_distance(cg, ref)
        st.scale_elems += ur.size + uc.size
        st.scale_ulp1 += int(np.count_nonzero(ur)) + int(np.count_nonzero(uc))
        st.max_rhat_ulp = max(st.max_rhat_ulp, int(ur.max()))
        st.max_chat_ulp = max(st.max_chat_ulp, int(uc.max()))
        if ur.max() > 1 or uc.max() > 1:
            rel = row_rel()
            account(ur, allowed_ulps(rel[is_int]))
            used = np.abs(np.where(is_int[:, None], 1, 0) * sign_extend(fg, rb)) > 0
            rel_c = np.where(used, rel[:, None], 0.0).max(axis=0)
            account(uc, allowed_ulps(rel_c))
        else:
            account(np.maximum(ur.max(), uc.max()), 1)
    else:
        if np.any(cg != 0) or np.any(co != 0):
            st.max_scale_ulp = max(st.max_scale_ulp, 99)
    if np.any(rg[~is_int] != 0) or np.any(ro[~is_int] != 0):
        st.max_scale_ulp = max(st.max_scale_ulp, 99)
    if piv.any():
        u = half_ulp_distance(fg[piv], fo[piv])
        st.piv_elems += u.size
        st.piv_ulp1 += int(np.count_nonzero(u))
        st.max_piv_ulp = max(st.max_piv_ulp, int(u.max()))
        if u.max() > 1:
            c = get_ctx()
            if "Mt" in c:
                A = update_error_scale(c)[piv]
                val = np.abs(fo[piv].astype(np.uint16).view(np.float16).astype(np.float64))
                ulp = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(val, 2.0 ** -14))) - 10), 2.0 ** -24)
                account(u, 1 + np.ceil(D * EPS32 * A / ulp).astype(np.int64))
            else:
                account(u, 1)
        else:
            account(u, 1)
    f32 = rb == 32
    if f32.any():
        a = fg[f32].astype(np.uint32).view(np.float32).astype(np.float64)
        b = fo[f32].astype(np.uint32).view(np.float32).astype(np.float64)
        scale = np.maximum(np.abs(b).max(axis=1, keepdims=True), 1e-30)
        st.max_f32_err = max(st.max_f32_err, float((np.abs(a - b) / scale).max()))


def compare_pools(ol: O.OracleLayout, slots, tiles, pool_g, sc_g, pool_o, sc_o, st: Stats, ctx_for=None) -> None:
    """ctx_for(b, h): the tile context compare_tile needs (see there)."""
    H = ol.H
    for t in tiles:
        b, h = divmod(int(t), H)
        s = int(slots[b])
        rg, cg = ol.tile_scales(sc_g, s, h)
        ro, co = ol.tile_scales(sc_o, s, h)
        f = None if ctx_for is None else (lambda b=b, h=h: ctx_for(b, h))
        compare_tile(ol, h, ol.tile_words(pool_g, s, h), rg, cg, ol.tile_words(pool_o, s, h), ro, co, st, f)


def o_rel(o_g: np.ndarray, o_o: np.ndarray, tiles, H: int) -> float:
    idx = [divmod(int(t), H) for t in tiles]
    a = np.stack([o_g[b, h] for b, h in idx]).astype(np.float64)
    b_ = np.stack([o_o[b, h] for b, h in idx]).astype(np.float64)
    return float(np.linalg.norm(a - b_) / max(np.linalg.norm(b_), 1e-30))
