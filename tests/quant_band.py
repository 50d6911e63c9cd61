"""Comparison of quantised rows produced on the GPU with the oracle's, where the
two sides reach the pre-rounding value by different float32 evaluations.

The oracle rotates (RoPE, Hadamard) exactly in float64 and rounds once to
float32; the GPU evaluates the same rotations in float32 (butterflies, fused
multiply-adds). Both results are correct roundings of the same exact value up
to the float32 evaluation error, so a quantised code may legitimately differ by
one step where the exact value lies within that error of a rounding midpoint
(and an MXFP4 shared exponent where the block's largest magnitude lies within it
of a power of two). Everything else must agree exactly.

Error bound used (absolute, per element of a row): the float32 fast
Walsh-Hadamard transform of D = 2^m elements rounds every output m times, each
rounding bounded by 2^-24 times a partial sum of |inputs|, and the final scaling
by 1/sqrt(D) once more; a float32 RoPE pair rotation (two products and a sum)
adds at most 2^-23 (|x| + |y|) per element before the transform. Hence
    |v_gpu - v_exact| <= (m + 4) 2^-24 ||x||_1 / sqrt(D),
doubled for margin (BAND_MARGIN). ||x||_1 is the 1-norm of the row before any
rotation.

Each function returns, besides the verdict, the per-element value deltas of
the elements inside the band (the difference between the two candidate
dequantised values), so that a caller can widen a logit tolerance by exactly
what those elements can change: an indexer logit is 1-Lipschitz in each head's
dot product (ReLU), so |d logit_j| <= sum_h w_h (sum_d |dq_hd| |k_jd| +
sum_d |q_hd| |dk_jd| + sum_d |dq_hd| |dk_jd|).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import csa_oracle as O

BAND_MARGIN = 2.0
E2M1_MIDS = (O.E2M1_VALUES[:-1] + O.E2M1_VALUES[1:]) / 2


def rotation_error_bound(x_in: np.ndarray, D: int, rope: bool = False) -> np.ndarray:
    """Per-row absolute bound of the float32 evaluation error of the rotation
    (Hadamard over D, plus RoPE when `rope`) of rows x_in [..., D]."""
    m = int(round(math.log2(D)))
    l1 = np.abs(np.asarray(x_in, dtype=np.float64)).sum(axis=-1)
    return BAND_MARGIN * (m + (4 if rope else 2)) * 2.0 ** -24 * l1 / math.sqrt(D)


def exact_rotated(x_in, hadamard: bool, rope=None) -> np.ndarray:
    """The oracle's exact (float64) rotated rows, before rounding to float32."""
    x = np.asarray(x_in, dtype=np.float64)
    if rope is not None:
        cos, sin, rd = rope
        x = O.rope_rotate(x, cos, sin, rd)
    if hadamard:
        x = O.hadamard_rotate(x)
    return x


def _elem_err(err, shape):
    """An error bound per row [...] or per element [..., D] as [rows, D]."""
    e = np.asarray(err, dtype=np.float64)
    if e.ndim < len(shape):
        e = e[..., None]
    return np.broadcast_to(e, shape).reshape(-1, shape[-1])


def fp8_rows_match(gpu_codes, gpu_scale, x_exact, err):
    """GPU FP8 rows (codes [..., D], scales [...]) against the oracle's
    quantisation of the exact rows x_exact [..., D] with evaluation error bound
    err, per row [...] or per element [..., D].

    Scales: the GPU's amax is within err of the exact amax, so its scale is
    within err / 448 (plus two float32 roundings) of the oracle's.
    Codes: equal in value (+0 == -0), or adjacent codes whose midpoint lies
    within the band of the oracle's exact ratio v / scale; the band is err
    divided by the scale plus the ratio's own relative uncertainty.
    Returns (ok, message, delta) with delta [..., D] the dequantised value
    difference of every mismatching element (0 elsewhere)."""
    x = np.asarray(x_exact, dtype=np.float64)
    D = x.shape[-1]
    xs = x.reshape(-1, D)
    ee = _elem_err(err, x.shape)
    e = ee.max(axis=1)  # error bound of the row's amax
    gc = np.asarray(gpu_codes).reshape(-1, D)
    gs = np.asarray(gpu_scale, dtype=np.float64).reshape(-1)
    oc, osc = O.quant_fp8_rows(xs.astype(np.float32))
    osc = osc.astype(np.float64)
    amax = np.abs(xs).max(axis=1)
    tol_s = e / 448.0 + 2.0 ** -22 * osc
    bad_s = np.flatnonzero(np.abs(gs - osc) > tol_s)
    if len(bad_s):
        r = bad_s[0]
        return False, f"row {r}: scale {gs[r]!r} vs oracle {osc[r]!r} (tol {tol_s[r]:.3g})", None
    delta = np.zeros_like(xs)
    gv = O.E4M3_VALUES[gc]
    ov = O.E4M3_VALUES[oc]
    rows, cols = np.nonzero(gv != ov)
    fin = O.E4M3_VALUES[np.isfinite(O.E4M3_VALUES)]
    for r, c in zip(rows, cols):
        a, b = gv[r, c], ov[r, c]
        lo, hi = min(a, b), max(a, b)
        if np.any((fin > lo) & (fin < hi)):
            return False, f"row {r} elem {c}: codes {gc[r, c]:#x} vs {oc[r, c]:#x} not adjacent", None
        ratio = xs[r, c] / osc[r]
        rel = e[r] / max(amax[r], 1e-300) + 2.0 ** -21
        band = ee[r, c] / osc[r] + abs(ratio) * rel
        mid = (a + b) / 2
        if abs(ratio - mid) > band:
            return False, (f"row {r} elem {c}: codes {gc[r, c]:#x} vs {oc[r, c]:#x}, exact ratio "
                           f"{ratio!r} is {abs(ratio - mid):.3g} from the midpoint (band {band:.3g})"), None
        delta[r, c] = abs(a - b) * max(osc[r], gs[r])
    return True, f"{len(rows)} in-band code steps", delta.reshape(x.shape)


def _unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_rows_match(gpu_packed, gpu_sbytes, x_exact, err):
    """GPU MXFP4 rows (packed [..., D/2], e8m0 bytes [..., D/32]) against the
    oracle's quantisation of the exact rows x_exact [..., D] with per-row
    evaluation error bound err [...].

    Shared exponent: equal to the oracle's, or one off where the block's exact
    amax lies within err of the power of two between them (then the block is
    compared against the oracle's quantisation at the GPU's exponent, the other
    correct decision). Codes: equal in value (+0 == -0), or adjacent on the
    e2m1 grid with the exact scaled value within err / 2^X of the midpoint.
    Returns (ok, message, delta) with delta [..., D] the dequantised value
    difference an element may carry (0 where the codes cannot differ)."""
    x = np.asarray(x_exact, dtype=np.float64)
    D = x.shape[-1]
    xs = x.reshape(-1, D)
    nb = D // 32
    e = np.broadcast_to(np.asarray(err, dtype=np.float64), x.shape[:-1]).reshape(-1)
    gcode = _unpack(np.asarray(gpu_packed).reshape(-1, D // 2))
    gX = np.asarray(gpu_sbytes).reshape(-1, nb).astype(np.int64) - 127
    op, osb = O.quant_mxfp4_rows(xs.astype(np.float32))
    oX = osb.astype(np.int64) - 127
    delta = np.zeros_like(xs)
    n_steps = n_edges = 0
    for r in range(xs.shape[0]):
        for blk in range(nb):
            seg = xs[r, blk * 32:(blk + 1) * 32]
            amax = np.abs(seg).max()
            X = int(gX[r, blk])
            if X != oX[r, blk]:
                edge = 2.0 ** (max(X, oX[r, blk]) + 2)  # the power of two between the binades
                if abs(X - oX[r, blk]) != 1 or abs(amax - edge) > e[r]:
                    return False, f"row {r} block {blk}: exponent {X} vs oracle {oX[r, blk]}", None
                n_edges += 1
            elif abs(amax - 2.0 ** (X + 2)) <= e[r] or abs(amax - 2.0 ** (X + 3)) <= e[r]:
                n_edges += 1  # could have flipped: every element may carry a coarse step
                delta[r, blk * 32:(blk + 1) * 32] = 3.0 * 2.0 ** X
            scaled = seg / 2.0 ** X
            if X != oX[r, blk]:
                # the oracle's quantiser at the GPU's exponent: round scaled values on the grid
                mag = O._rne_to_grid(np.abs(scaled), O.E2M1_VALUES)
                ov = np.where(np.signbit(scaled), -O.E2M1_VALUES[mag], O.E2M1_VALUES[mag])
            else:
                oc = _unpack(op[r])[blk * 32:(blk + 1) * 32]
                ov = np.where(oc & 8, -O.E2M1_VALUES[oc & 7], O.E2M1_VALUES[oc & 7])
            gc = gcode[r, blk * 32:(blk + 1) * 32]
            gv = np.where(gc & 8, -O.E2M1_VALUES[gc & 7], O.E2M1_VALUES[gc & 7])
            for i in np.flatnonzero(gv != ov):
                a, b = gv[i], ov[i]
                ia = np.searchsorted(O.E2M1_VALUES, abs(a))
                ib = np.searchsorted(O.E2M1_VALUES, abs(b))
                same_side = (a >= 0) == (b >= 0) or a == 0 or b == 0
                if not same_side or abs(ia - ib) != 1:
                    return False, f"row {r} elem {blk * 32 + i}: e2m1 {a} vs {b} not adjacent", None
                mid = (abs(a) + abs(b)) / 2
                if abs(abs(scaled[i]) - mid) > e[r] / 2.0 ** X:
                    return False, (f"row {r} elem {blk * 32 + i}: e2m1 {a} vs {b}, exact "
                                   f"{scaled[i]!r} away from the midpoint {mid}"), None
                delta[r, blk * 32 + i] = max(delta[r, blk * 32 + i], abs(a - b) * 2.0 ** X)
                n_steps += 1
    return True, f"{n_steps} in-band code steps, {n_edges} exponent edges", delta.reshape(x.shape)


def fp8_band_delta(x_exact, err):
    """Without the GPU's codes: the dequantised value difference each element
    of FP8-quantised rows may carry, nonzero exactly where the exact ratio lies
    within the evaluation band of a rounding midpoint (as fp8_rows_match)."""
    x = np.asarray(x_exact, dtype=np.float64)
    D = x.shape[-1]
    xs = x.reshape(-1, D)
    ee = _elem_err(err, x.shape)
    e = ee.max(axis=1)
    _, osc = O.quant_fp8_rows(xs.astype(np.float32))
    osc = osc.astype(np.float64)
    amax = np.abs(xs).max(axis=1)
    ratio = np.abs(xs) / osc[:, None]
    band = ee / osc[:, None] + ratio * (e / np.maximum(amax, 1e-300) + 2.0 ** -21)[:, None]
    fin = O.E4M3_VALUES[:127]
    mids = (fin[:-1] + fin[1:]) / 2
    idx = np.clip(np.searchsorted(mids, ratio), 0, len(mids) - 1)
    near = np.zeros_like(ratio, dtype=bool)
    step = np.zeros_like(ratio)
    for k in (idx - 1, idx):
        kk = np.clip(k, 0, len(mids) - 1)
        hit = np.abs(ratio - mids[kk]) <= band
        near |= hit
        step = np.where(hit, np.maximum(step, fin[kk + 1] - fin[kk]), step)
    return (step * osc[:, None] * near).reshape(x.shape)


def mxfp4_band_delta(x_exact, err):
    """As fp8_band_delta for MXFP4 rows: an element near an e2m1 midpoint may
    carry one grid step; every element of a block whose amax is near a power of
    two (the shared exponent may flip) may carry 3 * 2^X."""
    x = np.asarray(x_exact, dtype=np.float64)
    D = x.shape[-1]
    xs = x.reshape(-1, D // 32, 32)
    e = np.broadcast_to(np.asarray(err, dtype=np.float64), x.shape[:-1]).reshape(-1)
    _, osb = O.quant_mxfp4_rows(x.reshape(-1, D).astype(np.float32))
    X = osb.astype(np.float64) - 127.0
    p2 = np.exp2(X)[..., None]
    scaled = np.abs(xs) / p2
    eb = (e[:, None] / np.exp2(X))[..., None]
    idx = np.clip(np.searchsorted(E2M1_MIDS, scaled), 0, len(E2M1_MIDS) - 1)
    step = np.zeros_like(scaled)
    for k in (idx - 1, idx):
        kk = np.clip(k, 0, len(E2M1_MIDS) - 1)
        hit = np.abs(scaled - E2M1_MIDS[kk]) <= eb
        st = O.E2M1_VALUES[kk + 1] - O.E2M1_VALUES[kk]
        step = np.where(hit, np.maximum(step, st), step)
    delta = step * p2
    amax = np.abs(xs).max(axis=-1)
    edge = (np.abs(amax - 4 * np.exp2(X)) <= e[:, None]) | (np.abs(amax - 8 * np.exp2(X)) <= e[:, None])
    delta = np.where(edge[..., None], np.maximum(delta, 3.0 * p2), delta)
    return delta.reshape(x.shape)


def band_delta(x_exact, err, fmt: str):
    if fmt == "fp8":
        return fp8_band_delta(x_exact, err)
    if fmt == "mxfp4":
        return mxfp4_band_delta(x_exact, err)
    return np.zeros_like(np.asarray(x_exact, dtype=np.float64))


def logit_slack(q_hat, dq, w, k_hat, dk):
    """Largest change of each logit of one query row when its dequantised query
    q_hat [H, D] moves by at most dq [H, D] per element and the index-K rows
    k_hat [n, D] by at most dk [n, D] (ReLU is 1-Lipschitz):
        sum_h w_h (|dq_h| . |k_j| + |q_h| . |dk_j| + |dq_h| . |dk_j|)."""
    aq, ak = np.abs(q_hat), np.abs(k_hat)
    dq = np.asarray(dq, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = np.zeros(k_hat.shape[0])
    if np.any(dq):
        out += (ak @ dq.T) @ w + (dk @ dq.T) @ w
    if np.any(dk):
        out += (dk @ aq.T) @ w
    return out


def bf16_match(gpu_bits, exact, err):
    """bf16 values of the GPU against the exact values `exact` (float64): equal
    bit patterns, or one ulp apart with the exact value within err (absolute,
    broadcastable) of the rounding midpoint between them (+0 == -0)."""
    g = np.asarray(gpu_bits, dtype=np.uint16).ravel()
    x = np.asarray(exact, dtype=np.float64).ravel()
    e = np.broadcast_to(np.asarray(err, dtype=np.float64), np.asarray(exact).shape).ravel()
    o = O.bf16_bits(x.astype(np.float32))
    gv, ov = O.bf16_decode(g), O.bf16_decode(o)
    bad = np.flatnonzero(gv != ov)
    for i in bad:
        a, b = gv[i], ov[i]
        if (g[i] >> 15) != (o[i] >> 15) or abs(int(g[i]) - int(o[i])) != 1:
            return False, f"elem {i}: bf16 {g[i]:#06x} vs {o[i]:#06x} more than one ulp apart"
        if abs(x[i] - (a + b) / 2) > e[i] + 2.0 ** -24 * abs(x[i]):
            return False, f"elem {i}: bf16 {g[i]:#06x} vs {o[i]:#06x} with the exact value off the midpoint"
    return True, f"{len(bad)} in-band ulps"


def compress_error_bound(x_block, gate_w, depth: int = 64) -> np.ndarray:
    """Absolute bound of the float32 evaluation error of a softmax-gated pooled
    entry c = sum_i a_i x_i, a = softmax(w . x_i + b_i), per output dim.
    x_block [R, 576] (the block's rows), gate_w [576].

    Each gate is a 576-term float32 dot product. Summed in any order whose
    longest chain of roundings is at most `depth` (a tree, or per-lane partial
    sums of up to a few dozen terms combined by a tree, as a wavefront sums
    it), its error is <= gamma_depth sum_d |w_d x_id| with
    gamma_n = n 2^-24 / (1 - n 2^-24); exp, the softmax
    normalisation and the weighted sum add a few roundings. A gate error of
    dg changes each a_i by at most a_i (e^(2 dg) - 1) ~ 2 dg a_i, so
    |dc_d| <= 2 dg max_i |x_id| + (R + 4) 2^-24 sum_i a_i |x_id|; bounded here
    with max_i |x_id| for the second sum, and doubled (BAND_MARGIN)."""
    x = np.asarray(x_block, dtype=np.float64)
    w = np.asarray(gate_w, dtype=np.float64)
    gamma = depth * 2.0 ** -24 / (1 - depth * 2.0 ** -24)
    dg = gamma * (np.abs(x) * np.abs(w)[None, :]).sum(axis=1).max() + 8 * 2.0 ** -24
    xmax = np.abs(x).max(axis=0)
    return BAND_MARGIN * (2 * dg * xmax + (x.shape[0] + 4) * 2.0 ** -24 * xmax)
