"""Parity rules between the HIP path and the float64 oracle.

The rules make the quantiser's parity operational (readings of "bit-exact
codes except at elements within 1e-6 relative of a rounding boundary"):

P1  fp16 scale/zero: equal bit for bit, except groups whose float64 value
    before fp16 rounding lies within 1e-6 relative of an fp16 rounding
    midpoint ("boundary groups").
P2  codes: equal to the oracle's codes of the float64 rotated value on the
    GPU's own stored grid, except elements whose float64 value lies within
    1e-6 * max(|b|, s16) of a code boundary b = z16 + (j + 1/2) s16; the
    exempt count must be <= 1e-5 of all elements.  Values encoded as given
    (the value rotation folded into the caller's weights) keep the 8
    significant bits of bfloat16, so many of them sit exactly on a boundary
    of the fp16 grid.  There (x - z16) / s16 is exactly j + 1/2 in float32 as
    in float64 (the difference has at most 13 significant bits, so the
    float32 subtraction is exact, and the quotient is correctly rounded), so
    such exact ties must take the round-half-even code: zero mismatches.
    Exact ties are counted and printed; the rest of the exempt band counts
    toward the 1e-5 bound.
    The bound is a rate: every check adds its counts to a tally, a sample of
    at least GATE_MIN_ELEMENTS elements is held to it on its own, and the
    tally over a whole test module at its end.  Raw agreement with the
    oracle's codes on the oracle's own scale/zero is reported beside it.
P3  bytes: the cache is read back through the oracle's layout functions; bytes
    of slots that were not written keep their previous contents.
P4  attention: the oracle decodes the GPU's own cache in float64; the max over
    (sequence, query head) of ||o - o_ref||_inf / ||o_ref||_inf is <= 2e-3.
"""
from __future__ import annotations

import numpy as np

import oracle as O

REL = 1e-6
EXEMPT_FRACTION = 1e-5
ATTN_TOL = 2e-3


def fp16_midpoint_distance(raw):
    """Relative distance of float64 values to the nearest fp16 rounding midpoint."""
    raw = np.asarray(raw, np.float64)
    r16 = O.fp16_sat(raw)
    # neighbours of r16 in fp16
    up = np.nextafter(r16.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(r16.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mid = np.where(raw >= r16, (r16 + up) / 2, (r16 + dn) / 2)
    scale = np.maximum(np.abs(mid), np.finfo(np.float16).smallest_subnormal)
    return np.abs(raw - mid) / scale


def check_scale_zero(gpu_s, gpu_z, ref_s, ref_z, raw_s, raw_z):
    """P1.  Returns (mismatches outside boundary groups, boundary groups)."""
    ms = gpu_s != ref_s
    mz = gpu_z != ref_z
    bs = fp16_midpoint_distance(raw_s) <= REL
    bz = fp16_midpoint_distance(raw_z) <= REL
    bad = (ms & ~bs) | (mz & ~bz)
    boundary = (ms & bs) | (mz & bz)
    return int(bad.sum()), int(boundary.sum())


GATE_MIN_ELEMENTS = 1_000_000
# exempt: elements in the exempt band (exact ties of values encoded as given
# excluded); elements: all compared; ties / tie_bad: exact ties of values
# encoded as given and those whose code differs; raw_bad: codes differing from
# the oracle's codes on the oracle's own scale/zero
TALLY = dict(exempt=0, elements=0, ties=0, tie_bad=0, raw_bad=0)


def tally_reset():
    for k in TALLY:
        TALLY[k] = 0


def code_parity(gpu_codes, x, gpu_s, gpu_z, group, oracle_codes=None, given=False):
    """P2 in full for one (token range, head, K or V): asserts no mismatch
    outside the exempt band and, for values encoded as given (`given`), none
    at an exact tie; returns the counts (also added to TALLY)."""
    ref = O.quantize_on_grid(x, gpu_s, gpu_z, group)
    d = x.shape[-1]
    G = d // group
    xg = np.asarray(x, np.float64).reshape(x.shape[:-1] + (G, group))
    s = np.asarray(gpu_s, np.float64)[..., None]
    z = np.asarray(gpu_z, np.float64)[..., None]
    near = np.zeros(xg.shape, bool)
    tie = np.zeros(xg.shape, bool)
    for j in range(3):
        bnd = z + (j + 0.5) * s
        near |= (np.abs(xg - bnd) <= REL * np.maximum(np.abs(bnd), s)) & (s > 0)
        tie |= (xg == bnd) & (s > 0)
    near = near.reshape(x.shape)
    tie = tie.reshape(x.shape)
    got = np.asarray(gpu_codes)
    mismatch = got != ref
    bad = int((mismatch & ~near).sum())
    assert bad == 0, f"{bad} code mismatches outside the exempt band"
    res = dict(elements=int(mismatch.size), ties=0, tie_bad=0)
    if given:
        res["ties"] = int(tie.sum())
        res["tie_bad"] = int((mismatch & tie).sum())
        assert res["tie_bad"] == 0, f"{res['tie_bad']} exact ties not rounded half to even"
        res["exempt"] = int((near & ~tie).sum())
    else:
        res["exempt"] = int(near.sum())
    res["raw_bad"] = int((got != np.asarray(oracle_codes)).sum()) if oracle_codes is not None else 0
    for k in TALLY:
        TALLY[k] += res[k]
    return res


def gate_exempt(exempt: int, elements: int, label: str = "") -> None:
    """Print a check's exempt count; hold it to the 1e-5 rate when the sample
    is large enough for a rate to mean something."""
    print(f"  {label}elements {elements}  exempt {exempt}  "
          f"({exempt / max(elements, 1):.2e}; bound {EXEMPT_FRACTION:.0e})", flush=True)
    if elements >= GATE_MIN_ELEMENTS:
        assert exempt <= EXEMPT_FRACTION * elements


def check_codes(gpu_codes, x, gpu_s, gpu_z, group, with_exempt_mismatches=False):
    """P2.  Returns (mismatches outside exemptions, exempt elements, elements)
    and, with with_exempt_mismatches, the exempt elements whose code differs."""
    ref = O.quantize_on_grid(x, gpu_s, gpu_z, group)
    d = x.shape[-1]
    G = d // group
    xg = np.asarray(x, np.float64).reshape(x.shape[:-1] + (G, group))
    s = np.asarray(gpu_s, np.float64)[..., None]
    z = np.asarray(gpu_z, np.float64)[..., None]
    near = np.zeros(xg.shape, bool)
    for j in range(3):
        bnd = z + (j + 0.5) * s
        near |= (np.abs(xg - bnd) <= REL * np.maximum(np.abs(bnd), s)) & (s > 0)
    near = near.reshape(x.shape)
    mismatch = np.asarray(gpu_codes) != ref
    res = (int((mismatch & ~near).sum()), int(near.sum()), int(mismatch.size))
    if with_exempt_mismatches:
        return res + (int((mismatch & near).sum()),)
    return res


def attention_error(o_gpu, o_ref):
    """P4 metric: max over rows of ||o - o_ref||_inf / ||o_ref||_inf."""
    o_gpu = np.asarray(o_gpu, np.float64).reshape(-1, o_gpu.shape[-1])
    o_ref = np.asarray(o_ref, np.float64).reshape(-1, o_ref.shape[-1])
    den = np.abs(o_ref).max(-1)
    num = np.abs(o_gpu - o_ref).max(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(rel.max()) if rel.size else 0.0
