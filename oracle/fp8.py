"""Float64 CPU oracle for the fp8 forward with a bounded rebase of the running max.

TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and nothing here
is shared with the GPU library.

Source: FlyDSL PR #1033, "[Bugfix][Kernel] Fix NaN from the lazy rescale on a wide score
range", section "The fp8 helper, second commit". That section describes an fp8 forward
whose softmax helper differs from the bf16 one in three ways, which this module follows
step by step (it is an algorithm with quantised intermediates, not a closed form, so the
oracle walks the key tiles in order):

* the rescale test is applied to scores already multiplied by the logit scale, so the
  threshold (8, log2 units) is measured on the scaled scores;
* when the wave-wide test fires, a row does not keep max(m_row, m_tile): it is rebased
  onto its own tile max even when that is lower than the running max, which keeps the
  exponentials of the current tile near 1 where fp8 resolves them best;
* the fix caps how far the base may fall at 16 (log2 units), so the factor applied to the
  row's accumulators is at most 2**16. Without the cap a row dragged along by another
  row's rise multiplies its sums by 2**(m_row - m_tile), which overflows on a wide score
  range (the NaN the section reports).

Readings where the section is silent (each is listed in the design notes):

* inputs are OCP fp8 e4m3 (4 exponent bits, bias 7, 3 mantissa bits, largest finite 448)
  with one float descale per tensor; the logit scale is scale * q_descale * k_descale
  * log2(e), and v_descale multiplies the normalised output;
* the exponentials p are rounded to e4m3 (nearest, ties to even) before the P.V product,
  while the row sum l adds the unrounded p, as the bf16 path sums p before its bf16
  rounding; hence lse is exact and only out carries the fp8 rounding of P;
* the wave-wide test covers `group_rows` consecutive query rows (32 on the GPU: one row
  per lane pair of a 64-wide wave), the key tile is `block_n` keys (64 on the GPU);
* a row with no visible key so far keeps m = -inf, its factor is taken as 1 (its sums are
  zero), and lse = (m + log2 l) * ln 2 is the natural-log LSE of the bf16 path;
* the cap is measured from the row's running max M (the largest visible scaled score seen
  so far): a rebase sets the base to max(m_tile, M - 16). Then the base never sits more
  than 16 below M, and the sums never exceed 2**16 times their max-based values. Capping
  each rebase against the previous base instead lets drops compound when other rows keep
  firing (eight capped drops already exceed the fp32 range); the two readings agree
  whenever a row's base never falls more than 16 below its running max.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["E4M3_MAX", "round_e4m3", "fp8_forward"]

E4M3_MAX = 448.0
_LOG2E = 1.0 / math.log(2.0)
_LN2 = math.log(2.0)


def round_e4m3(x):
    """Nearest OCP e4m3 value of each element of x (ties to even), in float64.

    Normal binades [2^e, 2^(e+1)) for e >= -6 hold 8 values spaced 2^(e-3); below 2^-6 the
    subnormals are spaced 2^-9. Magnitudes above 448 are out of range and rejected (the
    fp8 forward never produces them: every exponential is at most 2^8).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the e4m3 range")
    _, e = np.frexp(a)                      # a = m * 2^e with 0.5 <= m < 1, so floor(log2 a) = e - 1
    quantum = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.copysign(np.round(a / quantum) * quantum, x)   # np.round: half to even


def fp8_forward(q8, k8, v8, q_descale, k_descale, v_descale, *, causal=False, scale=None,
                block_n=64, group_rows=32, tau=8.0, bound=16.0, quantize_p=True,
                return_stats=False, units=None, row_groups=None, cap_from="running_max"):
    """fp8 attention forward, tile by tile as the FlyDSL fp8 helper does (see module doc).

    q8 [B, Sq, H, D], k8 / v8 [B, Sk, Hkv, D]: float arrays holding e4m3 values (decoded,
    without their descales). Returns out [B, Sq, H, D] and lse [B, H, Sq] in float64.
    ``bound=None`` rebases onto the tile max without a cap (the behaviour before the fix);
    ``quantize_p=False`` skips the e4m3 rounding of P (then the result is the exact
    attention of the dequantised inputs, whatever the rebase sequence).
    ``cap_from`` picks the reading of the cap: "running_max" (the default) bounds the base
    at `bound` below the row's running max; "previous_base" bounds each rebase at `bound`
    below the base it replaces, so successive drops can add up.
    With ``return_stats`` a dict counts triggered tiles and rebases that lowered a base,
    and those the cap limited. ``units`` (a list of (b, h)) and ``row_groups`` (indices of
    groups of ``group_rows`` rows) restrict the work; entries left out are NaN. A group's
    rows share every decision, so a group is computed whole or not at all.
    """
    if cap_from not in ("running_max", "previous_base"):
        raise ValueError(cap_from)
    q8, k8, v8 = (np.asarray(t, dtype=np.float64) for t in (q8, k8, v8))
    B, Sq, H, D = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    c2 = scale * q_descale * k_descale * _LOG2E          # logit scale, log2 units
    subset = units is not None or row_groups is not None
    out = np.full((B, Sq, H, D), np.nan if subset else 0.0)
    lse = np.full((B, H, Sq), np.nan if subset else -np.inf)
    stats = {"triggers": 0, "lowered": 0, "capped": 0}
    if row_groups is None:
        rows = np.arange(Sq)
    else:
        rows = np.concatenate([np.arange(gi * group_rows, min((gi + 1) * group_rows, Sq))
                               for gi in row_groups])
    n = rows.size
    group = np.unique(rows // group_rows, return_inverse=True)[1].reshape(-1)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        g = h // (H // Hkv)
        s2 = (q8[b, rows, h, :] @ k8[b, :, g, :].T) * c2       # [n, Sk]
        m = np.full(n, -np.inf)        # base of the exponentials
        m_max = np.full(n, -np.inf)    # running max of the visible scaled scores
        l = np.zeros(n)
        acc = np.zeros((n, D))
        for j0 in range(0, Sk, block_n):
            cols = np.arange(j0, min(j0 + block_n, Sk))
            vis = np.ones((n, cols.size), dtype=bool)
            if causal:
                vis &= cols[None, :] <= rows[:, None]
            st = np.where(vis, s2[:, cols], -np.inf)
            m_tile = st.max(axis=1)
            m_max = np.maximum(m_max, m_tile)
            # 1. rescale test per row (a row with m = -inf and a visible key fires:
            #    +inf > tau), then made common to each group of rows
            with np.errstate(invalid="ignore"):
                fire_row = (m_tile - m) > tau
            fire_grp = np.zeros(group.max() + 1, dtype=bool)
            np.logical_or.at(fire_grp, group, fire_row)
            fire = fire_grp[group]
            # 2. rebase: onto the row's tile max, never more than `bound` below its
            #    running max (or below its previous base)
            if fire.any():
                stats["triggers"] += int(fire_grp.sum())
                if bound is None:
                    m_new = m_tile
                    floor = np.full(n, -np.inf)
                elif cap_from == "running_max":
                    floor = m_max - bound
                else:
                    floor = np.where(m == -np.inf, -np.inf, m - bound)
                m_new = np.maximum(m_tile, floor)
                stats["lowered"] += int(np.sum(fire & (m_new < m)))
                stats["capped"] += int(np.sum(fire & (m_tile < floor)))
                with np.errstate(over="ignore", invalid="ignore"):
                    corr = np.where(m == -np.inf, 1.0, np.exp2(m - m_new))
                corr = np.where(fire, corr, 1.0)
                with np.errstate(over="ignore", invalid="ignore"):
                    l = l * corr
                    acc = acc * corr[:, None]
                m = np.where(fire, m_new, m)
            # 3. exponentials against the (possibly stale) base, row sum of unrounded p
            m_use = np.where(m == -np.inf, 0.0, m)
            with np.errstate(over="ignore", invalid="ignore"):
                p = np.where(vis, np.exp2(st - m_use[:, None]), 0.0)
            l = l + p.sum(axis=1)
            # 4. P rounded to e4m3, then P . V with the raw fp8 values of V
            pq = round_e4m3(p) if quantize_p else p
            with np.errstate(over="ignore", invalid="ignore"):
                acc = acc + pq @ v8[b, cols, g, :]
        m_use = np.where(m == -np.inf, 0.0, m)
        ok = l != 0                    # NaN sums propagate
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            out[b, rows, h, :] = np.where(ok[:, None], acc * v_descale / np.where(ok, l, 1.0)[:, None], 0.0)
            lse[b, h, rows] = np.where(ok, (m_use + np.log2(np.where(ok, l, 1.0))) * _LN2, -np.inf)
    if return_stats:
        return out, lse, stats
    return out, lse
