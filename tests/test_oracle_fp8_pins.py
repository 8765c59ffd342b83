"""Pins of the fp8-forward oracle (oracle/fp8.py) to things other than itself.

* Its e4m3 rounding against torch's float8_e4m3fn conversion (a library routine).
* With the rounding of P switched off, the tile walk with its rebases must reproduce the
  exact attention of the dequantised inputs (the float64 definition, itself pinned in
  test_oracle_pins.py), whatever rebases happen; this checks every rescale factor.
* lse never sees the rounding of P, so it equals the exact lse with the rounding on.
* Closed form: q = 0 gives p = 1 exactly, hence out = the mean of the visible values.
* The cap (FlyDSL PR #1033, "The fp8 helper, second commit"): a constructed case where an
  uncapped rebase overflows and the capped one stays finite, and ordinary inputs where the
  cap never acts and the two agree bit for bit (the section's claim that a cap of 16 leaves
  working ranges unchanged).
* With V = ones the output stays near 1 (the section's V = ones measurements).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import fp8_forward, round_e4m3
from exact_attention_40_amd import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _codes():
    """Every finite e4m3 value (decoded by torch)."""
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.unique(b[np.isfinite(b)])


def test_round_e4m3_matches_torch():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-12, math.log2(440.0), 20000))
    x = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    vals = _codes()
    pos = vals[vals >= 0]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)        # ties: exactly halfway
    x = np.concatenate([x, mids, -mids, vals.astype(np.float32), np.float32([0.0, 1e-9, 448.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = round_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_e4m3_fixed_points_and_range():
    v = _codes()
    assert np.array_equal(round_e4m3(v), v)
    assert v.max() == 448.0 and v.size == 253        # 254 finite codes; +0 and -0 compare equal
    with pytest.raises(ValueError):
        round_e4m3(np.array([449.0]))


def _dequant(p):
    q, k, v = p.decoded()
    return q * p.q_descale, k * p.k_descale, v * p.v_descale


CASES = [
    # B, Sq, Sk, H, Hkv, D, causal, k_mult, block_n, group_rows
    (1, 70, 150, 2, 1, 16, False, 1.0, 64, 32),
    (2, 45, 45, 2, 2, 16, True, 1.0, 16, 32),
    (1, 64, 200, 4, 2, 32, False, 40.0, 32, 8),      # wide: rebases that lower the base
    (1, 50, 50, 2, 1, 16, True, 300.0, 16, 32),      # very wide: the cap acts
]


@pytest.mark.parametrize("case", CASES)
def test_unrounded_walk_is_exact_attention(case):
    B, Sq, Sk, H, Hkv, D, causal, km, bn, gr = case
    p = workloads.fp8_dense(B, Sq, Sk, H, Hkv, D, seed=31, causal=causal, k_mult=km)
    q, k, v = p.decoded()
    out, lse, st = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, causal=causal,
                               block_n=bn, group_rows=gr, quantize_p=False, return_stats=True)
    eo, el = oracle.attention_forward(*_dequant(p), causal=causal)
    assert _rel(out, eo) < 1e-12
    assert np.max(np.abs(lse - el)) < 1e-10
    if km >= 40:
        assert st["lowered"] > 0          # the walk really rebased downwards
    if km >= 300:
        assert st["capped"] > 0           # ... and the cap engaged


@pytest.mark.parametrize("case", CASES)
def test_lse_is_exact_with_rounding(case):
    B, Sq, Sk, H, Hkv, D, causal, km, bn, gr = case
    p = workloads.fp8_dense(B, Sq, Sk, H, Hkv, D, seed=32, causal=causal, k_mult=km)
    q, k, v = p.decoded()
    out, lse = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, causal=causal,
                           block_n=bn, group_rows=gr)
    eo, el = oracle.attention_forward(*_dequant(p), causal=causal)
    assert np.max(np.abs(lse - el)) < 1e-10
    # out differs from the exact result only by the e4m3 rounding of P (3 mantissa bits:
    # at most 1/16 relative per element)
    err = _rel(out, eo)
    assert err < 0.07
    if km == 1.0:
        assert err > 1e-3                 # the rounding did happen


def test_zero_query_gives_mean_of_values():
    p = workloads.fp8_dense(1, 40, 90, 2, 1, 16, seed=33, causal=True)
    q, k, v = p.decoded()
    q[:] = 0.0
    out, lse = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, causal=True, block_n=32)
    vd = v * p.v_descale
    for i in range(40):
        for h in range(2):
            assert np.allclose(out[0, i, h], vd[0, :i + 1, 0].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[0, h, i] - math.log(i + 1)) < 1e-13


def test_uncapped_rebase_overflows_capped_does_not():
    # Two rows share one rescale decision. Row 0's scores rise by 100 (log2 units) per key
    # tile, so it fires on every tile; row 1 peaks in tile 0 and then falls 3000 below.
    # Uncapped, row 1 is rebased onto that low tile max and its sums are multiplied by
    # 2^3000 (inf); capped, its base stays within 16 of its running max (0).
    D, n = 4, 4
    ntile = 3
    Sk = n * ntile
    s_target = np.zeros((2, Sk))
    for t in range(ntile):
        s_target[0, t * n:(t + 1) * n] = 100.0 * t
        s_target[1, t * n:(t + 1) * n] = 0.0 if t == 0 else -3000.0
    # realise the scores as q . k with an identity-like construction: q = e_row, k = s
    q = np.zeros((1, 2, 1, D)); q[0, 0, 0, 0] = 1.0; q[0, 1, 0, 1] = 1.0
    k = np.zeros((1, Sk, 1, D)); k[0, :, 0, 0] = s_target[0]; k[0, :, 0, 1] = s_target[1]
    v = np.ones((1, Sk, 1, D))
    c = math.sqrt(D) * math.log(2.0)   # scale 1/sqrt(D) times log2(e) times c is exactly 1
    kw = dict(block_n=n, group_rows=2, quantize_p=False)
    with np.errstate(all="ignore"):
        o_free, _ = fp8_forward(q, k, v, 1.0, c, 1.0, bound=None, **kw)
    o_cap, l_cap, st = fp8_forward(q, k, v, 1.0, c, 1.0, bound=16.0, return_stats=True, **kw)
    assert not np.all(np.isfinite(o_free[0, 1]))
    assert np.all(np.isfinite(o_cap)) and st["capped"] == 2 and st["lowered"] == 1
    assert np.allclose(o_cap, 1.0, rtol=0, atol=1e-12)      # V = ones: out = 1 exactly
    assert abs(l_cap[0, 0, 1] - (math.log(n) + 0.0)) < 1e-9  # row 1: lse = ln(4 e^0 + tiny)


@pytest.mark.parametrize("k_mult", [1.0, 2.0])
def test_cap_is_inactive_on_ordinary_ranges(k_mult):
    p = workloads.fp8_dense(1, 96, 300, 2, 1, 32, seed=34, k_mult=k_mult)
    q, k, v = p.decoded()
    a = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, bound=16.0, return_stats=True)
    b = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, bound=None)
    assert a[2]["capped"] == 0 and a[2]["triggers"] > 0
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("k_mult", [1.0, 100.0])
def test_value_ones_output_near_one(k_mult):
    p = workloads.fp8_dense(1, 128, 1024, 2, 1, 32, seed=35, k_mult=k_mult, v_ones=True)
    q, k, v = p.decoded()
    out, _ = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale)
    assert np.all(np.isfinite(out))
    assert np.mean(np.abs(out - 1.0)) < 5e-3


def test_subsets_match_the_whole():
    p = workloads.fp8_dense(2, 100, 130, 2, 1, 16, seed=36, causal=True, k_mult=20.0)
    q, k, v = p.decoded()
    kw = dict(causal=True, block_n=32, group_rows=32)
    out, lse = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, **kw)
    so, sl = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, units=[(1, 0)],
                         row_groups=[0, 3], **kw)
    rows = np.r_[0:32, 96:100]
    assert np.array_equal(so[1, rows, 0], out[1, rows, 0])
    assert np.array_equal(sl[1, 0, rows], lse[1, 0, rows])
    assert np.all(np.isnan(so[0])) and np.all(np.isnan(so[1, 32:96, 0]))


def test_cap_bounds_the_base_below_the_running_max():
    """Rows firing in turn must not drag a quiet row's base ever lower: with one row rising
    on every tile and the other far below its own max, the quiet row's base falls once, by
    16, and its sums stay within 2^16 of their max-based values (finite in fp32 terms)."""
    D, n, ntile = 4, 4, 40
    Sk = n * ntile
    q = np.zeros((1, 2, 1, D)); q[0, 0, 0, 0] = 1.0; q[0, 1, 0, 1] = 1.0
    k = np.zeros((1, Sk, 1, D))
    for t in range(ntile):
        k[0, t * n:(t + 1) * n, 0, 0] = 20.0 * t           # row 0 fires on every tile
        k[0, t * n:(t + 1) * n, 0, 1] = 0.0 if t == 0 else -500.0
    c = math.sqrt(D) * math.log(2.0)
    out, lse, st = fp8_forward(q, k, np.ones((1, Sk, 1, D)), 1.0, c, 1.0, block_n=n,
                               group_rows=2, quantize_p=False, return_stats=True)
    assert st["triggers"] == ntile and st["lowered"] == 1
    assert np.allclose(out, 1.0, rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 1] - math.log(n)) < 1e-9


def test_page_fp8_table_wide_range_v_ones():
    """FlyDSL PR #1033, "The fp8 helper, second commit" (tests/golden/page_values.json,
    fp8_bound_table): with V = ones and K scaled by 5000 or 20000 the uncapped rebase
    produced NaN while a bound of 16 kept every output finite with mean |o - 1| at most a
    few 1e-3. The same holds for the oracle (on fewer keys than the page's 12288)."""
    g = GOLDEN["fp8_bound_table"]
    worst = max(x for x in g["bound_16_mean_abs_o_minus_1"] if x is not None)
    for km in g["k_scale"]:
        p = workloads.fp8_dense(1, 64, 2048, 2, 1, 32, seed=37, k_mult=float(km), v_ones=True)
        q, k, v = p.decoded()
        out, _ = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale)
        assert np.all(np.isfinite(out))
        assert np.mean(np.abs(out - 1.0)) <= 5 * worst
        if km >= 5000:
            with np.errstate(all="ignore"):
                free, _ = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, bound=None)
            assert not np.all(np.isfinite(free))


def test_cap_reading_pinned_by_page_table():
    """Which base the cap of 16 is measured from. FlyDSL PR #1033, "The fp8 helper, second
    commit" (tests/golden/page_values.json, fp8_bound_table) reports zero NaN elements with
    bound 16 at K x 1000, 5000 and 20000, V = ones, S = 12288. On that workload (four
    32-row decision groups, 12288 keys) the cap measured from the row's running max keeps
    every output finite, while a cap measured from the previous base lets the drops of
    successive rebases add up and overflows; so the page's table rules out the second
    reading."""
    g = GOLDEN["fp8_bound_table"]
    assert g["bound_16_nan_elements"] == [0, 0, 0]
    for km in g["k_scale"]:
        p = workloads.fp8_dense(1, 128, 12288, 2, 1, 128, seed=37, k_mult=float(km), v_ones=True)
        q, k, v = p.decoded()
        out, _ = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale, cap_from="running_max")
        assert np.all(np.isfinite(out)), km
        with np.errstate(all="ignore"):
            prev, _ = fp8_forward(q, k, v, p.q_descale, p.k_descale, p.v_descale,
                                  cap_from="previous_base")
        assert not np.all(np.isfinite(prev)), km
