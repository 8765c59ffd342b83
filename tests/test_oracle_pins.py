"""Pins of the float64 oracle to things other than itself.

Each test ties the oracle to an independent source: torch's float64 CPU attention (a
library implementation), 50-digit mpmath evaluation of the definition with no max
subtraction, central finite differences of the forward, closed forms, invariants of the
mathematics, and values printed on the pages (tests/golden/page_values.json).
"""

import itertools
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from exact_attention_40_amd import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------------------------------------------
# 1. torch float64 CPU attention (library cross-check)
# ------------------------------------------------------------------------------------------

def _torch_ref(q, k, v, dout, causal, scale, mask=None, kind="none"):
    """out, lse, dq, dk, dv from torch on the CPU in float64 (BSHD in, BSHD out)."""
    H, Hkv = q.shape[2], k.shape[2]
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_(True)
    kk = tk.repeat_interleave(H // Hkv, dim=1)
    vv = tv.repeat_interleave(H // Hkv, dim=1)
    am = None
    if kind == "bool":
        am = torch.tensor(mask)
    elif kind == "additive":
        am = torch.tensor(mask, dtype=torch.float64)
    out = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=am,
                                                           is_causal=causal, scale=scale)
    # LSE from the library logsumexp over the same masked scores
    s = scale * tq.detach() @ kk.detach().transpose(-1, -2)
    Sq, Sk = s.shape[-2:]
    if causal:
        s = s.masked_fill(~torch.ones(Sq, Sk, dtype=torch.bool).tril(), -math.inf)
    if kind == "bool":
        s = s.masked_fill(~am, -math.inf)
    elif kind == "additive":
        s = s + am
    lse = torch.logsumexp(s, dim=-1)
    out.backward(torch.tensor(dout).permute(0, 2, 1, 3))
    bshd = lambda t: t.permute(0, 2, 1, 3).detach().numpy()  # noqa: E731
    return bshd(out), lse.detach().numpy(), bshd(tq.grad), bshd(tk.grad), bshd(tv.grad)


@pytest.mark.parametrize("case", [
    dict(B=2, Sq=13, Sk=13, H=2, Hkv=2, D=16, causal=False, kind="none"),
    dict(B=1, Sq=17, Sk=17, H=2, Hkv=2, D=8, causal=True, kind="none"),
    dict(B=2, Sq=9, Sk=21, H=4, Hkv=2, D=8, causal=False, kind="bool"),
    dict(B=1, Sq=11, Sk=7, H=2, Hkv=1, D=8, causal=True, kind="none"),   # top-left causal, Sq != Sk
    dict(B=2, Sq=6, Sk=10, H=2, Hkv=2, D=4, causal=False, kind="additive"),
    dict(B=1, Sq=8, Sk=8, H=4, Hkv=1, D=8, causal=True, kind="bool"),
])
def test_matches_torch_float64(case):
    rng = np.random.default_rng(7)
    B, Sq, Sk, H, Hkv, D = (case[x] for x in ("B", "Sq", "Sk", "H", "Hkv", "D"))
    q, k, v = _rand(rng, B, Sq, H, D), _rand(rng, B, Sk, Hkv, D), _rand(rng, B, Sk, Hkv, D)
    dout = _rand(rng, B, Sq, H, D)
    scale = 0.37
    mask = None
    if case["kind"] == "bool":
        mask = rng.random((B, H, Sq, Sk)) > 0.3
        mask[..., 0] = True  # keep every row non-empty (torch's empty-row convention differs)
    elif case["kind"] == "additive":
        mask = rng.standard_normal((B, 1, Sq, Sk))
        mask[rng.random(mask.shape) < 0.3] = -np.inf
        mask[..., 0] = 0.5
    ref = _torch_ref(q, k, v, dout, case["causal"], scale, mask, case["kind"])
    out, lse = oracle.attention_forward(q, k, v, causal=case["causal"], scale=scale,
                                        mask=mask, mask_kind=case["kind"])
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=case["causal"], scale=scale,
                                           mask=mask, mask_kind=case["kind"])
    for mine, theirs in zip((out, lse, dq, dk, dv), ref):
        np.testing.assert_allclose(mine, theirs, rtol=1e-11, atol=1e-12)


def test_lse_matches_torch_cpu_flash_lse():
    """torch's CPU flash kernel returns its own logsumexp: natural-log units."""
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 1, 2, 33, 16) for _ in range(3))  # BHSD for the aten op
    out_t, lse_t = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), 0.0, True, scale=0.25)[:2]
    bshd = lambda a: np.transpose(a, (0, 2, 1, 3))  # noqa: E731
    out, lse = oracle.attention_forward(bshd(q), bshd(k), bshd(v), causal=True, scale=0.25)
    np.testing.assert_allclose(lse, lse_t.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out, bshd(out_t.numpy()), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------------------------------
# 2. brute force in 50-digit arithmetic, no max subtraction, every bool mask of a 2x3 tile
# ------------------------------------------------------------------------------------------

def _mp_forward(q, k, v, scale, vis):
    mpmath.mp.dps = 50
    sq, sk, d = q.shape[0], k.shape[0], v.shape[1]
    out = np.zeros((sq, d))
    lse = np.zeros(sq)
    for i in range(sq):
        terms = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, t]) * mpmath.mpf(k[j, t])
                                                           for t in range(q.shape[1])))
                 if vis[i, j] else mpmath.mpf(0) for j in range(sk)]
        z = mpmath.fsum(terms)
        if z == 0:
            lse[i] = -np.inf
            continue
        lse[i] = float(mpmath.log(z))
        for t in range(d):
            out[i, t] = float(mpmath.fsum(terms[j] * mpmath.mpf(v[j, t]) for j in range(sk)) / z)
    return out, lse


def test_every_mask_of_a_2x3_tile_against_mpmath():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 3), _rand(rng, 3, 3), _rand(rng, 3, 2)
    scale = 0.9
    n = 0
    for causal in (False, True):
        for bits in itertools.product((False, True), repeat=6):
            keep = np.array(bits).reshape(2, 3)
            vis = oracle.visibility(2, 3, causal, keep)
            out, lse, P = oracle.unit_forward(q, k, v, scale, vis)
            mo, ml = _mp_forward(q, k, v, scale, vis)
            np.testing.assert_allclose(out, mo, rtol=1e-14, atol=1e-15)
            assert np.array_equal(np.isneginf(lse), np.isneginf(ml))
            fin = np.isfinite(ml)
            np.testing.assert_allclose(lse[fin], ml[fin], rtol=1e-14, atol=1e-15)
            # empty rows: out = 0, lse = -inf, P row = 0 (reading of "defined output")
            empty = ~vis.any(axis=1)
            assert np.all(out[empty] == 0) and np.all(P[empty] == 0)
            n += 1
    assert n == 128


def test_random_small_against_mpmath_and_mp_gradient():
    """dq of one row against 50-digit numerical differentiation of the exact forward."""
    rng = np.random.default_rng(5)
    q, k, v, do = _rand(rng, 3, 4), _rand(rng, 5, 4), _rand(rng, 5, 3), _rand(rng, 3, 3)
    scale = 0.6
    vis = oracle.visibility(3, 5, True)
    out, lse, _ = oracle.unit_forward(q, k, v, scale, vis)
    mo, ml = _mp_forward(q, k, v, scale, vis)
    np.testing.assert_allclose(out, mo, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, ml, rtol=1e-14, atol=1e-15)
    dq, dk, dv = oracle.unit_backward(q, k, v, do, scale, vis)
    mpmath.mp.dps = 40

    def loss_of_q(i, t):
        def f(x):
            qq = [[mpmath.mpf(c) for c in row] for row in q]
            qq[i][t] = x
            tot = mpmath.mpf(0)
            for r in range(3):
                e = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(qq[r][a] * mpmath.mpf(k[j, a])
                                                              for a in range(4)))
                     if vis[r, j] else mpmath.mpf(0) for j in range(5)]
                z = mpmath.fsum(e)
                for c in range(3):
                    tot += mpmath.mpf(do[r, c]) * mpmath.fsum(e[j] * mpmath.mpf(v[j, c])
                                                              for j in range(5)) / z
            return tot
        return f
    for (i, t) in ((0, 0), (1, 2), (2, 3)):
        g = float(mpmath.diff(loss_of_q(i, t), mpmath.mpf(q[i, t])))
        assert abs(g - dq[i, t]) <= 1e-12 * max(1.0, abs(g))


# ------------------------------------------------------------------------------------------
# 3. central finite differences of L = sum(out * dO)
# ------------------------------------------------------------------------------------------

def _fd_check(fwd, args, grads, names, eps=1e-6, tol=1e-7, samples=12, seed=0):
    rng = np.random.default_rng(seed)
    for name in names:
        x = args[name]
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(samples, flat.size), replace=False):
            h = eps * max(1.0, abs(flat[idx]))
            old = flat[idx]
            flat[idx] = old + h
            lp = fwd()
            flat[idx] = old - h
            lm = fwd()
            flat[idx] = old
            num = (lp - lm) / (2 * h)
            ana = grads[name].reshape(-1)[idx]
            assert abs(num - ana) <= tol * max(1.0, abs(num)), (name, idx, num, ana)


@pytest.mark.parametrize("case", [
    dict(causal=False, kind="none", H=2, Hkv=2),
    dict(causal=True, kind="none", H=4, Hkv=2),
    dict(causal=False, kind="bool", H=2, Hkv=1),
    dict(causal=True, kind="additive", H=2, Hkv=2),
])
def test_finite_differences_dense(case):
    rng = np.random.default_rng(19)
    B, Sq, Sk, D = 2, 5, 7, 6
    H, Hkv = case["H"], case["Hkv"]
    args = dict(q=_rand(rng, B, Sq, H, D), k=_rand(rng, B, Sk, Hkv, D), v=_rand(rng, B, Sk, Hkv, D))
    dout = _rand(rng, B, Sq, H, D)
    mask = None
    if case["kind"] == "bool":
        mask = rng.random((B, 1, Sq, Sk)) > 0.4
        mask[1, 0, 2, :] = False  # one fully-masked row
    elif case["kind"] == "additive":
        mask = 0.3 * rng.standard_normal((1, H, Sq, Sk))
        mask[rng.random(mask.shape) < 0.3] = -np.inf
    kw = dict(causal=case["causal"], scale=0.45, mask=mask, mask_kind=case["kind"])

    def loss():
        out, _ = oracle.attention_forward(args["q"], args["k"], args["v"], **kw)
        return float(np.sum(out * dout))
    dq, dk, dv = oracle.attention_backward(args["q"], args["k"], args["v"], dout, **kw)
    _fd_check(loss, args, dict(q=dq, k=dk, v=dv), ("q", "k", "v"))


def test_finite_differences_varlen():
    rng = np.random.default_rng(23)
    lens = [3, 6, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, Hkv, D = int(cu[-1]) + 2, 4, 2, 5  # two uncovered rows past cu[-1]
    args = dict(q=_rand(rng, T, H, D), k=_rand(rng, T, Hkv, D), v=_rand(rng, T, Hkv, D))
    dout = _rand(rng, T, H, D)
    kw = dict(causal=True, scale=0.5, cu_seqlens_q=cu, cu_seqlens_k=cu)

    def loss():
        out, _ = oracle.attention_forward(args["q"], args["k"], args["v"], **kw)
        return float(np.sum(out * dout))
    dq, dk, dv = oracle.attention_backward(args["q"], args["k"], args["v"], dout, **kw)
    _fd_check(loss, args, dict(q=dq, k=dk, v=dv), ("q", "k", "v"), samples=20)
    out, lse = oracle.attention_forward(args["q"], args["k"], args["v"], **kw)
    assert np.all(out[cu[-1]:] == 0) and np.all(np.isneginf(lse[:, cu[-1]:]))
    assert np.all(dq[cu[-1]:] == 0) and np.all(dk[cu[-1]:] == 0) and np.all(dv[cu[-1]:] == 0)


# ------------------------------------------------------------------------------------------
# 4. closed forms and special cases
# ------------------------------------------------------------------------------------------

def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(2)
    Sq, Sk, D = 6, 9, 4
    q, k, v, do = np.zeros((Sq, D)), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
    keep = rng.random((Sq, Sk)) > 0.5
    keep[:, 0] = True
    vis = oracle.visibility(Sq, Sk, False, keep)
    out, lse, _ = oracle.unit_forward(q, k, v, 0.7, vis)
    n = vis.sum(axis=1)
    for i in range(Sq):
        np.testing.assert_allclose(out[i], v[vis[i]].mean(axis=0), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse[i], math.log(n[i]), rtol=1e-15)
    # with q = 0, dq_i = (scale / n_i) * sum_j dO_i.(v_j - vbar_i) k_j over visible j
    dq, _, _ = oracle.unit_backward(q, k, v, do, 0.7, vis)
    for i in range(Sq):
        vis_j = np.nonzero(vis[i])[0]
        vbar = v[vis_j].mean(axis=0)
        want = 0.7 / n[i] * sum((do[i] @ (v[j] - vbar)) * k[j] for j in vis_j)
        np.testing.assert_allclose(dq[i], want, rtol=1e-12, atol=1e-14)


def test_single_visible_key_and_causal_row_zero():
    rng = np.random.default_rng(4)
    Sq = Sk = 5
    D = 3
    q, k, v, do = (_rand(rng, Sq, D) for _ in range(4))
    vis = oracle.visibility(Sq, Sk, True)
    out, lse, _ = oracle.unit_forward(q, k, v, 0.8, vis)
    assert np.array_equal(out[0], v[0])          # causal row 0 sees only key 0
    np.testing.assert_allclose(lse[0], 0.8 * q[0] @ k[0], rtol=1e-15)
    # one visible key everywhere: out = v_j, dq = 0, dk = 0, dv_j = sum of dO over its rows
    keep = np.zeros((Sq, Sk), dtype=bool)
    keep[:, 2] = True
    vis = oracle.visibility(Sq, Sk, False, keep)
    out, _, _ = oracle.unit_forward(q, k, v, 0.8, vis)
    dq, dk, dv = oracle.unit_backward(q, k, v, do, 0.8, vis)
    assert np.array_equal(out, np.broadcast_to(v[2], out.shape))
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[2], do.sum(axis=0), rtol=1e-15)
    assert np.all(dv[[0, 1, 3, 4]] == 0)


def test_two_keys_is_a_logistic():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 4, 3), _rand(rng, 2, 3), _rand(rng, 2, 3)
    vis = oracle.visibility(4, 2, False)
    out, _, P = oracle.unit_forward(q, k, v, 1.3, vis)
    d = 1.3 * (q @ k[0] - q @ k[1])
    sig = 1.0 / (1.0 + np.exp(-d))
    np.testing.assert_allclose(P[:, 0], sig, rtol=1e-14)
    np.testing.assert_allclose(out, sig[:, None] * v[0] + (1 - sig)[:, None] * v[1], rtol=1e-13)


# ------------------------------------------------------------------------------------------
# 5. invariants
# ------------------------------------------------------------------------------------------

def _problem(rng, B=2, Sq=9, Sk=11, H=4, Hkv=2, D=8):
    return (_rand(rng, B, Sq, H, D), _rand(rng, B, Sk, Hkv, D), _rand(rng, B, Sk, Hkv, D),
            _rand(rng, B, Sq, H, D))


def test_rows_of_p_sum_to_one_and_gradient_sums():
    rng = np.random.default_rng(12)
    q, k, v, do = (_rand(rng, 7, 5), _rand(rng, 10, 5), _rand(rng, 10, 5), _rand(rng, 7, 5))
    keep = rng.random((7, 10)) > 0.5
    keep[3] = False  # an empty row
    vis = oracle.visibility(7, 10, True, keep)
    _, _, P = oracle.unit_forward(q, k, v, 0.5, vis)
    nonempty = vis.any(axis=1)
    np.testing.assert_allclose(P[nonempty].sum(axis=1), 1.0, rtol=1e-15)
    dq, dk, dv = oracle.unit_backward(q, k, v, do, 0.5, vis)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-13)           # sum_j dS_ij = 0
    np.testing.assert_allclose(dv.sum(axis=0), do[nonempty].sum(axis=0), rtol=1e-13)
    assert np.all(dq[~nonempty] == 0)


def test_masked_zero_key_padding_changes_nothing():
    """Zero keys appended and masked out: the real results are unchanged (OpenWAM PR #64,
    'Fix': padded keys receive exactly zero attention) and the padded keys get dk = dv = 0."""
    rng = np.random.default_rng(13)
    q, k, v, do = _problem(rng, Sk=77)
    pad = 128 - 77
    kp = np.concatenate([k, np.zeros((2, pad, 2, 8))], axis=1)
    vp = np.concatenate([v, np.zeros((2, pad, 2, 8))], axis=1)
    for kind in ("none", "bool", "additive"):
        if kind == "none":
            m, mp = None, np.concatenate([np.ones((1, 1, 1, 77), bool), np.zeros((1, 1, 1, pad), bool)], -1)
            kind_p = "bool"
        elif kind == "bool":
            m = rng.random((2, 1, 9, 77)) > 0.2
            mp = np.concatenate([m, np.zeros((2, 1, 9, pad), bool)], axis=-1)
            kind_p = "bool"
        else:
            m = np.where(rng.random((2, 1, 9, 77)) > 0.2, 0.0, -np.inf)
            mp = np.concatenate([m, np.full((2, 1, 9, pad), -np.inf)], axis=-1)
            kind_p = "additive"
        a = oracle.attention_forward(q, k, v, mask=m, mask_kind=kind)
        b = oracle.attention_forward(q, kp, vp, mask=mp, mask_kind=kind_p)
        ga = oracle.attention_backward(q, k, v, do, mask=m, mask_kind=kind)
        gb = oracle.attention_backward(q, kp, vp, do, mask=mp, mask_kind=kind_p)
        np.testing.assert_allclose(b[0], a[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(gb[0], ga[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gb[1][:, :77], ga[1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gb[2][:, :77], ga[2], rtol=1e-12, atol=1e-13)
        assert np.all(gb[1][:, 77:] == 0) and np.all(gb[2][:, 77:] == 0)


def test_bool_equals_additive_and_causal_equals_triangle():
    rng = np.random.default_rng(14)
    q, k, v, do = _problem(rng, Sq=10, Sk=10)
    keep = rng.random((2, 4, 10, 10)) > 0.3
    add = np.where(keep, 0.0, -np.inf)
    assert all(np.array_equal(x, y, equal_nan=True) for x, y in zip(
        oracle.attention_forward(q, k, v, mask=keep, mask_kind="bool"),
        oracle.attention_forward(q, k, v, mask=add, mask_kind="additive")))
    tri = np.where(np.tril(np.ones((10, 10), bool)), 0.0, -np.inf)[None, None]
    a = oracle.attention_backward(q, k, v, do, causal=True)
    b = oracle.attention_backward(q, k, v, do, mask=tri, mask_kind="additive")
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-14, atol=1e-15)


def test_key_shift_and_permutation():
    rng = np.random.default_rng(15)
    q, k, v, do = _problem(rng, H=2, Hkv=2)
    c = rng.standard_normal(8)
    out, lse = oracle.attention_forward(q, k, v, scale=0.3)
    out2, lse2 = oracle.attention_forward(q, k + c, v, scale=0.3)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    shift = 0.3 * np.einsum("bshd,d->bhs", q, c)
    np.testing.assert_allclose(lse2, lse + shift, rtol=1e-12, atol=1e-12)
    g1 = oracle.attention_backward(q, k, v, do, scale=0.3)
    g2 = oracle.attention_backward(q, k + c, v, do, scale=0.3)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(y, x, rtol=1e-10, atol=1e-11)
    perm = rng.permutation(k.shape[1])
    out3, lse3 = oracle.attention_forward(q, k[:, perm], v[:, perm], scale=0.3)
    np.testing.assert_allclose(out3, out, rtol=1e-13, atol=1e-14)
    g3 = oracle.attention_backward(q, k[:, perm], v[:, perm], do, scale=0.3)
    np.testing.assert_allclose(g3[0], g1[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g3[1], g1[1][:, perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g3[2], g1[2][:, perm], rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(16)
    q, k, v, do = _problem(rng, H=6, Hkv=2)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    a = oracle.attention_forward(q, k, v, causal=True)
    b = oracle.attention_forward(q, kr, vr, causal=True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    ga = oracle.attention_backward(q, k, v, do, causal=True)
    gb = oracle.attention_backward(q, kr, vr, do, causal=True)
    np.testing.assert_array_equal(ga[0], gb[0])
    np.testing.assert_allclose(ga[1], gb[1].reshape(2, 11, 2, 3, 8).sum(3), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ga[2], gb[2].reshape(2, 11, 2, 3, 8).sum(3), rtol=1e-13, atol=1e-14)


def test_varlen_equals_per_sequence_dense():
    rng = np.random.default_rng(17)
    lens = [5, 1, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, Hkv, D = int(cu[-1]), 4, 2, 6
    q, k, v, do = _rand(rng, T, H, D), _rand(rng, T, Hkv, D), _rand(rng, T, Hkv, D), _rand(rng, T, H, D)
    out, lse = oracle.attention_forward(q, k, v, causal=True, cu_seqlens_q=cu, cu_seqlens_k=cu)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=True, cu_seqlens_q=cu, cu_seqlens_k=cu)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        o1, l1 = oracle.attention_forward(q[None, a:b], k[None, a:b], v[None, a:b], causal=True)
        g1 = oracle.attention_backward(q[None, a:b], k[None, a:b], v[None, a:b], do[None, a:b], causal=True)
        np.testing.assert_array_equal(out[a:b], o1[0])
        np.testing.assert_array_equal(lse[:, a:b], l1[0])
        np.testing.assert_array_equal(dq[a:b], g1[0][0])
        np.testing.assert_array_equal(dk[a:b], g1[1][0])
        np.testing.assert_array_equal(dv[a:b], g1[2][0])


def test_sampled_rows_and_keys_match_whole_oracle():
    rng = np.random.default_rng(18)
    q, k, v, do = _problem(rng, B=1, Sq=40, Sk=40, H=1, Hkv=1, D=8)
    out, lse = oracle.attention_forward(q, k, v, causal=True, scale=0.4)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=True, scale=0.4)
    rows = np.array([0, 7, 39])
    o, l = oracle.rows_forward(q[0, rows, 0], k[0, :, 0], v[0, :, 0], rows, 0.4, True)
    np.testing.assert_allclose(o, out[0, rows, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l, lse[0, 0, rows], rtol=1e-14)
    d = oracle.rows_backward_dq(q[0, rows, 0], k[0, :, 0], v[0, :, 0], do[0, rows, 0], rows, 0.4, True)
    np.testing.assert_allclose(d, dq[0, rows, 0], rtol=1e-12, atol=1e-13)
    keys = np.array([0, 21, 39])
    dk2, dv2 = oracle.keys_backward(q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0], keys, 0.4, True,
                                    row_chunk=16)
    np.testing.assert_allclose(dk2, dk[0, keys, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv2, dv[0, keys, 0], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------------
# 6. values the pages print
# ------------------------------------------------------------------------------------------

def test_lse_range_at_k_scale_32_matches_page():
    """At k scaled 32x the page's finite rows had LSE in [80.8, 217.8] (natural-log units).
    A log2 LSE, or a dropped 1/sqrt(D) scale, would leave that interval."""
    g = GOLDEN["lse_good_rows_k32"]
    p = workloads.dense(1, 256, 8192, 1, 1, 128, seed=3032, k_mult=32.0)
    q = p.q.double().numpy()[0, :, 0]
    k = p.k.double().numpy()[0, :, 0]
    v = p.v.double().numpy()[0, :, 0]
    _, lse = oracle.rows_forward(q, k, v, np.arange(256), 1 / math.sqrt(128), False)
    assert lse.min() >= g["lo"] and lse.max() <= g["hi"], (lse.min(), lse.max())
    assert (lse / math.log(2)).max() > g["hi"]  # the log2 reading is ruled out


@pytest.mark.parametrize("shape", workloads.PADDED_TILE_SHAPES)
@pytest.mark.parametrize("kind", ["none", "bool", "additive"])
def test_anti_aligned_row_lse_matches_page(shape, kind):
    g = GOLDEN["anti_aligned_row_lse"]
    p = workloads.padded_tile(*shape, mask_kind=kind)
    out, lse = oracle.attention_forward(p.q.double().numpy(), p.k.double().numpy(),
                                        p.v.double().numpy(), mask=None if p.mask is None else
                                        p.mask.double().numpy() if kind == "additive" else p.mask.numpy(),
                                        mask_kind=p.mask_kind)
    for b, r in p.meta["anti_rows"].items():
        row = lse[b, :, r]
        assert np.all(row >= g["lo"]) and np.all(row <= g["hi"]), row
        # below the point where exp(0 - lse) overflows fp32
        assert np.all(row < GOLDEN["exp_overflow_lse"]["value"])
    assert np.isfinite(out).all()


def test_nonfinite_inputs_propagate():
    """Reading: non-finite inputs propagate through IEEE arithmetic and are never cleaned.
    A NaN in one query row makes that row's out, lse and dq NaN and, since the row sees
    every key, all of dk and dv; the other rows' out, lse and dq are unchanged bit for
    bit. A NaN in one key reaches every row that sees it."""
    rng = np.random.default_rng(77)
    q, k, v, do = (rng.standard_normal(s) for s in ((1, 6, 2, 8), (1, 5, 1, 8), (1, 5, 1, 8), (1, 6, 2, 8)))
    o0, l0 = oracle.attention_forward(q, k, v)
    g0 = oracle.attention_backward(q, k, v, do)
    qn = q.copy()
    qn[0, 2, 1, 3] = np.nan
    o1, l1 = oracle.attention_forward(qn, k, v)
    dq1, dk1, dv1 = oracle.attention_backward(qn, k, v, do)
    assert np.all(np.isnan(o1[0, 2, 1])) and np.isnan(l1[0, 1, 2]) and np.all(np.isnan(dq1[0, 2, 1]))
    keep = np.ones(o1.shape[:3], dtype=bool)
    keep[0, 2, 1] = False
    assert np.array_equal(o1[keep], o0[keep]) and np.array_equal(dq1[keep], g0[0][keep])
    assert np.array_equal(np.delete(l1[0, 1], 2), np.delete(l0[0, 1], 2)) and np.array_equal(l1[0, 0], l0[0, 0])
    assert np.all(np.isnan(dk1)) and np.all(np.isnan(dv1))
    kn = k.copy()
    kn[0, 4, 0, 0] = np.nan
    o2, _ = oracle.attention_forward(q, kn, v, causal=True)
    assert np.all(np.isfinite(o2[0, :4])) and np.all(np.isnan(o2[0, 4:]))   # rows >= 4 see key 4
