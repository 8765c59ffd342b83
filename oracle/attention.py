"""Float64 CPU oracle for exact softmax attention: forward (out, lse) and backward (dq, dk, dv).

TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and nothing here
is shared with the GPU library.

What it computes is the plain definition, written out per (batch or sequence, query head)
unit with full score matrices. Tiling and online rescaling are exact reformulations of the
same function, so the oracle does neither. Sources:

* Forward with a log-sum-exp output and a max-stabilised exponent: FlyDSL PR #1033,
  "[Bugfix][Kernel] Fix NaN from the lazy rescale on a wide score range", sections
  "Root cause" and "The fix" (the running max is max(m_row, m_tile); the LSE is a per-row
  output whose range is quoted under "Evidence").
* Backward products dv = P^T dO and dk = dS^T q: flash-dmattn PR #122, "Fix NaN/Inf values
  in dV gradients during backward pass", section "Solution", item 2.
* Backward evaluates P from the stored LSE, exp(s - lse): OpenWAM PR #64 (cuDNN SDPA
  backward padding fix), "Summary".
* Mask semantics (bool False hides a key, additive -inf hides a key, padded keys receive
  exactly zero attention): OpenWAM PR #64, "Fix".
* Grouped KV heads (num_kv_heads) and causal masking: flash-dmattn PR #122, "Problem".
* Packed variable-length rows and the rows past cu_seqlens_q[-1]: PFCCLab cudnn-frontend
  PR #9, "DSA: fix dK SMEM handoff race and two latent NaN sources in the dense indexer",
  item 2.

Readings where the pages are silent (each is listed in the design notes):
* lse is the natural log of the row's sum of exp(s).
* A row with no visible key has out = 0, lse = -inf, dq = 0 and contributes nothing to
  dk/dv.
* Causal alignment is top-left: key j is visible to query i iff j <= i (indices local to
  the sequence in the packed layout).
* Query head h uses KV head h // (H // Hkv).
* A finite additive-mask value is a bias; only -inf hides a key.

Parity unpinned (pinned by definition only): the empty-row sentinel (out = 0, lse = -inf)
and the top-left causal alignment for S_q != S_kv.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "visibility",
    "unit_forward",
    "unit_backward",
    "attention_forward",
    "attention_backward",
    "rows_forward",
    "rows_backward_dq",
    "keys_backward",
]


# ----------------------------------------------------------------------------------------
# One unit: one query head of one batch entry (or one packed sequence) against its KV head.
# ----------------------------------------------------------------------------------------

def visibility(sq, sk, causal, keep=None, bias=None, row_index=None):
    """Boolean [sq, sk] matrix: True where query i may attend key j.

    A key is hidden by causality (j > i, top-left alignment), by a False entry of a bool
    mask, or by a -inf entry of an additive mask (OpenWAM PR #64, "Fix").
    ``row_index`` gives the sequence-local index of each query row when only a subset of
    rows is evaluated (default: 0..sq-1).
    """
    vis = np.ones((sq, sk), dtype=bool)
    if causal:
        i = np.arange(sq) if row_index is None else np.asarray(row_index)
        vis &= np.arange(sk)[None, :] <= i[:, None]
    if keep is not None:
        vis &= np.asarray(keep, dtype=bool)
    if bias is not None:
        vis &= ~np.isneginf(bias)
    return vis


def _scores(q, k, scale, bias):
    s = scale * (q @ k.T)
    if bias is not None:
        b = np.where(np.isneginf(bias), 0.0, bias)  # hidden entries are removed via vis
        s = s + b
    return s


def unit_forward(q, k, v, scale, vis, bias=None):
    """Softmax attention of one unit by the definition.

    q [sq, d], k [sk, d], v [sk, d] float64; vis [sq, sk] bool; bias [sq, sk] or None.
    Returns out [sq, d], lse [sq], P [sq, sk].

    s_ij = scale * q_i . k_j + bias_ij; m_i = max over visible j; e_ij = exp(s_ij - m_i)
    on visible entries, 0 elsewhere; l_i = sum_j e_ij; P = e / l; out = P v;
    lse = m + ln l. A row with no visible key gets P = 0, out = 0, lse = -inf.
    """
    s = _scores(q, k, scale, bias)
    s_vis = np.where(vis, s, -np.inf)
    m = s_vis.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    nonempty = vis.any(axis=1) if s.shape[1] else np.zeros(s.shape[0], dtype=bool)
    m_safe = np.where(nonempty, m, 0.0)
    e = np.where(vis, np.exp(s_vis - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    P = np.where(nonempty[:, None], e / np.where(nonempty, l, 1.0)[:, None], 0.0)
    out = P @ v
    lse = np.where(nonempty, m_safe + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return out, lse, P


def unit_backward(q, k, v, dout, scale, vis, bias=None):
    """Gradients of sum(out * dout) for one unit, by the analytic formulas.

    P is recomputed by the definition; dV = P^T dO; dP = dO V^T; Delta_i = dO_i . out_i;
    dS = P * (dP - Delta); dQ = scale * dS K; dK = scale * dS^T Q.
    Returns dq [sq, d], dk [sk, d], dv [sk, d].
    """
    out, _, P = unit_forward(q, k, v, scale, vis, bias)
    dv = P.T @ dout
    dP = dout @ v.T
    delta = np.sum(dout * out, axis=1)
    dS = P * (dP - delta[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Whole tensors: BSHD dense batches or THD packed sequences.
# ----------------------------------------------------------------------------------------

def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _mask_slices(mask, mask_kind, b, h, sq, sk):
    """Return (keep, bias) for unit (b, h) from a mask broadcastable to [B, H, sq, sk]."""
    if mask is None or mask_kind in (None, "none"):
        return None, None
    m = np.asarray(mask)
    while m.ndim < 4:
        m = m[None]
    mb = m[b if m.shape[0] > 1 else 0, h if m.shape[1] > 1 else 0]
    mb = np.broadcast_to(mb, (sq, sk))
    if mask_kind == "bool":
        return mb.astype(bool), None
    if mask_kind == "additive":
        return None, mb.astype(np.float64)
    raise ValueError(f"unknown mask kind {mask_kind!r}")


def _units(varlen, batch, nseq, heads):
    n = nseq if varlen else batch
    return [(u, h) for u in range(n) for h in range(heads)]


def attention_forward(q, k, v, *, causal=False, scale=None, mask=None, mask_kind=None,
                      cu_seqlens_q=None, cu_seqlens_k=None, units=None):
    """Oracle forward over a whole problem.

    Dense: q [B, Sq, H, D], k/v [B, Sk, Hkv, D]; returns out [B, Sq, H, D], lse [B, H, Sq].
    Packed: q [Tq, H, D], k/v [Tk, Hkv, D] with cu_seqlens (nseq + 1 offsets);
    returns out [Tq, H, D], lse [H, Tq]. Rows past cu_seqlens_q[-1] get out = 0 and
    lse = -inf (PFCCLab cudnn-frontend PR #9, item 2: every row of the output is written).
    ``units`` restricts the work to a list of (batch or sequence, head); other units are
    NaN in the result.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    varlen = cu_seqlens_q is not None
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    H, Hkv = q.shape[-2], k.shape[-2]
    grp = H // Hkv
    out = np.full(q.shape, np.nan)
    if varlen:
        cq, ck = np.asarray(cu_seqlens_q), np.asarray(cu_seqlens_k)
        nseq = len(cq) - 1
        lse = np.full((H, q.shape[0]), np.nan)
        out[cq[-1]:] = 0.0
        lse[:, cq[-1]:] = -np.inf
    else:
        B, Sq = q.shape[0], q.shape[1]
        Sk = k.shape[1]
        lse = np.full((B, H, Sq), np.nan)
    todo = units if units is not None else _units(varlen, q.shape[0], len(cu_seqlens_q) - 1
                                                  if varlen else 0, H)
    for (u, h) in todo:
        g = h // grp
        if varlen:
            qs, qe, ks, ke = cq[u], cq[u + 1], ck[u], ck[u + 1]
            qu, ku, vu = q[qs:qe, h], k[ks:ke, g], v[ks:ke, g]
            keep = bias = None
        else:
            qu, ku, vu = q[u, :, h], k[u, :, g], v[u, :, g]
            keep, bias = _mask_slices(mask, mask_kind, u, h, Sq, Sk)
        vis = visibility(qu.shape[0], ku.shape[0], causal, keep, bias)
        o, l, _ = unit_forward(qu, ku, vu, scale, vis, bias)
        if varlen:
            out[qs:qe, h] = o
            lse[h, qs:qe] = l
        else:
            out[u, :, h] = o
            lse[u, h] = l
    return out, lse


def attention_backward(q, k, v, dout, *, causal=False, scale=None, mask=None, mask_kind=None,
                       cu_seqlens_q=None, cu_seqlens_k=None, kv_units=None):
    """Oracle backward over a whole problem: returns dq, dk, dv in the layouts of q, k, v.

    dk and dv of a KV head sum the contributions of every query head that shares it.
    Rows past cu_seqlens_q[-1] get dq = 0 and keys past cu_seqlens_k[-1] get dk = dv = 0.
    ``kv_units`` restricts the work to a list of (batch or sequence, kv head); dq of the
    query heads of those groups and dk/dv of those kv heads are filled, the rest is NaN.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    varlen = cu_seqlens_q is not None
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    H, Hkv = q.shape[-2], k.shape[-2]
    grp = H // Hkv
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    if varlen:
        cq, ck = np.asarray(cu_seqlens_q), np.asarray(cu_seqlens_k)
        nseq = len(cq) - 1
        dq[cq[-1]:] = 0.0
        dk[ck[-1]:] = 0.0
        dv[ck[-1]:] = 0.0
        todo = kv_units if kv_units is not None else [(s, g) for s in range(nseq)
                                                      for g in range(Hkv)]
    else:
        B, Sq, Sk = q.shape[0], q.shape[1], k.shape[1]
        todo = kv_units if kv_units is not None else [(b, g) for b in range(B)
                                                      for g in range(Hkv)]
    for (u, g) in todo:
        if varlen:
            qs, qe, ks, ke = cq[u], cq[u + 1], ck[u], ck[u + 1]
            dk_acc = np.zeros((ke - ks, D))
        else:
            dk_acc = np.zeros((Sk, D))
        dv_acc = np.zeros_like(dk_acc)
        for h in range(g * grp, (g + 1) * grp):
            if varlen:
                qu, ku, vu, du = q[qs:qe, h], k[ks:ke, g], v[ks:ke, g], dout[qs:qe, h]
                keep = bias = None
            else:
                qu, ku, vu, du = q[u, :, h], k[u, :, g], v[u, :, g], dout[u, :, h]
                keep, bias = _mask_slices(mask, mask_kind, u, h, Sq, Sk)
            vis = visibility(qu.shape[0], ku.shape[0], causal, keep, bias)
            dqu, dku, dvu = unit_backward(qu, ku, vu, du, scale, vis, bias)
            dk_acc += dku
            dv_acc += dvu
            if varlen:
                dq[qs:qe, h] = dqu
            else:
                dq[u, :, h] = dqu
        if varlen:
            dk[ks:ke, g] = dk_acc
            dv[ks:ke, g] = dv_acc
        else:
            dk[u, :, g] = dk_acc
            dv[u, :, g] = dv_acc
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Sampled rows and keys, for problems too large for the whole oracle. Query rows are
# independent in the definition, so a subset of rows is the definition on those rows.
# ----------------------------------------------------------------------------------------

def rows_forward(q_rows, k, v, row_index, scale, causal, keep_rows=None, bias_rows=None):
    """out and lse of selected query rows of one unit.

    q_rows [n, d] are the selected query vectors, ``row_index`` their sequence-local
    indices (used by causal masking), k/v [sk, d] the unit's keys and values.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    vis = visibility(q_rows.shape[0], k.shape[0], causal, keep_rows, bias_rows, row_index)
    out, lse, _ = unit_forward(q_rows, k, v, scale, vis, bias_rows)
    return out, lse


def rows_backward_dq(q_rows, k, v, dout_rows, row_index, scale, causal,
                     keep_rows=None, bias_rows=None):
    """dq of selected query rows of one unit (each row's dq needs only that row's P)."""
    q_rows, k, v, dout_rows = _f64(q_rows), _f64(k), _f64(v), _f64(dout_rows)
    vis = visibility(q_rows.shape[0], k.shape[0], causal, keep_rows, bias_rows, row_index)
    dq, _, _ = unit_backward(q_rows, k, v, dout_rows, scale, vis, bias_rows)
    return dq


def keys_backward(q, k, v, dout, key_index, scale, causal, row_chunk=1024, row_offset=0):
    """dk and dv of selected keys of one unit, summing over every query row.

    q/dout [n, d] hold the unit's query rows starting at sequence-local row ``row_offset``;
    each query row's P is the definition over all keys (its normaliser needs them all), and
    only the selected key columns of dS and P enter dk = scale * dS^T q and dv = P^T dO.
    Rows are visited in chunks to bound memory; every given row is visited exactly once.
    Leaving out the rows before ``row_offset`` is exact only when none of them can see a
    selected key, i.e. causal masking with every selected key at or after ``row_offset``.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    key_index = np.asarray(key_index)
    if row_offset:
        assert causal and key_index.min() >= row_offset, "rows before row_offset see the keys"
    sq = q.shape[0]
    dk = np.zeros((len(key_index), q.shape[1]))
    dv = np.zeros_like(dk)
    for r0 in range(0, sq, row_chunk):
        rows = np.arange(r0, min(sq, r0 + row_chunk))
        vis = visibility(len(rows), k.shape[0], causal, row_index=rows + row_offset)
        out, _, P = unit_forward(q[rows], k, v, scale, vis)
        dP = dout[rows] @ v[key_index].T
        delta = np.sum(dout[rows] * out, axis=1)
        Psel = P[:, key_index]
        dS = Psel * (dP - delta[:, None])
        dv += Psel.T @ dout[rows]
        dk += scale * (dS.T @ q[rows])
    return dk, dv
