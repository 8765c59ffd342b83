"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI (via the
package binding), run the float64 oracle on the same bf16 inputs, and compare."""

import sys

import numpy as np
import torch

import oracle
from exact_attention_40_amd import api

# Parity bars (bf16 inputs, fp32 accumulation): rel-L2 against the float64 oracle.
TOL = dict(out=1e-2, lse=1e-2, dq=2e-2, dk=2e-2, dv=2e-2)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_inputs(p, layout="bshd"):
    """Upload a problem's tensors; 'bhsd' stores them head-major and passes BSHD views."""
    def up(t):
        t = t.cuda()
        if layout == "bhsd" and t.dim() == 4:
            t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        return t
    kw = dict(causal=p.causal, scale=p.scale)
    if p.mask is not None:
        kw["mask"] = p.mask.cuda()
    if p.varlen:
        kw.update(cu_seqlens_q=p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k)
    return up(p.q), up(p.k), up(p.v), up(p.dout), kw


def run_gpu(p, layout="bshd", backward=True):
    q, k, v, do, kw = gpu_inputs(p, layout)
    out, lse = api.exattn_fwd(q, k, v, **kw)
    res = dict(out=out, lse=lse)
    if backward:
        dq, dk, dv = api.exattn_bwd(q, k, v, out, do, lse, **kw)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def oracle_mask(p):
    if p.mask is None:
        return None
    return p.mask.float().numpy() if p.mask_kind == "additive" else p.mask.numpy()


def run_oracle(p, backward=True, units=None, kv_units=None):
    kw = dict(causal=p.causal, scale=p.softmax_scale, mask=oracle_mask(p), mask_kind=p.mask_kind)
    if p.varlen:
        kw.update(cu_seqlens_q=p.cu_seqlens_q.numpy(), cu_seqlens_k=p.cu_seqlens_k.numpy())
    q, k, v, do = f64(p.q), f64(p.k), f64(p.v), f64(p.dout)
    out, lse = oracle.attention_forward(q, k, v, units=units, **kw)
    res = dict(out=out, lse=lse)
    if backward:
        dq, dk, dv = oracle.attention_backward(q, k, v, do, kv_units=kv_units, **kw)
        res.update(dq=dq, dk=dk, dv=dv)
    return res


def rel_l2(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def nonfinite(t):
    return int((~torch.isfinite(t)).sum().item())


def compare(gpu, ref, names=("out", "lse", "dq", "dk", "dv"), select=None, tag=""):
    """Check rel-L2 per tensor, zero non-finite values, and exact empty-row sentinels.

    ``select`` maps a tensor name to an index expression restricting the comparison
    (for sampled units); entries the oracle left NaN are never compared.
    """
    report = {}
    for n in names:
        g = f64(gpu[n])
        r = ref[n]
        if select and n in select:
            g, r = g[select[n]], r[select[n]]
        if n == "lse":
            empty = np.isneginf(r)
            assert np.array_equal(np.isneginf(g), empty), f"{tag} lse sentinel mismatch"
            keep = ~empty & ~np.isnan(r)
            assert np.isfinite(g[keep]).all(), f"{tag} non-finite lse"
            g, r = g[keep], r[keep]
        else:
            keep = ~np.isnan(r)
            assert np.isfinite(g[keep]).all(), f"{tag} {n}: {int((~np.isfinite(g[keep])).sum())} non-finite"
            g, r = g[keep], r[keep]
        e = rel_l2(g, r)
        report[n] = e
        assert e <= TOL[n], f"{tag} {n}: rel-L2 {e:.3e} > {TOL[n]:.0e}"
    say(f"  {tag} " + " ".join(f"{n}={e:.2e}" for n, e in report.items()))
    return report


def dq_reassociation_bound(p, block_n=128):
    """Per-element bound on run-to-run differences of dq (float64 numpy, dq's layout).

    dq sums one fp32 partial per block of `block_n` keys with atomics, so two runs differ
    only by the order of those additions. For N terms that is at most
    (N - 1) * 2**-24 * sum_i |t_i| (PFCCLab cudnn-frontend PR #9, "How it was verified"),
    and sum_i |t_i| <= scale * sum_j |dS_ij k_jd|; dS comes from the float64 oracle.
    Dense problems only.
    """
    q, k, v, do = f64(p.q), f64(p.k), f64(p.v), f64(p.dout)
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    scale = p.softmax_scale
    nblk = max(1, -(-Sk // block_n))
    bound = np.zeros_like(q)
    m = oracle_mask(p)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            keep = bias = None
            if m is not None:
                mm = m
                while mm.ndim < 4:
                    mm = mm[None]
                mb = np.broadcast_to(mm[b if mm.shape[0] > 1 else 0, h if mm.shape[1] > 1 else 0],
                                     (Sq, Sk))
                if p.mask_kind == "bool":
                    keep = mb.astype(bool)
                else:
                    bias = mb.astype(np.float64)
            vis = oracle.visibility(Sq, Sk, p.causal, keep, bias)
            out, _, P = oracle.unit_forward(q[b, :, h], k[b, :, g], v[b, :, g], scale, vis, bias)
            dP = do[b, :, h] @ v[b, :, g].T
            dS = P * (dP - np.sum(do[b, :, h] * out, axis=1)[:, None])
            bound[b, :, h] = (nblk - 1) * 2.0 ** -24 * scale * (np.abs(dS) @ np.abs(k[b, :, g]))
    return bound


def dq_runs_agree(a, b, bound):
    """|a - b| <= bound + one bf16 ulp of max(|a|, |b|); reports the worst ratio."""
    a64, b64 = f64(a), f64(b)
    mag = np.maximum(np.abs(a64), np.abs(b64))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    diff = np.abs(a64 - b64)
    lim = bound + ulp
    worst = float(np.max(diff / np.where(lim > 0, lim, 1e-300))) if diff.size else 0.0
    say(f"  dq run-to-run: {int((diff > 0).sum())} of {diff.size} elements differ, "
        f"worst diff/bound = {worst:.3f}")
    return bool(np.all(diff <= lim))
