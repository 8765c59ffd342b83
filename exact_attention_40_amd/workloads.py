"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and arranges them into tensors; it holds none of
the attention arithmetic. The oracle and the GPU library both consume what it returns,
so they always see identical bf16 bits.

Random source: NumPy PCG64 float32 standard normals, rounded to bf16 by torch
(round-to-nearest-even). Seeds follow ``1000 * workload + variant``.

Workloads (the pages describe the shapes; every value here is synthetic):

* ``dv_nan_repro`` - B1 H1 Hkv1 S256 D64 causal, dout = ones (loss = out.sum()): the
  failing configuration of flash-dmattn PR #122 ("Fix NaN/Inf values in dV gradients
  during backward pass", section "Problem").
* ``padded_tile`` - B2 H4 D128 with (S_q, S_kv) in {(392,392), (360,64), (100,77)} and bool,
  additive, key-broadcast or no mask, with one query row per (b, h) anti-aligned with keys
  that share a large component so its LSE is about -111 to -120 (OpenWAM PR #64,
  "Validation", the minimal reproduction).
* ``wide_logit`` - B2 S8192 H32 D128 non-causal with k = bf16(N(0,1) * s) (FlyDSL PR #1033,
  "Repro" and "Result": the K-scale sweep).
* ``varlen_gqa`` - 16 packed sequences with lengths uniform in [128, 4096], H32 Hkv8, causal.
* ``long_causal`` - B1 S61380 H32 D128 causal (FlyDSL PR #1033, "Result": the shortest
  sequence length of its throughput table).
* ``masked`` - dense inputs with a bool mask or an additive bf16 bias in a chosen shape
  (per-head [B, H, S_q, S_k], per-batch [B, 1, S_q, S_k] or 2-D [S_q, S_k]): OpenWAM PR #64
  ("Fix") reads an additive mask's -inf as hidden and a finite value as a bias added to
  the score. Biases are N(0,1) * bias_std rounded to bf16, with a fraction of -inf entries;
  optional rows hold one constant bias for every key (a constant cancels in the softmax).
* ``fp8_dense`` - fp8 e4m3 q, k, v with one descale per tensor for the fp8 forward
  (FlyDSL PR #1033, "The fp8 helper, second commit": K scaled by a large factor, V = ones
  in some of its runs). ``kind="normal"`` quantises N(0,1) draws (the descale maps the
  largest magnitude to 448); ``kind="grid"`` draws q and k from {0, +-0.5, +-1, +-1.5, +-2}
  and v from {+-0.5, +-1}, whose products and dot products are exact in fp32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Problem", "Fp8Problem", "fp8_dense", "dense", "dv_nan_repro", "padded_tile", "wide_logit", "varlen_gqa",
           "long_causal", "masked", "PADDED_TILE_SHAPES", "WIDE_LOGIT_SCALES"]

PADDED_TILE_SHAPES = ((392, 392), (360, 64), (100, 77))
WIDE_LOGIT_SCALES = (1, 8, 16, 24, 32, 48, 64)


@dataclass
class Problem:
    """One attention problem: bf16 CPU tensors plus its options."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dout: torch.Tensor
    causal: bool = False
    scale: Optional[float] = None
    mask: Optional[torch.Tensor] = None       # bool (True = attend) or bf16 additive
    mask_kind: str = "none"                   # "none" | "bool" | "additive"
    cu_seqlens_q: Optional[torch.Tensor] = None  # int32 CPU, nseq + 1 offsets
    cu_seqlens_k: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens_q is not None

    @property
    def head_dim(self) -> int:
        return self.q.shape[-1]

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim) if self.scale is None else float(self.scale)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, mult=1.0, dtype=torch.bfloat16):
    """float32 standard normals (times mult) rounded to the 16-bit input format."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return torch.from_numpy(x).to(dtype)


def dense(B, Sq, Sk, H, Hkv, D, seed, *, causal=False, k_mult=1.0, dout_ones=False,
          name="dense", dtype=torch.bfloat16):
    """q, v, dout ~ N(0,1), k ~ N(0,1) * k_mult, all in `dtype` (bf16 or fp16), BSHD
    contiguous."""
    rng = _rng(seed)
    q = _normal(rng, (B, Sq, H, D), dtype=dtype)
    k = _normal(rng, (B, Sk, Hkv, D), k_mult, dtype=dtype)
    v = _normal(rng, (B, Sk, Hkv, D), dtype=dtype)
    dout = (torch.ones((B, Sq, H, D), dtype=dtype) if dout_ones
            else _normal(rng, (B, Sq, H, D), dtype=dtype))
    return Problem(name, q, k, v, dout, causal=causal,
                   meta=dict(B=B, Sq=Sq, Sk=Sk, H=H, Hkv=Hkv, D=D, seed=seed, k_mult=k_mult,
                             dtype=str(dtype)))


def dv_nan_repro(seed=42):
    """B1 H1 Hkv1 S256 D64, causal, dout = ones."""
    p = dense(1, 256, 256, 1, 1, 64, seed, causal=True, dout_ones=True, name="dv_nan_repro")
    return p


def padded_tile(sq, sk, mask_kind="bool", seed=2000, D=128, B=2, H=4, anti_row=True,
                dtype=torch.bfloat16):
    """Shapes off the 128-key tile, with one anti-aligned low-LSE query row per (b, h).

    Mask ([B, 1, sq, sk]): keep_bij = (j < L_b) and (u_bij >= 0.1 or j == 0) with
    L_0 = sk, L_1 = ceil(0.75 sk) and u ~ U(0, 1). "additive" is the same mask as 0 / -inf
    in bf16. "keypad" is a key-broadcast [B, 1, 1, sk] bool mask keep_bj = j < L_b.
    Anti-aligned row, per (b, h): a random unit vector u and a unit w orthogonal to it;
    every key of the head becomes n_j - (n_j . u) u + 16 u and the query row becomes
    -84 u + 8 w, all rounded to `dtype` (bf16 or fp16). The row is sq - 1 (inside the last,
    partial query tile) for b = 0 and sq // 2 for b = 1. The additive mask is bf16 either way.
    """
    rng = _rng(seed)
    q32 = rng.standard_normal(size=(B, sq, H, D), dtype=np.float32)
    k32 = rng.standard_normal(size=(B, sk, H, D), dtype=np.float32)
    v32 = rng.standard_normal(size=(B, sk, H, D), dtype=np.float32)
    do32 = rng.standard_normal(size=(B, sq, H, D), dtype=np.float32)
    rows = {}
    if anti_row:
        for b in range(B):
            r = sq - 1 if b == 0 else sq // 2
            rows[b] = r
            for h in range(H):
                u = rng.standard_normal(D)
                u /= np.linalg.norm(u)
                w = rng.standard_normal(D)
                w -= (w @ u) * u
                w /= np.linalg.norm(w)
                n = k32[b, :, h].astype(np.float64)
                k32[b, :, h] = (n - np.outer(n @ u, u) + 16.0 * u).astype(np.float32)
                q32[b, r, h] = (-84.0 * u + 8.0 * w).astype(np.float32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dtype)  # noqa: E731
    mask = None
    L = [sk, int(math.ceil(0.75 * sk))][:B] + [sk] * max(0, B - 2)
    if mask_kind in ("bool", "additive"):
        uu = rng.random(size=(B, 1, sq, sk))
        j = np.arange(sk)
        keep = np.zeros((B, 1, sq, sk), dtype=bool)
        for b in range(B):
            keep[b] = (j < L[b]) & ((uu[b] >= 0.1) | (j == 0))
        if mask_kind == "bool":
            mask = torch.from_numpy(keep)
        else:
            add = np.where(keep, 0.0, -np.inf).astype(np.float32)
            mask = torch.from_numpy(add).to(torch.bfloat16)
    elif mask_kind == "keypad":
        j = np.arange(sk)
        keep = np.stack([(j < L[b]) for b in range(B)])[:, None, None, :]
        mask = torch.from_numpy(np.ascontiguousarray(keep))
    elif mask_kind != "none":
        raise ValueError(mask_kind)
    kind = {"bool": "bool", "keypad": "bool", "additive": "additive", "none": "none"}[mask_kind]
    return Problem(f"padded_tile_{sq}x{sk}_{mask_kind}", bf(q32), bf(k32), bf(v32), bf(do32),
                   causal=False, mask=mask, mask_kind=kind,
                   meta=dict(B=B, Sq=sq, Sk=sk, H=H, Hkv=H, D=D, seed=seed, anti_rows=rows))


def masked(B, Sq, Sk, H, Hkv, D, seed, *, kind="additive", shape="per_head", causal=False,
           bias_std=4.0, hide_frac=0.1, const_rows=(), dtype=torch.bfloat16):
    """Dense inputs (q, k, v, dout ~ N(0,1)) with a mask of `shape` "per_head"
    [B, H, Sq, Sk], "per_batch" [B, 1, Sq, Sk] or "2d" [Sq, Sk].

    kind "additive": bf16 bias N(0,1) * bias_std, with about `hide_frac` of the entries -inf
    (key 0 of every row stays finite). kind "bool": True = attend with probability
    1 - hide_frac (key 0 always kept). ``const_rows`` is a list of ((b, h, i), value): that
    row of the bias holds `value` for every key (additive, per-head shape only).
    """
    p = dense(B, Sq, Sk, H, Hkv, D, seed, causal=causal, name=f"masked_{kind}_{shape}",
              dtype=dtype)
    rng = _rng(seed + 500)
    full = {"per_head": (B, H, Sq, Sk), "per_batch": (B, 1, Sq, Sk), "2d": (Sq, Sk)}[shape]
    hide = rng.random(size=full) < hide_frac
    hide[..., 0] = False
    if kind == "bool":
        mask = torch.from_numpy(~hide)
    elif kind == "additive":
        bias = rng.standard_normal(size=full).astype(np.float32) * np.float32(bias_std)
        bias[hide] = -np.inf
        for (b, h, i), value in const_rows:
            if shape != "per_head":
                raise ValueError("constant rows need the per-head shape")
            bias[b, h, i, :] = np.float32(value)
        mask = torch.from_numpy(bias).to(torch.bfloat16)
    else:
        raise ValueError(kind)
    p.mask, p.mask_kind = mask, ("bool" if kind == "bool" else "additive")
    p.meta.update(mask_shape=shape, const_rows=list(const_rows))
    return p


def wide_logit(s, seed=None, B=2, S=8192, H=32, D=128, dtype=torch.bfloat16):
    """B2 S8192 H32 D128 non-causal, k = bf16(N(0,1) * s), dout ~ N(0,1)."""
    seed = 3000 + int(s) if seed is None else seed
    p = dense(B, S, S, H, H, D, seed, causal=False, k_mult=float(s), name=f"wide_logit_s{s}",
              dtype=dtype)
    p.meta["k_scale"] = s
    return p


def varlen_gqa(seed=4000, nseq=16, lmin=128, lmax=4096, H=32, Hkv=8, D=128, extra_rows=0,
               lengths=None, causal=True, dtype=torch.bfloat16):
    """Packed THD sequences, total_q = total_k, GQA, causal by default.

    ``extra_rows`` appends rows past cu_seqlens[-1] (their outputs must still be written).
    ``lengths`` overrides the drawn lengths.
    """
    rng = _rng(seed)
    if lengths is None:
        lengths = rng.integers(lmin, lmax + 1, size=nseq)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1]) + int(extra_rows)
    q = _normal(rng, (T, H, D), dtype=dtype)
    k = _normal(rng, (T, Hkv, D), dtype=dtype)
    v = _normal(rng, (T, Hkv, D), dtype=dtype)
    dout = _normal(rng, (T, H, D), dtype=dtype)
    cu_t = torch.from_numpy(cu.copy())
    return Problem(f"varlen_gqa_n{len(lengths)}", q, k, v, dout, causal=causal,
                   cu_seqlens_q=cu_t, cu_seqlens_k=cu_t.clone(),
                   meta=dict(lengths=lengths.tolist(), H=H, Hkv=Hkv, D=D, seed=seed,
                             total=T, covered=int(cu[-1])))


def long_causal(seed=5000, S=61380, H=32, D=128):
    """B1 S61380 H32 D128 causal, q, k, v, dout ~ N(0,1)."""
    p = dense(1, S, S, H, H, D, seed, causal=True, name="long_causal")
    return p


@dataclass
class Fp8Problem:
    """fp8 e4m3 CPU tensors (torch.float8_e4m3fn) with their per-tensor descales."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_descale: float
    k_descale: float
    v_descale: float
    causal: bool = False
    scale: Optional[float] = None

    def decoded(self):
        """q, k, v as float64 NumPy arrays of their e4m3 values (descales not applied)."""
        return tuple(t.to(torch.float64).numpy() for t in (self.q, self.k, self.v))


def _quantise_e4m3(x):
    """float32 array -> (e4m3 tensor, descale) with the largest magnitude mapped to 448."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    d = amax / 448.0 if amax > 0 else 1.0
    return torch.from_numpy(x / np.float32(d)).to(torch.float8_e4m3fn), d


def fp8_dense(B, Sq, Sk, H, Hkv, D, seed, *, causal=False, kind="normal", k_mult=1.0,
              v_ones=False, name=None):
    """Seeded fp8 inputs in BSHD layout. ``k_mult`` multiplies k's descale (the logit
    spread); ``v_ones`` makes every value 1."""
    rng = _rng(seed)
    if kind == "grid":
        qv = rng.integers(-4, 5, size=(B, Sq, H, D)).astype(np.float32) * 0.5
        kv = rng.integers(-4, 5, size=(B, Sk, Hkv, D)).astype(np.float32) * 0.5
        vv = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0], dtype=np.float32), size=(B, Sk, Hkv, D))
        q, k, v = (torch.from_numpy(t).to(torch.float8_e4m3fn) for t in (qv, kv, vv))
        dq = dk = dvs = 1.0
    else:
        q, dq = _quantise_e4m3(rng.standard_normal(size=(B, Sq, H, D), dtype=np.float32))
        k, dk = _quantise_e4m3(rng.standard_normal(size=(B, Sk, Hkv, D), dtype=np.float32))
        v, dvs = _quantise_e4m3(rng.standard_normal(size=(B, Sk, Hkv, D), dtype=np.float32))
    if v_ones:
        v = torch.ones((B, Sk, Hkv, D), dtype=torch.float8_e4m3fn)
        dvs = 1.0
    return Fp8Problem(name or f"fp8_{kind}_b{B}_sq{Sq}_sk{Sk}_h{H}_{Hkv}_d{D}_k{k_mult:g}",
                      q, k, v, dq, dk * k_mult, dvs, causal)
