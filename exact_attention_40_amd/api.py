"""Python boundary over libexattn: argument marshalling and stream-ordered allocation.

Every step of the computation runs in the library's HIP kernels; this module only checks
the cross-tensor contract, allocates outputs with torch on the launch stream and passes raw
pointers. The contract follows NVIDIA cudnn-frontend PR #429 ("Fix stream-ordering and
input-validation holes in the SM100 DSA backward interface"): the stream is resolved first
and every allocation, copy and clear happens on it; companion tensors are checked against
q's shape and device; only bf16 is accepted; non-contiguous inputs are normalised on the
stream, outputs are always fresh contiguous tensors.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = ["exattn_fwd", "exattn_fwd_fp8", "exattn_bwd", "exattn_bwd_noalloc", "exattn_check", "attn_fwd", "attn_bwd", "attention",
           "AttnFunction", "timing_enable", "timing_read", "workspace_size"]


def _fail(lib, status):
    msg = _lib.status_message(lib, status)
    if status == _lib.ERR_HIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _norm(t: torch.Tensor) -> torch.Tensor:
    """Head dim contiguous, other strides multiples of 8 elements, 16-byte aligned."""
    ok = (t.stride(-1) == 1 and all(s % 8 == 0 for s in t.stride()[:-1])
          and t.data_ptr() % 16 == 0)
    return t if ok else t.contiguous()


_DTYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.float16: _lib.DTYPE_FP16}


def _strides3(t: torch.Tensor, varlen: bool):
    if varlen:  # [T, H, D]
        return (0, t.stride(0), t.stride(1))
    return (t.stride(0), t.stride(1), t.stride(2))


class _Spec:
    """Validated shapes and options of one call."""

    def __init__(self, q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, fwd_variant=0, bwd_variant=0):
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not isinstance(t, torch.Tensor):
                raise ValueError(f"{name} must be a tensor")
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on a GPU device, got {t.device}")
            if t.device != q.device:
                raise ValueError(f"{name} is on {t.device}, q is on {q.device}")
            if t.dtype not in _DTYPES:
                raise ValueError(f"{name} has dtype {t.dtype}; torch.bfloat16 or torch.float16 "
                                 "is supported")
            if t.dtype != q.dtype:
                raise ValueError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
        self.dtype = q.dtype
        self.varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
        if self.varlen:
            if cu_seqlens_q is None or cu_seqlens_k is None:
                raise ValueError("cu_seqlens_q and cu_seqlens_k must be given together")
            if mask is not None:
                raise ValueError("a mask cannot be combined with cu_seqlens")
            if q.dim() != 3 or k.dim() != 3:
                raise ValueError("packed q/k/v must be [tokens, heads, head_dim]")
            Tq, H, D = q.shape
            Tk, Hkv, Dk = k.shape
            self.batch, self.sq, self.sk = 1, Tq, Tk
        else:
            if q.dim() != 4 or k.dim() != 4:
                raise ValueError("q/k/v must be [batch, seq, heads, head_dim]")
            B, Sq, H, D = q.shape
            Bk, Sk, Hkv, Dk = k.shape
            if Bk != B:
                raise ValueError(f"k batch {Bk} != q batch {B}")
            self.batch, self.sq, self.sk = B, Sq, Sk
        if tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"v shape {tuple(v.shape)} != k shape {tuple(k.shape)}")
        if Dk != D:
            raise ValueError(f"k head_dim {Dk} != q head_dim {D}")
        if Hkv < 1 or H % Hkv != 0:
            raise ValueError(f"heads_q={H} must be a multiple of heads_kv={Hkv}")
        self.H, self.Hkv, self.D = H, Hkv, D
        self.causal = bool(causal)
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        if not math.isfinite(self.scale):
            raise ValueError("scale must be finite")
        self.mask = mask
        self.cu_q, self.cu_k = cu_seqlens_q, cu_seqlens_k
        self.max_q, self.max_k = max_seqlen_q, max_seqlen_k
        self.fwd_variant, self.bwd_variant = int(fwd_variant), int(bwd_variant)

    @property
    def q_shape(self):
        return ((self.sq, self.H, self.D) if self.varlen
                else (self.batch, self.sq, self.H, self.D))

    @property
    def lse_shape(self):
        return (self.H, self.sq) if self.varlen else (self.batch, self.H, self.sq)

    def prepare_side_inputs(self, device):
        """Mask and cu_seqlens as device tensors (called inside the stream context)."""
        mask_kind, mask_t, mask_stride = _lib.MASK_NONE, None, (0, 0, 0, 1)
        if self.mask is not None:
            m = self.mask
            if not isinstance(m, torch.Tensor):
                raise ValueError("mask must be a tensor")
            if m.device != device:
                raise ValueError(f"mask is on {m.device}, q is on {device}")
            if m.dtype == torch.bool:
                mask_kind = _lib.MASK_BOOL_U8
                m = m.to(torch.uint8)
            elif m.dtype == torch.bfloat16:
                mask_kind = _lib.MASK_ADD_BF16
            else:
                raise ValueError(f"mask dtype {m.dtype}: use torch.bool or an additive torch.bfloat16")
            if m.dim() > 4 or m.dim() < 2:
                raise ValueError("mask must have 2 to 4 dimensions")
            while m.dim() < 4:
                m = m.unsqueeze(0)
            try:
                m = torch.broadcast_to(m, (self.batch, self.H, self.sq, self.sk))
            except RuntimeError as e:
                raise ValueError(f"mask shape {tuple(self.mask.shape)} does not broadcast to "
                                 f"{(self.batch, self.H, self.sq, self.sk)}") from e
            if m.stride(-1) != 1 and self.sk > 1:
                m = m.contiguous()
            mask_t = m
            mask_stride = tuple(m.stride()[:3]) + (1,)
        cu_q = cu_k = None
        nseq = 0
        max_q, max_k = self.max_q, self.max_k
        if self.varlen:
            tensors = []
            for name, cu, total in (("cu_seqlens_q", self.cu_q, self.sq),
                                    ("cu_seqlens_k", self.cu_k, self.sk)):
                if not isinstance(cu, torch.Tensor) or cu.dim() != 1 or cu.numel() < 2:
                    raise ValueError(f"{name} must be a 1-D tensor with at least 2 entries")
                if cu.dtype != torch.int32:
                    raise ValueError(f"{name} must be int32")
                if cu.device.type == "cpu":
                    given = max_q if name == "cu_seqlens_q" else max_k
                    longest = _host_cu_longest(cu.tolist(), total, name, given)
                    if name == "cu_seqlens_q":
                        max_q = longest if max_q is None else max_q
                    else:
                        max_k = longest if max_k is None else max_k
                    cu = cu.to(device, non_blocking=False)
                elif cu.device != device:
                    raise ValueError(f"{name} is on {cu.device}, q is on {device}")
                tensors.append(cu.contiguous())
            cu_q, cu_k = tensors
            if cu_q.numel() != cu_k.numel():
                raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
            nseq = cu_q.numel() - 1
            if max_q is None or max_k is None:
                raise ValueError("max_seqlen_q/max_seqlen_k are required with device cu_seqlens")
        return mask_kind, mask_t, mask_stride, cu_q, cu_k, nseq, max_q, max_k

    def problem(self, q, k, v, side, out=None, dout=None):
        mask_kind, mask_t, mask_stride, cu_q, cu_k, nseq, max_q, max_k = side
        p = _lib.Problem()
        p.dtype = _DTYPES[self.dtype]
        p.batch = self.batch
        p.seqlen_q, p.seqlen_k = self.sq, self.sk
        p.heads_q, p.heads_kv, p.head_dim = self.H, self.Hkv, self.D
        p.causal = int(self.causal)
        p.scale = self.scale
        p.mask_kind = mask_kind
        p.q_stride[:] = _strides3(q, self.varlen)
        p.k_stride[:] = _strides3(k, self.varlen)
        p.v_stride[:] = _strides3(v, self.varlen)
        if out is not None:
            p.o_stride[:] = _strides3(out, self.varlen)
        if dout is not None:
            p.do_stride[:] = _strides3(dout, self.varlen)
        p.mask_stride[:] = mask_stride
        p.mask = mask_t.data_ptr() if mask_t is not None else None
        p.cu_seqlens_q = cu_q.data_ptr() if cu_q is not None else None
        p.cu_seqlens_k = cu_k.data_ptr() if cu_k is not None else None
        p.num_seqs = nseq
        p.max_seqlen_q = max_q or 0
        p.max_seqlen_k = max_k or 0
        p.fwd_variant = self.fwd_variant
        p.bwd_variant = self.bwd_variant
        return p


def _host_cu_longest(c, total, name, given):
    """Check host cu_seqlens offsets `c` against `total` packed rows and return the longest
    sequence. A given max_seqlen below it is rejected: the library would truncate that
    sequence (include/exattn.h, packed sequences)."""
    if c[0] != 0 or any(b < a for a, b in zip(c, c[1:])) or c[-1] > total:
        raise ValueError(f"{name} must start at 0, be non-decreasing and end at most at {total}")
    longest = max(b - a for a, b in zip(c, c[1:]))
    if given is not None and given < longest:
        raise ValueError(f"max_seqlen_{name[-1]}={given} is below the longest sequence "
                         f"({longest}): its rows past {given} would not be computed")
    return longest


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def exattn_check(q, k, v, *, causal=False, scale=None, mask=None, cu_seqlens_q=None,
                 cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None) -> bool:
    """Metadata-only support check through the library; raises ValueError if unsupported."""
    lib = _lib.load()
    spec = _Spec(q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k)
    with torch.cuda.device(q.device):
        side = spec.prepare_side_inputs(q.device)
        p = spec.problem(_norm(q), _norm(k), _norm(v), side)
        st = lib.exattn_check(ctypes.byref(p))
    if st != _lib.OK:
        _fail(lib, st)
    return True


def exattn_fwd(q, k, v, *, causal=False, scale=None, mask=None, cu_seqlens_q=None,
               cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, variant=0
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward attention: returns (out, lse).

    Dense: q [B, Sq, H, D], k/v [B, Sk, Hkv, D] -> out [B, Sq, H, D], lse [B, H, Sq] fp32.
    Packed: q [Tq, H, D], k/v [Tk, Hkv, D] with int32 cu_seqlens -> out [Tq, H, D],
    lse [H, Tq]. q, k, v are bf16 or fp16 (all the same); out has their dtype.
    mask: bool (True = attend) or additive bf16 (for either input dtype), broadcastable to
    [B, H, Sq, Sk]. lse is the natural-log log-sum-exp; empty rows give out 0, lse -inf.
    variant: the forward tiling for this call (fwd_variant in include/exattn.h).
    """
    lib = _lib.load()
    spec = _Spec(q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k, fwd_variant=variant)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device)
        with torch.cuda.stream(stream):
            side = spec.prepare_side_inputs(q.device)
            qn, kn, vn = _norm(q), _norm(k), _norm(v)
            out = torch.empty(spec.q_shape, dtype=spec.dtype, device=q.device)
            lse = torch.empty(spec.lse_shape, dtype=torch.float32, device=q.device)
            p = spec.problem(qn, kn, vn, side)
            st = lib.exattn_fwd(ctypes.byref(p), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(out),
                                _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if st != _lib.OK:
        _fail(lib, st)
    return out, lse


def _norm_fp8(t: torch.Tensor) -> torch.Tensor:
    """Head dim contiguous, other strides multiples of 16 elements, 16-byte aligned."""
    ok = (t.stride(-1) == 1 and all(s % 16 == 0 for s in t.stride()[:-1])
          and t.data_ptr() % 16 == 0)
    return t if ok else t.contiguous()


def exattn_fwd_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, *, causal=False,
                   scale=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp8 forward: q [B, Sq, H, 128], k/v [B, Sk, Hkv, 128] as torch.float8_e4m3fn with one
    descale per tensor (the represented values are q * q_descale, ...). Returns out
    [B, Sq, H, 128] bf16 and lse [B, H, Sq] fp32 (natural log). The softmax walks key tiles
    with a bounded rebase of its running max and rounds P to e4m3 for the P.V product (see
    exattn_fwd_fp8 in include/exattn.h)."""
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's GPU device, got {t.device}")
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError(f"{name} has dtype {t.dtype}; the fp8 forward takes torch.float8_e4m3fn")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, seq, heads, head_dim]")
    B, Sq, H, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shapes q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)} do not match")
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"heads_q={H} must be a multiple of heads_kv={Hkv}")
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    for name, x in (("scale", sc), ("q_descale", q_descale), ("k_descale", k_descale),
                    ("v_descale", v_descale)):
        if not math.isfinite(float(x)):
            raise ValueError(f"{name} must be finite")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device)
        with torch.cuda.stream(stream):
            qn, kn, vn = _norm_fp8(q), _norm_fp8(k), _norm_fp8(v)
            out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q.device)
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
            p = _lib.Problem()
            p.dtype = _lib.DTYPE_FP8_E4M3
            p.batch, p.seqlen_q, p.seqlen_k = B, Sq, Sk
            p.heads_q, p.heads_kv, p.head_dim = H, Hkv, D
            p.causal = int(bool(causal))
            p.scale = sc
            p.mask_kind = _lib.MASK_NONE
            p.q_stride[:] = _strides3(qn, False)
            p.k_stride[:] = _strides3(kn, False)
            p.v_stride[:] = _strides3(vn, False)
            st = lib.exattn_fwd_fp8(ctypes.byref(p), _ptr(qn), _ptr(kn), _ptr(vn),
                                    float(q_descale), float(k_descale), float(v_descale),
                                    _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if st != _lib.OK:
        _fail(lib, st)
    return out, lse


def workspace_size(q, k, v, **kw) -> int:
    """Bytes of workspace exattn_bwd uses for these inputs."""
    lib = _lib.load()
    spec = _Spec(q, k, v, kw.get("causal", False), kw.get("scale"), kw.get("mask"),
                 kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"), kw.get("max_seqlen_q"),
                 kw.get("max_seqlen_k"), bwd_variant=kw.get("variant", 0))
    with torch.cuda.device(q.device):
        side = spec.prepare_side_inputs(q.device)
        p = spec.problem(_norm(q), _norm(k), _norm(v), side, out=_norm(q), dout=_norm(q))
        return int(lib.exattn_bwd_workspace_size(ctypes.byref(p)))


def exattn_bwd(q, k, v, out, dout, lse, *, causal=False, scale=None, mask=None,
               cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
               variant=0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward attention: returns (dq, dk, dv) for the same options as the forward.

    out and lse must be the forward's outputs for these inputs; dout = dL/dout.
    variant: the backward kernels for this call (bwd_variant in include/exattn.h).
    """
    lib = _lib.load()
    spec = _Spec(q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k, bwd_variant=variant)
    for name, t in (("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != spec.q_shape:
            raise ValueError(f"{name} must have q's shape {spec.q_shape}, got "
                             f"{None if not isinstance(t, torch.Tensor) else tuple(t.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q is on {q.device}")
        if t.dtype != spec.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}; q has {spec.dtype}")
    if not isinstance(lse, torch.Tensor) or tuple(lse.shape) != spec.lse_shape:
        raise ValueError(f"lse must have shape {spec.lse_shape}, got "
                         f"{None if not isinstance(lse, torch.Tensor) else tuple(lse.shape)}")
    if lse.device != q.device or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device)
        with torch.cuda.stream(stream):
            side = spec.prepare_side_inputs(q.device)
            qn, kn, vn, on, don = _norm(q), _norm(k), _norm(v), _norm(out), _norm(dout)
            lsen = lse.contiguous()
            dq = torch.empty(spec.q_shape, dtype=spec.dtype, device=q.device)
            dk = torch.empty(tuple(k.shape), dtype=spec.dtype, device=q.device)
            dv = torch.empty(tuple(v.shape), dtype=spec.dtype, device=q.device)
            p = spec.problem(qn, kn, vn, side, out=on, dout=don)
            ws_bytes = int(lib.exattn_bwd_workspace_size(ctypes.byref(p)))
            ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=q.device)
            ws_ptr = (ws.data_ptr() + 255) // 256 * 256
            st = lib.exattn_bwd(ctypes.byref(p), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(on),
                                _ptr(don), _ptr(lsen), _ptr(dq), _ptr(dk), _ptr(dv),
                                ws_ptr if ws_bytes else None, ws_bytes,
                                ctypes.c_void_p(stream.cuda_stream))
    if st != _lib.OK:
        _fail(lib, st)
    return dq, dk, dv


def exattn_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, *, causal=False, scale=None,
                       mask=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                       max_seqlen_k=None, variant=0) -> None:
    """Backward into caller-provided dq, dk, dv through exattn_bwd_noalloc, whose workspace
    is a library-owned device array (include/exattn.h): the C call allocates nothing. The
    tensors must already be in an accepted layout (head_dim contiguous, strides multiples of
    8 elements, 16-byte aligned; dq/dk/dv contiguous), since a copy here would allocate;
    a bool mask or host cu_seqlens still cost a conversion, so pass a uint8 mask and device
    offsets with max_seqlen to keep the whole call allocation-free."""
    lib = _lib.load()
    spec = _Spec(q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k, bwd_variant=variant)
    for name, t, shape in (("out", out, spec.q_shape), ("dout", dout, spec.q_shape),
                           ("dq", dq, spec.q_shape), ("dk", dk, tuple(k.shape)),
                           ("dv", dv, tuple(v.shape))):
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != shape or t.dtype != spec.dtype:
            raise ValueError(f"{name} must be a {spec.dtype} tensor of shape {shape}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q is on {q.device}")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if _norm(t) is not t:
            raise ValueError(f"{name} is not in an accepted layout; a copy would allocate")
    if (not isinstance(lse, torch.Tensor) or tuple(lse.shape) != spec.lse_shape
            or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {spec.lse_shape}")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device)
        with torch.cuda.stream(stream):
            side = spec.prepare_side_inputs(q.device)
            p = spec.problem(q, k, v, side, out=out, dout=dout)
            st = lib.exattn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                        ctypes.c_void_p(stream.cuda_stream))
    if st != _lib.OK:
        _fail(lib, st)


attn_fwd = exattn_fwd
attn_bwd = exattn_bwd


class AttnFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves (q, k, v, out, lse); backward recomputes P."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, scale=None, mask=None, cu_seqlens_q=None,
                cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None):
        kw = dict(causal=causal, scale=scale, mask=mask, cu_seqlens_q=cu_seqlens_q,
                  cu_seqlens_k=cu_seqlens_k, max_seqlen_q=max_seqlen_q,
                  max_seqlen_k=max_seqlen_k)
        out, lse = exattn_fwd(q, k, v, **kw)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.kw = kw
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = exattn_bwd(q, k, v, out, dout, lse, **ctx.kw)
        return dq, dk, dv, None, None, None, None, None, None, None


def attention(q, k, v, causal=False, scale=None, mask=None, cu_seqlens_q=None,
              cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None):
    """Differentiable attention output (in q's dtype, bf16 or fp16)."""
    return AttnFunction.apply(q, k, v, causal, scale, mask, cu_seqlens_q, cu_seqlens_k,
                              max_seqlen_q, max_seqlen_k)


def timing_enable(on: bool = True):
    _lib.load().exattn_timing_enable(1 if on else 0)


def timing_read():
    """{kernel name: (total ms, launches)} recorded since the last read."""
    lib = _lib.load()
    n = 16
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    k = lib.exattn_timing_read(names, ms, cnt, n)
    if k < 0:
        raise RuntimeError("exattn_timing_read failed")
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k)}
