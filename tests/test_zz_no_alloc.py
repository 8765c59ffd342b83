"""The allocation-free backward (exattn_bwd_noalloc, for callers that cannot allocate)
against exattn_bwd, called through the C ABI: same outputs on consecutive calls that
share the library's workspace array, each smaller than the one before, and a problem too
large for the array is rejected."""

import pytest
import torch

from exact_attention_40_amd import _lib, api, workloads
from gpu_util import gpu_inputs, say

pytestmark = pytest.mark.gpu


def _both(p, variant=0):
    q, k, v, do, kw = gpu_inputs(p)
    kw["variant"] = variant
    if p.varlen:   # device offsets, so the binding converts nothing
        kw = dict(kw, cu_seqlens_q=p.cu_seqlens_q.cuda(), cu_seqlens_k=p.cu_seqlens_k.cuda(),
                  max_seqlen_q=int((p.cu_seqlens_q[1:] - p.cu_seqlens_q[:-1]).max()),
                  max_seqlen_k=int((p.cu_seqlens_k[1:] - p.cu_seqlens_k[:-1]).max()))
    if p.mask is not None and p.mask.dtype == torch.bool:
        kw["mask"] = kw["mask"].to(torch.uint8).bool()
    fkw = {n: x for n, x in kw.items() if n != "variant"}
    out, lse = api.exattn_fwd(q, k, v, **fkw)
    ref = api.exattn_bwd(q, k, v, out, do, lse, **kw)
    got = [torch.full_like(t, float("nan")) for t in ref]
    api.exattn_bwd_noalloc(q, k, v, out, do, lse, *got, **kw)
    torch.cuda.synchronize()
    return ref, got


CASES = [
    ("dense B2 S1000 H4 Hkv2 D128 causal",
     lambda: workloads.dense(2, 1000, 1000, 4, 2, 128, seed=9001, causal=True)),
    ("packed 5 sequences H4 Hkv2 D128 causal",
     lambda: workloads.varlen_gqa(seed=9002, lengths=[300, 17, 512, 1, 129], H=4, Hkv=2,
                                  extra_rows=9)),
    ("dense B1 S200 H2 D64 additive mask",
     lambda: workloads.masked(1, 200, 150, 2, 1, 64, seed=9003, kind="additive", shape="per_head")),
    ("dense B1 S70 H1 D128",
     lambda: workloads.dense(1, 70, 33, 1, 1, 128, seed=9004)),
]


def test_noalloc_matches_bwd_on_consecutive_calls():
    """Four calls in a row on one stream, each smaller than the one before (the first two
    leave their Delta, lse2 and sequence ranking in the shared array): every output equals
    exattn_bwd's bit for bit (same kernels, fixed summation order)."""
    for name, make in CASES:
        ref, got = _both(make())
        for n, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(b).all(), (name, n)
            assert torch.equal(a, b), (name, n, float((a.float() - b.float()).abs().max()))
        say(f"  noalloc == bwd: {name}")


def test_noalloc_stored_ds_variant():
    """Backward variant 3 keeps dS in the workspace: through the array too, when it fits
    (16 MB here, then a smaller problem); bit for bit exattn_bwd's outputs."""
    for name, make in (("dense B2 S1000 H4 Hkv2 D128 causal",
                        lambda: workloads.dense(2, 1000, 1000, 4, 2, 128, seed=9011, causal=True)),
                       ("dense B1 S300 H2 Hkv1 D64",
                        lambda: workloads.dense(1, 300, 260, 2, 1, 64, seed=9012))):
        ref, got = _both(make(), variant=3)
        for n, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(b).all(), (name, n)
            assert torch.equal(a, b), (name, n, float((a.float() - b.float()).abs().max()))
        say(f"  noalloc == bwd, stored dS: {name}")


def test_noalloc_rejects_problem_beyond_the_array():
    """131072 query rows x 40 heads need 42 MB of Delta and lse2, more than the array holds:
    rejected with EXATTN_ERR_WORKSPACE before any launch. Inputs are stride-0 views."""
    S, H, D = 131072, 40, 64
    q = torch.zeros(1, 1, H, D, dtype=torch.bfloat16, device="cuda").expand(1, S, H, D)
    k = torch.zeros(1, 64, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, H, S, dtype=torch.float32, device="cuda")
    dq = torch.empty(1, S, H, D, dtype=torch.bfloat16, device="cuda")
    assert api.workspace_size(q, k, k) > _lib.NOALLOC_MAX_WORKSPACE
    with pytest.raises(ValueError, match="holds at most"):
        api.exattn_bwd_noalloc(q, k, k, q, q, lse, dq, torch.empty_like(k), torch.empty_like(k))
