"""Robustness of the HIP path: no dependence on prior buffer contents, stream ordering
under a busy ambient stream, run-to-run determinism, the masked zero-key padding
invariant, and the boundary contract (rejections instead of silent wrong results)."""

import numpy as np
import pytest
import torch

from exact_attention_40_amd import api, workloads
from gpu_util import compare, gpu_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _fill_allocator(value, nbytes=1 << 28):
    """Hand the caching allocator blocks full of `value` so later tensors start dirty."""
    junk = [torch.full((nbytes // 4 // 8,), value, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    del junk


@pytest.mark.parametrize("causal", [False, True])
def test_garbage_prefill_gives_identical_results(causal):
    """Outputs never depend on what the allocator held (flash-dmattn PR #122, "Root
    Cause" 1; PFCCLab cudnn-frontend PR #9, "Other checks": leak probe)."""
    p = workloads.dense(2, 700, 900, 4, 2, 128, seed=11, causal=causal)
    _fill_allocator(0.0)
    a = run_gpu(p)
    _fill_allocator(float("nan"))
    b = run_gpu(p)
    _fill_allocator(float("inf"))
    c = run_gpu(p)
    for n in ("out", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]) and torch.equal(a[n], c[n]), n


def test_busy_ambient_stream():
    """The ambient stream is kept busy while the call runs on a side stream
    (cudnn-frontend PR #429, first commit message: zero-fills must be ordered with the
    kernel on the launch stream); results equal a quiet run."""
    p = workloads.dense(1, 512, 640, 4, 4, 128, seed=12)
    q, k, v, do, kw = gpu_inputs(p)
    torch.cuda.synchronize()
    out0, lse0 = api.exattn_fwd(q, k, v, **kw)
    g0 = api.exattn_bwd(q, k, v, out0, do, lse0, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for _ in range(3):
        torch.cuda._sleep(200_000_000)          # ambient stream busy
        with torch.cuda.stream(side):
            out1, lse1 = api.exattn_fwd(q, k, v, **kw)
            g1 = api.exattn_bwd(q, k, v, out1, do, lse1, **kw)
        side.synchronize()
        assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
        for a, b in zip(g0, g1):
            assert torch.equal(a, b)
        assert torch.count_nonzero(g1[1]) > 0
    torch.cuda.synchronize()


def test_forward_and_backward_bit_deterministic():
    """Forward bit-identical over 60 repeats (PFCCLab cudnn-frontend PR #9, "Other
    checks"); the default backward sums every output in a fixed order (dK/dV per key
    block, dQ per query block, all in registers), so dq, dk, dv are bit-identical too."""
    p = workloads.padded_tile(392, 392, mask_kind="bool", seed=2500)
    q, k, v, do, kw = gpu_inputs(p)
    out0, lse0 = api.exattn_fwd(q, k, v, **kw)
    for _ in range(59):
        out, lse = api.exattn_fwd(q, k, v, **kw)
        assert torch.equal(out, out0) and torch.equal(lse, lse0)
    g0 = api.exattn_bwd(q, k, v, out0, do, lse0, **kw)
    for _ in range(8):
        g = api.exattn_bwd(q, k, v, out0, do, lse0, **kw)
        for a, b in zip(g, g0):
            assert torch.equal(a, b)


@pytest.mark.parametrize("kind", ["none", "bool", "additive"])
def test_masked_zero_key_padding_is_invisible(kind):
    """K/V padded with zero keys to the next multiple of 128, hidden by the mask
    (OpenWAM PR #64, "Fix"): out/lse/dq unchanged bit for bit, dk/dv of the real keys
    unchanged, padded keys get exactly zero."""
    Sq, Sk, pad = 100, 77, 128 - 77
    p = workloads.padded_tile(Sq, Sk, mask_kind=kind if kind != "none" else "none", seed=2600)
    q, k, v, do, kw = gpu_inputs(p)
    out, lse = api.exattn_fwd(q, k, v, **kw)
    g = api.exattn_bwd(q, k, v, out, do, lse, **kw)
    kp = torch.cat([k, torch.zeros(2, pad, 4, 128, dtype=k.dtype, device="cuda")], 1)
    vp = torch.cat([v, torch.zeros(2, pad, 4, 128, dtype=v.dtype, device="cuda")], 1)
    if kind == "none":
        m = torch.ones(2, 1, 1, Sk + pad, dtype=torch.bool, device="cuda")
        m[..., Sk:] = False
    elif kind == "bool":
        m = torch.cat([kw["mask"], torch.zeros(2, 1, Sq, pad, dtype=torch.bool, device="cuda")], -1)
    else:
        m = torch.cat([kw["mask"], torch.full((2, 1, Sq, pad), float("-inf"), dtype=torch.bfloat16,
                                              device="cuda")], -1)
    kw2 = dict(kw, mask=m)
    out2, lse2 = api.exattn_fwd(q, kp, vp, **kw2)
    g2 = api.exattn_bwd(q, kp, vp, out2, do, lse2, **kw2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)
    assert torch.equal(g2[1][:, :Sk], g[1]) and torch.equal(g2[2][:, :Sk], g[2])
    assert torch.count_nonzero(g2[1][:, Sk:]) == 0 and torch.count_nonzero(g2[2][:, Sk:]) == 0
    assert torch.equal(g2[0], g[0])


def test_autograd_function_matches_oracle():
    p = workloads.dense(1, 300, 300, 4, 2, 128, seed=13, causal=True)
    q, k, v, do, kw = gpu_inputs(p)
    q.requires_grad_(True), k.requires_grad_(True), v.requires_grad_(True)
    out = api.attention(q, k, v, causal=True)
    out.backward(do)
    torch.cuda.synchronize()
    ref = run_oracle(p)
    res = dict(out=out.detach(), dq=q.grad, dk=k.grad, dv=v.grad)
    compare(res, ref, names=("out", "dq", "dk", "dv"), tag="autograd")


# ------------------------------------------------------------------------------------------
# Contract: rejected, not run (cudnn-frontend PR #429 commit messages; PR #9 item 4)
# ------------------------------------------------------------------------------------------

def _qkv(B=1, S=64, H=2, D=128, dtype=torch.bfloat16, device="cuda"):
    g = torch.Generator(device="cpu").manual_seed(0)
    mk = lambda: torch.randn(B, S, H, D, generator=g).to(dtype).to(device)  # noqa: E731
    return mk(), mk(), mk()


def test_rejects_other_dtypes_and_bad_head_dim():
    """Unsupported inputs are rejected instead of run with the wrong element type
    (cudnn-frontend PR #429, second commit message: an fp16 tensor run as bf16 returns
    silently wrong gradients)."""
    for dt in (torch.float32, torch.float64):
        q, k, v = _qkv(dtype=dt)
        with pytest.raises(ValueError, match="bfloat16 or torch.float16"):
            api.exattn_fwd(q, k, v)
    q, k, v = _qkv(dtype=torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        api.exattn_fwd(q, k.bfloat16(), v)                          # mixed input dtypes
    for D in (96, 100, 112, 192, 256):
        q, k, v = _qkv(D=D)
        with pytest.raises(ValueError, match="head_dim"):
            api.exattn_fwd(q, k, v)


def test_rejects_mis_shaped_companions():
    q, k, v = _qkv(S=96)
    out, lse = api.exattn_fwd(q, k, v)
    do = torch.randn_like(q)
    with pytest.raises(ValueError, match="dout"):
        api.exattn_bwd(q, k, v, out, do.transpose(1, 2), lse)     # transposed dout
    with pytest.raises(ValueError, match="lse"):
        api.exattn_bwd(q, k, v, out, do, lse.transpose(1, 2))     # transposed lse
    with pytest.raises(ValueError):
        api.exattn_bwd(q, k, v, out[:, :50], do, lse)
    with pytest.raises(ValueError):
        api.exattn_fwd(q, k[:, :, :1].repeat(1, 1, 3, 1), v)        # heads not a multiple


def test_rejects_cpu_and_mixed_devices():
    q, k, v = _qkv(device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        api.exattn_fwd(q, k, v)
    qg, kg, vg = _qkv()
    with pytest.raises(ValueError):
        api.exattn_fwd(qg, kg, v)
    with pytest.raises(ValueError):
        api.exattn_fwd(qg, kg, vg, mask=torch.ones(64, 64, dtype=torch.bool))
    say("contract checks ok")


def test_nan_input_propagates_and_stays_local():
    """A NaN in one query row (reading: non-finite inputs propagate, never cleaned): that
    row's out, lse and dq are NaN, every other row's out, lse and dq equal the clean run bit
    for bit, and dk / dv of the KV head the row reads are NaN (the row sees every key). The
    exponent clamp of the backward keeps the NaN (a plain min would turn it into exp2(0))."""
    p = workloads.dense(1, 300, 260, 2, 1, 128, seed=6100)
    q, k, v, do = (t.cuda() for t in (p.q, p.k, p.v, p.dout))
    o0, l0 = api.exattn_fwd(q, k, v)
    g0 = api.exattn_bwd(q, k, v, o0, do, l0)
    qn = q.clone()
    qn[0, 77, 1, 5] = float("nan")
    o1, l1 = api.exattn_fwd(qn, k, v)
    dq1, dk1, dv1 = api.exattn_bwd(qn, k, v, o1, do, l1)
    torch.cuda.synchronize()
    assert torch.isnan(o1[0, 77, 1]).all() and torch.isnan(l1[0, 1, 77]) and torch.isnan(dq1[0, 77, 1]).all()
    keep = torch.ones(o1.shape[:3], dtype=torch.bool, device="cuda")
    keep[0, 77, 1] = False
    assert torch.equal(o1[keep], o0[keep]) and torch.equal(dq1[keep], g0[0][keep])
    lk = torch.ones_like(l1, dtype=torch.bool)
    lk[0, 1, 77] = False
    assert torch.equal(l1[lk], l0[lk])
    assert torch.isnan(dk1).all() and torch.isnan(dv1).all()


@pytest.mark.parametrize("bwd_variant", [0, 3])
def test_graph_capture_replays(bwd_variant):
    """The calls enqueue only kernels (zero-fills included, no memset nodes), so a caller
    may capture them in a HIP graph. Forward, backward and the allocation-free backward are
    captured once and replayed three times, with eager work and a synchronisation between
    the replays; every replay reproduces the eager results bit for bit."""
    p = workloads.dense(2, 300, 260, 4, 2, 128, seed=7301, causal=True)
    q, k, v, do, kw = gpu_inputs(p)
    out, lse = api.exattn_fwd(q, k, v, **kw)
    ref = (out, lse) + tuple(api.exattn_bwd(q, k, v, out, do, lse, variant=bwd_variant, **kw))
    nq = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    api.exattn_bwd_noalloc(q, k, v, out, do, lse, *nq, variant=bwd_variant, **kw)
    torch.cuda.synchronize()
    for a, b in zip(ref[2:], nq):
        assert torch.equal(a, b)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            g_out, g_lse = api.exattn_fwd(q, k, v, **kw)
            g_grads = api.exattn_bwd(q, k, v, g_out, do, g_lse, variant=bwd_variant, **kw)
            api.exattn_bwd_noalloc(q, k, v, g_out, do, g_lse, *nq, variant=bwd_variant, **kw)
    torch.cuda.current_stream().wait_stream(side)
    got = (g_out, g_lse) + tuple(g_grads)
    for rep in range(3):
        for t in got + tuple(nq):
            t.fill_(float("nan"))          # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), (rep, name)
        for name, a, b in zip(("dq", "dk", "dv"), ref[2:], nq):
            assert torch.equal(a, b), (rep, "noalloc " + name)
    say(f"  graph replays match eager (backward variant {bwd_variant})")
