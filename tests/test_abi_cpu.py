"""C-ABI tests that need no GPU: the library loads, exports every declared symbol, its
struct layout matches the binding, and every rejection path returns a status before any
HIP call is made (so these run on a machine without a GPU)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from exact_attention_40_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exattn.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(exattn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (exattn_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.exattn_abi_version() == _lib.ABI_VERSION


def test_struct_layout_matches_header():
    """Compile a C probe of the header with gcc and compare sizes and offsets."""
    fields = [f[0] for f in _lib.Problem._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(exattn_problem, {f}));' for f in fields)
    prog = f"""
#include <stdio.h>
#include <stddef.h>
#include "exattn.h"
int main(void) {{
  printf("size %zu\\n", sizeof(exattn_problem));
{body}
  return 0;
}}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    vals = dict(zip(lines[::2], map(int, lines[1::2])))
    assert vals["size"] == ctypes.sizeof(_lib.Problem)
    for f in fields:
        assert vals[f] == getattr(_lib.Problem, f).offset, f


def _problem(**kw):
    p = _lib.Problem()
    p.dtype = 0
    p.batch, p.seqlen_q, p.seqlen_k = 2, 100, 77
    p.heads_q, p.heads_kv, p.head_dim = 4, 2, 128
    p.scale = 0.088
    D, H, Hkv = 128, 4, 2
    p.q_stride[:] = (100 * H * D, H * D, D)
    p.k_stride[:] = (77 * Hkv * D, Hkv * D, D)
    p.v_stride[:] = (77 * Hkv * D, Hkv * D, D)
    p.o_stride[:] = p.q_stride[:]
    p.do_stride[:] = p.q_stride[:]
    p.mask_stride[:] = (0, 0, 0, 1)
    for k, v in kw.items():
        if isinstance(getattr(p, k), ctypes.Array):
            getattr(p, k)[:] = v
        else:
            setattr(p, k, v)
    return p


def test_check_accepts_valid_problem(lib):
    assert lib.exattn_check(ctypes.byref(_problem())) == 0
    assert lib.exattn_check(ctypes.byref(_problem(dtype=1))) == 0   # fp16
    assert lib.exattn_check(ctypes.byref(_problem(head_dim=64, q_stride=(100 * 256, 256, 64),
                                                  k_stride=(77 * 128, 128, 64),
                                                  v_stride=(77 * 128, 128, 64)))) == 0
    assert lib.exattn_bwd_workspace_size(ctypes.byref(_problem())) >= 2 * 2 * 100 * 4 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), 2),                        # an unknown dtype is rejected, not run as bf16
    (dict(dtype=-1), 2),
    (dict(head_dim=96), 3),                    # only 64 and 128
    (dict(head_dim=256), 3),
    (dict(heads_q=6, heads_kv=4), 4),          # not a multiple
    (dict(heads_kv=0), 4),
    (dict(seqlen_q=-1), 4),
    (dict(causal=2), 4),
    (dict(scale=float("nan")), 10),
    (dict(scale=float("inf")), 10),
    (dict(q_stride=(0, 512, 129)), 5),         # head stride not a multiple of 8
    (dict(k_stride=(-8, 256, 128)), 5),
    (dict(mask_kind=3), 7),
    (dict(mask_kind=1), 7),                    # NULL mask
    (dict(mask_kind=1, mask=16, mask_stride=(0, 0, 77, 2)), 7),
    (dict(mask_kind=1, mask=16, mask_stride=(-1, 0, 77, 1)), 7),
    (dict(cu_seqlens_q=4096), 8),              # only one of the pair
    (dict(cu_seqlens_q=4096, cu_seqlens_k=4096, num_seqs=0), 8),
    (dict(cu_seqlens_q=4096, cu_seqlens_k=4096, num_seqs=2, max_seqlen_q=101), 8),
    (dict(cu_seqlens_q=4096, cu_seqlens_k=4096, num_seqs=2, max_seqlen_q=10, max_seqlen_k=10,
          mask_kind=1, mask=16), 7),           # mask + varlen
    # token strides whose 128-row tile span would overflow the kernels' 32-bit offsets
    (dict(q_stride=(0, 1 << 23, 128)), 5),
    (dict(k_stride=(0, 1 << 23, 128)), 5),
    (dict(v_stride=(0, (1 << 23) + 8, 128)), 5),
    (dict(heads_q=65536, heads_kv=1), 4),      # heads * head_dim reaches 2^23
    (dict(fwd_variant=3), 4),                  # per-call tiling selectors
    (dict(fwd_variant=-1), 4),
    (dict(bwd_variant=4), 4),
    (dict(reserved=1), 4),
])
def test_check_rejects(lib, kw, status):
    p = _problem(**kw)
    assert lib.exattn_check(ctypes.byref(p)) == status
    assert lib.exattn_last_error().decode() != ""
    # the entry points reject the same problem before touching the device
    assert lib.exattn_fwd(ctypes.byref(p), 16, 16, 16, 16, 16, None) == status
    assert lib.exattn_bwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 30,
                          None) == status
    assert lib.exattn_bwd_workspace_size(ctypes.byref(p)) == 0


def _fp8(**kw):
    return _problem(**{"dtype": 2, **kw})


def _fwd_fp8(lib, p, q=16, k=16, v=16, ds=(1.0, 1.0, 1.0), out=16, lse=16):
    return lib.exattn_fwd_fp8(ctypes.byref(p), q, k, v, *ds, out, lse, None)


def test_fp8_forward_validation(lib):
    assert lib.exattn_check(ctypes.byref(_fp8())) == 0
    # the 16-bit entry points reject e4m3 problems, the fp8 one rejects 16-bit problems
    assert lib.exattn_fwd(ctypes.byref(_fp8()), 16, 16, 16, 16, 16, None) == 2
    assert lib.exattn_bwd(ctypes.byref(_fp8()), *([16] * 9), 256, 1 << 30, None) == 2
    assert _fwd_fp8(lib, _problem()) == 2
    assert _fwd_fp8(lib, _fp8(head_dim=64, q_stride=(100 * 256, 256, 64), k_stride=(77 * 128, 128, 64),
                              v_stride=(77 * 128, 128, 64))) == 3
    assert _fwd_fp8(lib, _fp8(mask_kind=1, mask=16)) == 7
    assert _fwd_fp8(lib, _fp8(cu_seqlens_q=4096, cu_seqlens_k=4096, num_seqs=1, max_seqlen_q=10,
                              max_seqlen_k=10)) == 8
    assert _fwd_fp8(lib, _fp8(q_stride=(100 * 520, 520, 136))) == 5   # multiple of 8, not 16
    assert _fwd_fp8(lib, _fp8(k_stride=(0, 1 << 24, 128))) == 5
    assert _fwd_fp8(lib, _fp8(), ds=(float("inf"), 1.0, 1.0)) == 10
    assert _fwd_fp8(lib, _fp8(), ds=(1.0, 1.0, float("nan"))) == 10
    assert _fwd_fp8(lib, _fp8(), ds=(1e30, 1e30, 1.0)) == 10          # logit scale overflows
    assert _fwd_fp8(lib, _fp8(), q=None) == 1
    assert _fwd_fp8(lib, _fp8(), q=24) == 6
    assert _fwd_fp8(lib, _fp8(), lse=18) == 6
    assert _fwd_fp8(lib, _fp8(batch=0), q=None, k=None, v=None, out=None, lse=None) == 0


def test_null_and_alignment_rejected_before_launch(lib):
    p = _problem()
    assert lib.exattn_fwd(None, 16, 16, 16, 16, 16, None) == 1
    assert lib.exattn_fwd(ctypes.byref(p), None, 16, 16, 16, 16, None) == 1
    assert lib.exattn_fwd(ctypes.byref(p), 24, 16, 16, 16, 16, None) == 6   # q not 16-aligned
    assert lib.exattn_fwd(ctypes.byref(p), 16, 16, 16, 16, 18, None) == 6   # lse not 4-aligned
    ws = lib.exattn_bwd_workspace_size(ctypes.byref(p))
    args = [16] * 9
    assert lib.exattn_bwd(ctypes.byref(p), *args, 256, ws - 1, None) == 9   # too small
    assert lib.exattn_bwd(ctypes.byref(p), *args, 272, ws, None) == 9       # misaligned
    assert lib.exattn_bwd(ctypes.byref(p), *args, None, ws, None) == 9      # NULL
    assert lib.exattn_bwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, 16, 8, 256, ws, None) == 6


def test_empty_problems_enqueue_nothing(lib):
    """Zero rows: OK without any launch (so this runs without a GPU)."""
    assert lib.exattn_fwd(ctypes.byref(_problem(batch=0)), None, None, None, None, None, None) == 0
    assert lib.exattn_fwd(ctypes.byref(_problem(seqlen_q=0)), None, None, None, None, None, None) == 0
    p = _problem(batch=0)
    assert lib.exattn_bwd(ctypes.byref(p), *([None] * 10), 0, None) == 0


def test_status_strings(lib):
    for code in range(12):
        assert lib.exattn_status_string(code).decode() not in ("", "unknown status")
    assert lib.exattn_status_string(99).decode() == "unknown status"


def test_timing_read_empty(lib):
    assert lib.exattn_timing_enable(1) == 0
    assert lib.exattn_timing_read(None, None, None, 0) == 0
    assert lib.exattn_timing_enable(0) == 0


@pytest.mark.parametrize("kw", [dict(o_stride=(0, 1 << 23, 128)), dict(do_stride=(0, 1 << 24, 128))])
def test_backward_only_strides_rejected(lib, kw):
    """out and dout strides exist only for the backward: it rejects them before any launch."""
    p = _problem(**kw)
    assert lib.exattn_bwd(ctypes.byref(p), *([16] * 9), 256, 1 << 30, None) == 5
    assert lib.exattn_bwd_workspace_size(ctypes.byref(p)) == 0


def test_token_stride_limit_boundary(lib):
    """The largest accepted token stride is 2^23 - 8 elements (a multiple of 8)."""
    big = (1 << 23) - 8
    assert lib.exattn_check(ctypes.byref(_problem(q_stride=(0, big, 128)))) == 0
    assert lib.exattn_check(ctypes.byref(_problem(k_stride=(0, big, 128)))) == 0


def test_variant_is_per_call(lib):
    """Each problem carries its own tiling selection, so the workspace size of one call
    never depends on another thread's choice."""
    ws = {v: lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=v))) for v in (0, 1, 2)}
    # the fused variant also needs the fp32 dQ accumulator [rows_q, H, D]
    assert ws[1] >= ws[0] + 2 * 100 * 4 * 128 * 4
    # the two split variants share the workspace layout
    assert ws[2] == ws[0]
    # fp16 runs the split backward for every variant
    assert lib.exattn_bwd_workspace_size(ctypes.byref(_problem(dtype=1, bwd_variant=1))) == ws[0]
    # the stored-dS variant adds B * H * ceil(Sq / 64) * ceil(Sk / 128) chunks of 16 KiB
    ws3 = lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=3)))
    assert ws3 == ws[0] + 2 * 4 * 2 * 1 * 16384
    # ... for dense layouts only: packed ones run variant 0
    packed = dict(batch=1, seqlen_q=100, seqlen_k=100, num_seqs=2, max_seqlen_q=60,
                  max_seqlen_k=60, cu_seqlens_q=4096, cu_seqlens_k=4096,
                  k_stride=(0, 2 * 128, 128), v_stride=(0, 2 * 128, 128))
    assert (lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=3, **packed))) ==
            lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=0, **packed))))
    # ... and only while dS takes at most 64 GiB: B1 S61380 H32 would need 236 GB
    S, H, D = 61380, 32, 128
    big = dict(batch=1, seqlen_q=S, seqlen_k=S, heads_q=H, heads_kv=H, causal=1,
               q_stride=(S * H * D, H * D, D), k_stride=(S * H * D, H * D, D),
               v_stride=(S * H * D, H * D, D), o_stride=(S * H * D, H * D, D),
               do_stride=(S * H * D, H * D, D))
    assert (lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=3, **big))) ==
            lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=0, **big))))
    # while B2 S8192 H32 stores its 8.6 GB
    S = 8192
    mid = dict(big, batch=2, seqlen_q=S, seqlen_k=S, causal=0,
               q_stride=(S * H * D, H * D, D), k_stride=(S * H * D, H * D, D),
               v_stride=(S * H * D, H * D, D), o_stride=(S * H * D, H * D, D),
               do_stride=(S * H * D, H * D, D))
    assert (lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=3, **mid))) -
            lib.exattn_bwd_workspace_size(ctypes.byref(_problem(bwd_variant=0, **mid)))) == \
        2 * 32 * 128 * 64 * 16384
    for v in (0, 1, 2):
        assert lib.exattn_check(ctypes.byref(_problem(fwd_variant=v))) == 0
    # the fp8 forward has one tiling
    assert lib.exattn_check(ctypes.byref(_problem(dtype=2, fwd_variant=1))) == 4
    assert not hasattr(lib, "exattn_set_variant")


def test_host_cu_seqlens_checks():
    """Host offsets are checked by the binding before anything reaches the library: start
    at 0, non-decreasing, end within the packed rows, and a given max_seqlen may not be
    below the longest sequence (its rows past max_seqlen would not be computed)."""
    from exact_attention_40_amd import api
    assert api._host_cu_longest([0, 3, 3, 10], 10, "cu_seqlens_q", None) == 7
    assert api._host_cu_longest([0, 3, 3, 10], 12, "cu_seqlens_q", 9) == 7
    for c, total, given in (([1, 3], 5, None), ([0, 4, 3], 5, None), ([0, 6], 5, None),
                            ([0, 3, 10], 10, 6)):
        with pytest.raises(ValueError):
            api._host_cu_longest(c, total, "cu_seqlens_q", given)


def test_noalloc_rejects_oversize_before_any_device_call(lib):
    """The allocation-free backward holds at most EXATTN_NOALLOC_MAX_WORKSPACE bytes of
    workspace; a larger problem is rejected before any HIP call (so this runs without a
    GPU), and invalid problems are rejected as by exattn_bwd."""
    D, H = 128, 32
    p = _problem(batch=64, seqlen_q=8192, seqlen_k=8192, heads_q=H, heads_kv=H,
                 q_stride=(8192 * H * D, H * D, D), k_stride=(8192 * H * D, H * D, D),
                 v_stride=(8192 * H * D, H * D, D), o_stride=(8192 * H * D, H * D, D),
                 do_stride=(8192 * H * D, H * D, D))
    assert lib.exattn_bwd_workspace_size(ctypes.byref(p)) > _lib.NOALLOC_MAX_WORKSPACE
    assert lib.exattn_bwd_noalloc(ctypes.byref(p), *([16] * 9), None) == 9
    assert b"exattn_bwd_noalloc holds at most" in lib.exattn_last_error()
    assert lib.exattn_bwd_noalloc(ctypes.byref(_problem(head_dim=96)), *([16] * 9), None) == 3
    assert lib.exattn_bwd_noalloc(None, *([16] * 9), None) == 1
