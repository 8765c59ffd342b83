// Host side of libexattn: argument validation, grid sizing and kernel launches.
// Every check runs before the first enqueue; on error nothing is enqueued.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/exattn.h"
#include "params.hpp"

namespace exattn {

const char* kernel_name(KernelId id) {
  switch (id) {
    case KernelId::Fwd: return "exattn_fwd_kernel";
    case KernelId::FwdTail: return "exattn_fwd_tail_kernel";
    case KernelId::Delta: return "exattn_bwd_delta_kernel";
    case KernelId::BwdDkDv: return "exattn_bwd_dkdv_kernel";
    case KernelId::BwdDq: return "exattn_bwd_dq_kernel";
    case KernelId::BwdFused: return "exattn_bwd_fused_kernel";
    case KernelId::DqReduce: return "exattn_bwd_dq_reduce_kernel";
    case KernelId::KvTail: return "exattn_bwd_kv_tail_kernel";
    case KernelId::QTail: return "exattn_bwd_q_tail_kernel";
    case KernelId::Zero: return "exattn_zero_kernel";
    case KernelId::FwdFp8: return "exattn_fwd_fp8_kernel";
    case KernelId::UnitOrder: return "exattn_bwd_unit_order_kernel";
    case KernelId::BwdDqDs: return "exattn_bwd_dq_ds_kernel";
    default: return "unknown";
  }
}

namespace {

thread_local char g_err[512] = "";

exattn_status fail(exattn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// ---- kernel timing (HIP events around each launch) ------------------------------------
struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_event_pool;
std::vector<TimedLaunch> g_launches;
constexpr size_t kMaxTimed = 4096;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct Timer {
  bool on = false;
  TimedLaunch t{};
  Timer(KernelId id, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_timing || g_launches.size() >= kMaxTimed) return;
    t.kernel = (int)id;
    t.start = take_event();
    t.stop = take_event();
    if (!t.start || !t.stop) return;
    on = hipEventRecord(t.start, s) == hipSuccess;
  }
  void done(hipStream_t s) {
    if (!on) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (hipEventRecord(t.stop, s) == hipSuccess) g_launches.push_back(t);
  }
};

template <class F>
hipError_t timed(KernelId id, hipStream_t s, F&& f) {
  Timer tm(id, s);
  hipError_t e = f();
  tm.done(s);
  return e;
}

template <class F>
hipError_t timed_if(bool timing, KernelId id, hipStream_t s, F&& f) {
  return timing ? timed(id, s, f) : f();
}

// ---- validation --------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides are in elements; rows must start on 16-byte boundaries (8 elements of 2 bytes,
// 16 of 1 byte).
// Token strides are bounded so that a tile of up to 128 rows stays inside the kernels'
// 32-bit buffer offsets (`max_token` elements).
exattn_status check_strides(const int64_t* st, bool varlen, const char* name, int mult,
                            int64_t max_token) {
  for (int i = varlen ? 1 : 0; i < 3; ++i) {
    if (st[i] < 0 || (st[i] % mult) != 0)
      return fail(EXATTN_ERR_STRIDE, "%s stride[%d] = %lld must be a non-negative multiple of %d",
                  name, i, (long long)st[i], mult);
  }
  if (st[1] >= max_token)
    return fail(EXATTN_ERR_STRIDE, "%s token stride %lld must be below %lld elements", name,
                (long long)st[1], (long long)max_token);
  return EXATTN_OK;
}

constexpr int64_t kMaxTokenStride16 = int64_t(1) << 23;  // 16-bit inputs
constexpr int64_t kMaxTokenStride8 = int64_t(1) << 24;   // fp8 inputs (64-row tiles)

// bwd: also check the out/dout strides. fp8: the problem of exattn_fwd_fp8 (e4m3 inputs,
// head_dim 128, dense, no mask).
exattn_status validate(const exattn_problem* p, bool bwd, bool fp8 = false) {
  if (!p) return fail(EXATTN_ERR_NULL, "problem pointer is NULL");
  if (fp8) {
    if (p->dtype != EXATTN_DTYPE_FP8_E4M3)
      return fail(EXATTN_ERR_DTYPE, "dtype %d: the fp8 forward takes EXATTN_DTYPE_FP8_E4M3 (2)", p->dtype);
    if (p->head_dim != 128)
      return fail(EXATTN_ERR_HEAD_DIM, "head_dim %d: the fp8 forward supports 128 only", p->head_dim);
    if (p->cu_seqlens_q || p->cu_seqlens_k)
      return fail(EXATTN_ERR_VARLEN, "the fp8 forward takes dense (batch) inputs only");
    if (p->mask_kind != EXATTN_MASK_NONE)
      return fail(EXATTN_ERR_MASK, "the fp8 forward takes no mask (causal only)");
  } else {
    if (p->dtype != EXATTN_DTYPE_BF16 && p->dtype != EXATTN_DTYPE_FP16)
      return fail(EXATTN_ERR_DTYPE, "dtype %d is not supported: bf16 (0) or fp16 (1)", p->dtype);
  }
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(EXATTN_ERR_HEAD_DIM, "head_dim %d is not supported: only 64 and 128", p->head_dim);
  if (p->heads_q < 1 || p->heads_kv < 1 || p->heads_q % p->heads_kv != 0)
    return fail(EXATTN_ERR_SHAPE, "heads_q=%d must be a positive multiple of heads_kv=%d",
                p->heads_q, p->heads_kv);
  if (p->seqlen_q < 0 || p->seqlen_k < 0)
    return fail(EXATTN_ERR_SHAPE, "negative sequence length");
  if (p->causal != 0 && p->causal != 1) return fail(EXATTN_ERR_SHAPE, "causal must be 0 or 1");
  if (p->reserved != 0) return fail(EXATTN_ERR_SHAPE, "reserved must be 0");
  if (fp8 && (p->fwd_variant != 0 || p->bwd_variant != 0))
    return fail(EXATTN_ERR_SHAPE, "the fp8 forward has one tiling: fwd_variant and bwd_variant must be 0");
  if (p->fwd_variant < 0 || p->fwd_variant > 2)
    return fail(EXATTN_ERR_SHAPE, "unknown fwd_variant %d (0, 1 or 2)", p->fwd_variant);
  if (p->bwd_variant < 0 || p->bwd_variant > 3)
    return fail(EXATTN_ERR_SHAPE, "unknown bwd_variant %d (0, 1, 2 or 3)", p->bwd_variant);
  if ((int64_t)p->heads_q * p->head_dim >= kMaxTokenStride16 ||
      (int64_t)p->heads_kv * p->head_dim >= kMaxTokenStride16)
    return fail(EXATTN_ERR_SHAPE, "heads * head_dim must be below 2^23 elements");
  if (!std::isfinite(p->scale)) return fail(EXATTN_ERR_SCALE, "scale must be finite");
  const bool varlen = p->cu_seqlens_q != nullptr || p->cu_seqlens_k != nullptr;
  if (varlen) {
    if (!p->cu_seqlens_q || !p->cu_seqlens_k)
      return fail(EXATTN_ERR_VARLEN, "cu_seqlens_q and cu_seqlens_k must both be given");
    if (p->num_seqs < 1) return fail(EXATTN_ERR_VARLEN, "num_seqs must be >= 1");
    if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
      return fail(EXATTN_ERR_VARLEN, "max_seqlen must be >= 0");
    if (p->max_seqlen_q > p->seqlen_q || p->max_seqlen_k > p->seqlen_k)
      return fail(EXATTN_ERR_VARLEN, "max_seqlen exceeds the packed row count");
    if (p->mask_kind != EXATTN_MASK_NONE)
      return fail(EXATTN_ERR_MASK, "a mask cannot be combined with cu_seqlens");
  } else {
    if (p->batch < 0) return fail(EXATTN_ERR_SHAPE, "negative batch");
  }
  if (p->mask_kind < EXATTN_MASK_NONE || p->mask_kind > EXATTN_MASK_ADD_BF16)
    return fail(EXATTN_ERR_MASK, "unknown mask kind %d", p->mask_kind);
  if (p->mask_kind != EXATTN_MASK_NONE) {
    if (!p->mask) return fail(EXATTN_ERR_MASK, "mask pointer is NULL");
    for (int i = 0; i < 3; ++i)
      if (p->mask_stride[i] < 0) return fail(EXATTN_ERR_MASK, "negative mask stride");
    if (p->mask_stride[3] != 1) return fail(EXATTN_ERR_MASK, "mask key stride must be 1");
    if (p->mask_kind == EXATTN_MASK_ADD_BF16 && (reinterpret_cast<uintptr_t>(p->mask) & 1u))
      return fail(EXATTN_ERR_ALIGN, "bf16 mask pointer must be 2-byte aligned");
  }
  exattn_status s;
  const int mult = fp8 ? 16 : 8;
  const int64_t mt = fp8 ? kMaxTokenStride8 : kMaxTokenStride16;
  if ((s = check_strides(p->q_stride, varlen, "q", mult, mt)) != EXATTN_OK) return s;
  if ((s = check_strides(p->k_stride, varlen, "k", mult, mt)) != EXATTN_OK) return s;
  if ((s = check_strides(p->v_stride, varlen, "v", mult, mt)) != EXATTN_OK) return s;
  if (bwd) {
    if ((s = check_strides(p->o_stride, varlen, "out", 8, mt)) != EXATTN_OK) return s;
    if ((s = check_strides(p->do_stride, varlen, "dout", 8, mt)) != EXATTN_OK) return s;
  }
  // Size limits: row counts times heads must index within int32 rows, blocks within 2^31.
  const int64_t rows_q = varlen ? (int64_t)p->seqlen_q : (int64_t)p->batch * p->seqlen_q;
  const int64_t rows_k = varlen ? (int64_t)p->seqlen_k : (int64_t)p->batch * p->seqlen_k;
  if (rows_q > INT32_MAX || rows_k > INT32_MAX || rows_q * p->heads_q > INT32_MAX ||
      rows_k * p->heads_kv > INT32_MAX)
    return fail(EXATTN_ERR_SHAPE, "problem too large");
  return EXATTN_OK;
}

struct Geometry {
  bool varlen;
  int units;
  int64_t rows_q, rows_k;
};

Geometry geometry(const exattn_problem* p) {
  Geometry g;
  g.varlen = p->cu_seqlens_q != nullptr;
  g.units = g.varlen ? p->num_seqs : p->batch;
  g.rows_q = g.varlen ? p->seqlen_q : (int64_t)p->batch * p->seqlen_q;
  g.rows_k = g.varlen ? p->seqlen_k : (int64_t)p->batch * p->seqlen_k;
  return g;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [lse2 | Delta] fp32 in the lse layout, then (packed layouts) the int32 ranking
// of the sequences, then the fp32 dQ accumulator [rows_q, H, D] when the fused variant is
// selected.
// The fused (atomic) backward is selected by variant 1 and exists for bf16 only.
bool fused_backward(const exattn_problem* p) {
  return p->bwd_variant == 1 && p->dtype == EXATTN_DTYPE_BF16;
}

// Variant 3 stores dS for dense layouts whose dS fits kMaxStoredDs bytes; other problems
// run variant 0.
constexpr size_t kMaxStoredDs = (size_t)64 << 30;
bool stored_ds(const exattn_problem* p) {
  return p->bwd_variant == 3 && p->cu_seqlens_q == nullptr &&
         stored_ds_bytes(p->batch, p->heads_q, p->seqlen_q, p->seqlen_k) <= kMaxStoredDs;
}

struct WsLayout {
  size_t lse2, delta, order, dq_acc, ds, total;
};

// Packed layouts with at most kMaxOrderedUnits sequences get a ranking of the sequences
// (int32, longest first) that orders the dK/dV grid.
bool ordered_units(const exattn_problem* p) {
  return p->cu_seqlens_q != nullptr && p->num_seqs <= kMaxOrderedUnits;
}

WsLayout ws_layout(const exattn_problem* p) {
  const Geometry g = geometry(p);
  WsLayout w;
  const size_t nq = (size_t)g.rows_q * p->heads_q;
  w.lse2 = 0;
  w.delta = w.lse2 + align256(nq * sizeof(float));
  w.order = w.delta + align256(nq * sizeof(float));
  w.dq_acc = w.order + (ordered_units(p) ? align256((size_t)p->num_seqs * sizeof(int32_t)) : 0);
  w.ds = w.dq_acc + (fused_backward(p) ? align256(nq * p->head_dim * sizeof(float)) : 0);
  w.total = w.ds + (stored_ds(p) ? stored_ds_bytes(p->batch, p->heads_q, p->seqlen_q, p->seqlen_k) : 0);
  return w;
}

void fill_common(const exattn_problem* p, int64_t* qs, int64_t* ks, int64_t* vs) {
  for (int i = 0; i < 3; ++i) {
    qs[i] = p->q_stride[i];
    ks[i] = p->k_stride[i];
    vs[i] = p->v_stride[i];
  }
}

exattn_status hip_fail(hipError_t e, const char* what) {
  return fail(EXATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace exattn

using namespace exattn;

extern "C" {

int exattn_abi_version(void) { return EXATTN_ABI_VERSION; }

exattn_status exattn_check(const exattn_problem* p) {
  g_err[0] = 0;
  return validate(p, false, p && p->dtype == EXATTN_DTYPE_FP8_E4M3);
}

const char* exattn_status_string(exattn_status s) {
  switch (s) {
    case EXATTN_OK: return "ok";
    case EXATTN_ERR_NULL: return "null pointer";
    case EXATTN_ERR_DTYPE: return "unsupported dtype";
    case EXATTN_ERR_HEAD_DIM: return "unsupported head_dim";
    case EXATTN_ERR_SHAPE: return "invalid shape";
    case EXATTN_ERR_STRIDE: return "invalid stride";
    case EXATTN_ERR_ALIGN: return "misaligned pointer";
    case EXATTN_ERR_MASK: return "invalid mask";
    case EXATTN_ERR_VARLEN: return "invalid packed-sequence description";
    case EXATTN_ERR_WORKSPACE: return "invalid workspace";
    case EXATTN_ERR_SCALE: return "non-finite scale";
    case EXATTN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* exattn_last_error(void) { return g_err; }

exattn_status exattn_fwd(const exattn_problem* p, const void* q, const void* k, const void* v,
                         void* out, float* lse, void* stream) {
  g_err[0] = 0;
  exattn_status st = validate(p, false);
  if (st != EXATTN_OK) return st;
  const Geometry g = geometry(p);
  const bool any = g.rows_q > 0 && p->heads_q > 0;
  if (any && (!q || !out || !lse)) return fail(EXATTN_ERR_NULL, "q, out or lse is NULL");
  if (any && g.rows_k > 0 && (!k || !v)) return fail(EXATTN_ERR_NULL, "k or v is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(EXATTN_ERR_ALIGN, "q/k/v/out must be 16-byte aligned and lse 4-byte aligned");
  if (!any) return EXATTN_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = p->head_dim, H = p->heads_q;
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
  // out is written contiguous
  a.o_sh = D;
  a.o_ss = (int64_t)H * D;
  a.o_sb = (int64_t)p->seqlen_q * H * D;
  a.mask = p->mask;
  a.m_sb = p->mask_stride[0];
  a.m_sh = p->mask_stride[1];
  a.m_si = p->mask_stride[2];
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.B = g.varlen ? 1 : p->batch;
  a.Sq = p->seqlen_q;
  a.Sk = p->seqlen_k;
  a.H = H;
  a.Hkv = p->heads_kv;
  a.group = H / p->heads_kv;
  a.num_units = g.units;
  const int bm = fwd_block_m(D, p->mask_kind, g.varlen);
  const int maxq = g.varlen ? p->max_seqlen_q : p->seqlen_q;
  a.num_q_tiles = (maxq + bm - 1) / bm;
  a.max_sq = maxq;
  a.max_sk = g.varlen ? p->max_seqlen_k : p->seqlen_k;
  a.lse_row = p->seqlen_q;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  if ((int64_t)a.num_units * H * a.num_q_tiles > INT32_MAX)
    return fail(EXATTN_ERR_SHAPE, "too many query tiles");

  hipError_t e;
  if (a.num_q_tiles > 0) {
    e = timed(KernelId::Fwd, s, [&] {
      return launch_fwd(a, D, p->dtype, p->causal != 0, p->mask_kind, g.varlen, p->fwd_variant, s);
    });
    if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
  }
  if (g.varlen) {
    e = timed(KernelId::FwdTail, s, [&] { return launch_fwd_tail(a, D, s); });
    if (e != hipSuccess) return hip_fail(e, "forward tail launch");
  }
  return EXATTN_OK;
}

exattn_status exattn_fwd_fp8(const exattn_problem* p, const void* q, const void* k,
                             const void* v, float q_descale, float k_descale, float v_descale,
                             void* out, float* lse, void* stream) {
  g_err[0] = 0;
  exattn_status st = validate(p, false, true);
  if (st != EXATTN_OK) return st;
  // K and V tiles are read through 32-bit buffer offsets: 64 rows of the token stride.
  if (p->k_stride[1] >= (1 << 24) || p->v_stride[1] >= (1 << 24))
    return fail(EXATTN_ERR_STRIDE, "the fp8 forward needs k/v token strides below 2^24 elements");
  if (!std::isfinite(q_descale) || !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return fail(EXATTN_ERR_SCALE, "descales must be finite");
  const double c2 = (double)p->scale * q_descale * k_descale * 1.4426950408889634;
  if (!std::isfinite((float)c2)) return fail(EXATTN_ERR_SCALE, "scale * q_descale * k_descale overflows");
  const Geometry g = geometry(p);
  const bool any = g.rows_q > 0 && p->heads_q > 0;
  if (any && (!q || !out || !lse)) return fail(EXATTN_ERR_NULL, "q, out or lse is NULL");
  if (any && g.rows_k > 0 && (!k || !v)) return fail(EXATTN_ERR_NULL, "k or v is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(EXATTN_ERR_ALIGN, "q/k/v/out must be 16-byte aligned and lse 4-byte aligned");
  if (!any) return EXATTN_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = p->head_dim, H = p->heads_q;
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sh = D;  // out: contiguous bf16
  a.o_ss = (int64_t)H * D;
  a.o_sb = (int64_t)p->seqlen_q * H * D;
  a.B = p->batch;
  a.Sq = p->seqlen_q;
  a.Sk = p->seqlen_k;
  a.H = H;
  a.Hkv = p->heads_kv;
  a.group = H / p->heads_kv;
  a.num_units = p->batch;
  const int bm = fwd_fp8_block_m();
  a.num_q_tiles = (p->seqlen_q + bm - 1) / bm;
  a.max_sq = p->seqlen_q;
  a.max_sk = p->seqlen_k;
  a.lse_row = p->seqlen_q;
  a.scale_log2 = (float)c2;
  a.v_descale = v_descale;
  if ((int64_t)a.num_units * H * a.num_q_tiles > INT32_MAX)
    return fail(EXATTN_ERR_SHAPE, "too many query tiles");
  hipError_t e = timed(KernelId::FwdFp8, s, [&] { return launch_fwd_fp8(a, p->causal != 0, s); });
  if (e != hipSuccess) return hip_fail(e, "fp8 forward kernel launch");
  return EXATTN_OK;
}

size_t exattn_bwd_workspace_size(const exattn_problem* p) {
  if (validate(p, true) != EXATTN_OK) return 0;
  return ws_layout(p).total;
}

}  // extern "C"

namespace exattn {
namespace {

// Workspace of the allocation-free backward: one array per GPU, resolved per device.
constexpr size_t kScratchBytes = EXATTN_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // device address of `scratch` per device id

// The backward after validation: checks pointers and the workspace, then enqueues.
// `timing` = false skips the timing events (their creation may allocate).
exattn_status bwd_run(const exattn_problem* p, const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, void* stream,
                      bool timing) {
  const Geometry g = geometry(p);
  const bool anyq = g.rows_q > 0;
  const bool anyk = g.rows_k > 0;
  if (anyq && (!q || !out || !dout || !lse || !dq))
    return fail(EXATTN_ERR_NULL, "q, out, dout, lse or dq is NULL");
  if (anyk && (!k || !v || !dk || !dv)) return fail(EXATTN_ERR_NULL, "k, v, dk or dv is NULL");
  const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(EXATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(EXATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  const WsLayout w = ws_layout(p);
  if (anyq) {  // the workspace is only touched when there are query rows
    if (!workspace) return fail(EXATTN_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < w.total)
      return fail(EXATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(EXATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (!anyq && !anyk) return EXATTN_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = p->head_dim, H = p->heads_q;
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  const bool fused = fused_backward(p);
  a.dq_acc = fused ? reinterpret_cast<float*>(ws + w.dq_acc) : nullptr;
  a.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  a.delta = reinterpret_cast<float*>(ws + w.delta);
  int32_t* order = ordered_units(p) ? reinterpret_cast<int32_t*>(ws + w.order) : nullptr;
  a.unit_order = order;
  a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sb = p->o_stride[0]; a.o_ss = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.do_sb = p->do_stride[0]; a.do_ss = p->do_stride[1]; a.do_sh = p->do_stride[2];
  a.mask = p->mask;
  a.m_sb = p->mask_stride[0];
  a.m_sh = p->mask_stride[1];
  a.m_si = p->mask_stride[2];
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.B = g.varlen ? 1 : p->batch;
  a.Sq = p->seqlen_q;
  a.Sk = p->seqlen_k;
  a.H = H;
  a.Hkv = p->heads_kv;
  a.group = H / p->heads_kv;
  a.num_units = g.units;
  const int bn = bwd_block_n(D);
  const int maxk = g.varlen ? p->max_seqlen_k : p->seqlen_k;
  a.num_k_blocks = (maxk + bn - 1) / bn;
  const int bmq = bwd_dq_block_m(D);
  const int maxq = g.varlen ? p->max_seqlen_q : p->seqlen_q;
  a.num_q_blocks = (maxq + bmq - 1) / bmq;
  a.max_sq = maxq;
  a.max_sk = maxk;
  a.lse_row = p->seqlen_q;
  a.rows_q = (int)g.rows_q;
  a.rows_k = (int)g.rows_k;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a.rotate = fused ? 1 : 0;
  const bool sds = stored_ds(p);
  a.ds = sds ? ws + w.ds : nullptr;
  a.ds_nqt = (p->seqlen_q + 63) / 64;
  if ((((int64_t)a.num_units + 7) / 8 * 8) * a.Hkv * a.num_k_blocks > INT32_MAX ||
      (int64_t)a.num_units * H * a.num_q_blocks > INT32_MAX)
    return fail(EXATTN_ERR_SHAPE, "too many blocks");

  hipError_t e;
  if (!anyq) {
    // no query rows: every key receives zero gradient
    const int64_t bytes = g.rows_k * p->heads_kv * D * 2;
    e = timed_if(timing, KernelId::Zero, s, [&] { return launch_zero16(dk, bytes, s); });
    if (e == hipSuccess) e = timed_if(timing, KernelId::Zero, s, [&] { return launch_zero16(dv, bytes, s); });
    if (e != hipSuccess) return hip_fail(e, "zero dk/dv");
    return EXATTN_OK;
  }
  if (order) {
    e = timed_if(timing, KernelId::UnitOrder, s, [&] { return launch_unit_order(a, order, s); });
    if (e != hipSuccess) return hip_fail(e, "unit order launch");
  }
  e = timed_if(timing, KernelId::Delta, s, [&] { return launch_delta(a, D, p->dtype, g.varlen, s); });
  if (e != hipSuccess) return hip_fail(e, "delta kernel launch");
  const bool causal = p->causal != 0;
  if (a.num_k_blocks > 0) {
    const bool pipelined = !fused && p->bwd_variant != 2;
    e = timed(fused ? KernelId::BwdFused : KernelId::BwdDkDv, s, [&] {
      return pipelined ? launch_bwd_kv(a, D, p->dtype, causal, p->mask_kind, g.varlen, sds, s)
                       : launch_bwd(a, D, p->dtype, causal, p->mask_kind, g.varlen, fused, s);
    });
    if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  }
  if (fused) {
    e = timed_if(timing, KernelId::DqReduce, s, [&] { return launch_dq_reduce(a, D, s); });
    if (e != hipSuccess) return hip_fail(e, "dq reduce launch");
  } else if (sds) {
    e = timed_if(timing, KernelId::BwdDqDs, s, [&] { return launch_bwd_dq_ds(a, D, p->dtype, causal, s); });
    if (e != hipSuccess) return hip_fail(e, "dq kernel launch");
  } else {
    e = timed_if(timing, KernelId::BwdDq, s, [&] { return launch_bwd_dq(a, D, p->dtype, causal, p->mask_kind, g.varlen, s); });
    if (e != hipSuccess) return hip_fail(e, "dq kernel launch");
    if (g.varlen) {
      e = timed_if(timing, KernelId::QTail, s, [&] { return launch_q_tail(a, D, s); });
      if (e != hipSuccess) return hip_fail(e, "q tail launch");
    }
  }
  if (g.varlen && anyk) {
    e = timed_if(timing, KernelId::KvTail, s, [&] { return launch_kv_tail(a, D, s); });
    if (e != hipSuccess) return hip_fail(e, "kv tail launch");
  }
  return EXATTN_OK;
}

}  // namespace
}  // namespace exattn

extern "C" {

exattn_status exattn_bwd(const exattn_problem* p, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse, void* dq,
                         void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_err[0] = 0;
  exattn_status st = validate(p, true);
  if (st != EXATTN_OK) return st;
  return bwd_run(p, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, stream, true);
}

exattn_status exattn_bwd_noalloc(const exattn_problem* p, const void* q, const void* k,
                                 const void* v, const void* out, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, void* stream) {
  g_err[0] = 0;
  exattn_status st = validate(p, true);
  if (st != EXATTN_OK) return st;
  const size_t need = ws_layout(p).total;
  if (need > kScratchBytes)
    return fail(EXATTN_ERR_WORKSPACE,
                "this backward needs %zu bytes of workspace; exattn_bwd_noalloc holds at most %zu "
                "(EXATTN_NOALLOC_MAX_WORKSPACE): use exattn_bwd with a caller workspace",
                need, kScratchBytes);
  // The array's device address, resolved once per device with that device current (each
  // GPU holds its own copy of `scratch`; in host code the name is only a stand-in).
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev] = ptr;
    }
    ws = g_scratch_ptr[dev];
  }
  return bwd_run(p, q, k, v, out, dout, lse, dq, dk, dv, ws, kScratchBytes, stream, false);
}


exattn_status exattn_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return EXATTN_OK;
}

int exattn_timing_read(const char** names, double* total_ms, int* launches, int max) {
  std::vector<TimedLaunch> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_launches);
  }
  const int nk = (int)KernelId::Count;
  std::vector<double> ms(nk, 0.0);
  std::vector<int> cnt(nk, 0);
  int rc = 0;
  for (auto& r : recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) rc = -1;
    float t = 0.f;
    if (rc == 0 && hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess) {
      ms[r.kernel] += t;
      cnt[r.kernel] += 1;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto& r : recs) {
      g_event_pool.push_back(r.start);
      g_event_pool.push_back(r.stop);
    }
  }
  if (rc != 0) return -1;
  int n = 0;
  for (int i = 0; i < nk && n < max; ++i) {
    if (cnt[i] == 0) continue;
    if (names) names[n] = kernel_name((KernelId)i);
    if (total_ms) total_ms[n] = ms[i];
    if (launches) launches[n] = cnt[i];
    ++n;
  }
  return n;
}

}  // extern "C"
