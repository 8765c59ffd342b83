// Kernel argument blocks and launcher declarations (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  const void* mask;
  int64_t m_sb, m_sh, m_si;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Sq, Sk, H, Hkv, group;
  int num_units;     // batch (dense) or num_seqs (packed)
  int num_q_tiles;   // per unit
  int lse_row;       // packed: row count of lse ([H, lse_row]); dense: Sq
  int max_sq;        // packed: sequences are truncated to max_sq query rows ...
  int max_sk;        // ... and max_sk key rows (max_seqlen); dense: Sq and Sk
  float scale_log2;  // scale * log2(e); fp8 forward: scale * q_descale * k_descale * log2(e)
  float v_descale;   // fp8 forward only: multiplies the normalised output
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;     // fp32 [rows_q, H, D], fused variant only (else NULL)
  float* lse2;       // fp32, lse layout: lse * log2(e), +inf for empty rows
  float* delta;      // fp32, lse layout: rowsum(dout * out)
  const int32_t* unit_order;  // packed: sequences by query length, longest first (NULL = in order)
  void* ds;          // stored dS chunks (backward variant 3, dense only), else NULL
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  const void* mask;
  int64_t m_sb, m_sh, m_si;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Sq, Sk, H, Hkv, group;
  int num_units;
  int num_k_blocks;  // key blocks per (unit, kv head), dK/dV kernel
  int num_q_blocks;  // query blocks per (unit, head), dQ kernel
  int lse_row;
  int max_sq;        // packed: sequences are truncated to max_sq query rows and max_sk key
  int max_sk;        // rows (max_seqlen); dense: Sq and Sk
  int rows_q;        // rows of q per head in total: B*Sq (dense) or total_q (packed)
  int rows_k;
  int rotate;        // query-tile order: 0 = in order, 1 = spread by key block, 2 = offset kbi % 8
  int ds_nqt;        // stored dS: 64-row query tiles per (unit, head), ceil(Sq / 64)
  float scale;
  float scale_log2;
};

enum class KernelId : int {
  Fwd = 0, FwdTail, Delta, BwdDkDv, BwdDq, BwdFused, DqReduce, KvTail, QTail, Zero, FwdFp8,
  UnitOrder, BwdDqDs, Count
};

const char* kernel_name(KernelId id);

// Launchers return hipGetLastError() after the launch. `variant` selects the tiling.
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, bool causal, int mask_mode,
                      bool varlen, int variant, hipStream_t s);
hipError_t launch_fwd_tail(const FwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_delta(const BwdArgs& a, int head_dim, int dtype, bool varlen, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask_mode,
                      bool varlen, bool fused_dq, hipStream_t s);
// Pipelined dK/dV kernel (default); with `store_ds` (dense only) it also writes dS to a.ds.
hipError_t launch_bwd_kv(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask_mode,
                         bool varlen, bool store_ds, hipStream_t s);
// dQ = dS K from the stored dS (dense only).
hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, int dtype, bool causal, hipStream_t s);
// Bytes of the stored dS for a dense problem: B * H * ceil(Sq / 64) * ceil(Sk / 128) * 16 KiB.
size_t stored_ds_bytes(int64_t batch, int64_t heads, int64_t sq, int64_t sk);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask_mode,
                         bool varlen, hipStream_t s);
hipError_t launch_q_tail(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_dq_reduce(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_kv_tail(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_zero16(void* p, int64_t bytes, hipStream_t s);  // bytes % 16 == 0
constexpr int kMaxOrderedUnits = 8192;  // packed sequences ranked for the dK/dV grid, at most
hipError_t launch_unit_order(const BwdArgs& a, int32_t* order, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs& a, bool causal, hipStream_t s);  // head_dim 128, dense

// Tile shapes the host needs for grid sizing.
int fwd_block_m(int head_dim, int mask, bool varlen);
int fwd_fp8_block_m();
int bwd_block_n(int head_dim);
int bwd_dq_block_m(int head_dim);

}  // namespace exattn
