// Backward kernels: recompute P from the stored LSE and produce dQ, dK, dV.
//
// Pass order on the caller's stream:
//   1. delta_kernel    Delta_i = sum_d dO_id * O_id (fp32), lse2_i = lse_i * log2(e)
//                      (+inf for empty rows so exp2(s - lse2) = 0), and the fp32 dQ
//                      accumulator cleared row by row (no memset node: graph-capture safe).
//   2. bwd_kernel      per (unit, kv head, block of 128 keys): dK and dV accumulate in
//                      registers over every query head of the group and every query tile;
//                      dQ partial products go to the fp32 accumulator with atomics.
//   3. dq_reduce       dq = bf16(dq_acc * scale).
//   4. kv_tail_kernel  packed layouts only: key rows past cu_seqlens_k[num_seqs] get
//                      dk = dv = 0.
//
// Sources: dv = P^T dO and dk = dS^T q (flash-dmattn PR #122 "Fix NaN/Inf values in dV
// gradients during backward pass", section "Solution", item 2); P = exp(s - lse) from the
// stored LSE, with the last partial key tile masked in the kernel so that out-of-range keys
// never produce exp(0 - lse) (OpenWAM PR #64, "Summary"); every output row written and
// no output read before it is written (flash-dmattn PR #122, "Root Cause" 1; PFCCLab
// cudnn-frontend PR #9 "DSA: fix dK SMEM handoff race and two latent NaN sources in the
// dense indexer", item 2); exponent bounded above (same page, item 3): exp2 of min(x, 0),
// since s - lse <= 0 for a consistent LSE.

#include <type_traits>

#include "common.hpp"
#include "params.hpp"

namespace exattn {

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// ----------------------------------------------------------------------------------------
// 1. Delta / lse2 / dQ-accumulator clear. One group of D/8 lanes per (row, head).
// ----------------------------------------------------------------------------------------
template <int D, bool VARLEN>
__global__ void __launch_bounds__(256) delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per block
  const int sub = threadIdx.x % LPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int64_t nrows = (int64_t)a.rows_q * a.H;
  if (r >= nrows) return;
  const int tok = (int)(r / a.H), head = (int)(r % a.H);
  int64_t o_off, do_off, st_idx;
  if constexpr (VARLEN) {
    o_off = (int64_t)tok * a.o_ss + (int64_t)head * a.o_sh;
    do_off = (int64_t)tok * a.do_ss + (int64_t)head * a.do_sh;
    st_idx = (int64_t)head * a.lse_row + tok;
  } else {
    const int b = tok / a.Sq, s = tok % a.Sq;
    o_off = (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)head * a.o_sh;
    do_off = (int64_t)b * a.do_sb + (int64_t)s * a.do_ss + (int64_t)head * a.do_sh;
    st_idx = ((int64_t)b * a.H + head) * a.Sq + s;
  }
  const bf16x8 o = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.out) + o_off + sub * 8);
  const bf16x8 g = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.dout) + do_off + sub * 8);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += (float)o[i] * (float)g[i];
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  float* dqa = a.dq_acc + r * D + sub * 8;
  reinterpret_cast<f32x4*>(dqa)[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  reinterpret_cast<f32x4*>(dqa)[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (sub == 0) {
    const float l = a.lse[st_idx];
    a.delta[st_idx] = acc;
    a.lse2[st_idx] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ----------------------------------------------------------------------------------------
// 2. Main backward kernel.
//
// One workgroup = 4 waves = 128 keys of one (unit, kv head); wave w owns keys 32w..32w+31
// and accumulates their dK and dV in fp32 (C layout: rows = keys, columns = d) across
// every query head of the group and every query tile that can see the block. The
// block's K and V stay in LDS for the whole loop. Per query tile of 64 rows, Q and dO are
// copied straight from global memory into LDS (double-buffered, zero past the end), and
// lse2/Delta through registers:
//   S  = Q K^T and dP = dO V^T          (lane = key column, registers = query rows)
//   P  = exp2(min(S*c + bias - lse2, 0)), dS = P * (dP - Delta); hidden entries are 0
//   dV += P^T dO, dK += dS^T Q          (P and dS are the A operand straight from registers;
//                                        dO and Q come from transposed LDS reads)
//   dS -> LDS [query][key]; each wave forms 32x32 dQ tiles over the block's 128 keys
//   (K from transposed LDS reads) and adds them to the fp32 accumulator with buffer
//   atomics, which drop rows past the end of the sequence.
// Row-major LDS tiles without padding use an XOR swizzle of their 16-byte chunks,
// chunk' = chunk ^ (2*(row & 3) + ((row >> 2) & 1)), which keeps both the 16-byte row reads
// and the 8-byte transposed reads free of bank conflicts.
// ----------------------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BN = 128;
  static constexpr int BM = 64;
  static constexpr int QB = BM / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int SLD = BN + 8;             // dS pitch (16 B mod 128 B)
  static constexpr int Q_ELEMS = BM * D;
  static constexpr int K_ELEMS = BN * D;
  static constexpr int S_ELEMS = BM * SLD;
  static constexpr int DQ_TILES = QB * DB;       // 32x32 dQ tiles per query tile
  static constexpr int DQ_PER_WAVE = DQ_TILES / NW;
  static_assert((BM * CPR) % (64 * NW) == 0 && (BN * CPR) % (64 * NW) == 0, "even copy split");
  static_assert(DQ_PER_WAVE * NW == DQ_TILES, "even dQ split");
};

__device__ __forceinline__ int swz_f(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

// Element offset of (row, col) in a swizzled row-major tile with D columns.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 3) ^ swz_f(row))) << 3) + (col & 7);
}

// Copy R rows of D bf16 (row stride `stride` elements, rows past the buffer range read as
// zero) into a swizzled LDS tile with direct global->LDS loads: each wave instruction
// fills 64 consecutive 16-byte LDS chunks, lane i the i-th, so lane i fetches the global
// chunk that the swizzle places there. Completion is tracked by vmcnt.
template <int D, int R, int NW>
__device__ __forceinline__ void copy_tile_to_lds(bf16* dst, __amdgpu_buffer_rsrc_t rs, int stride,
                                                 int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int ITER = R * CPR / 64 / NW;
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int pos = p0 + lane;
    const int row = pos / CPR, pc = pos % CPR;
    const int col = (pc ^ swz_f(row)) * 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + p0 * 8), 16,
        (int)((row * stride + col) * 2), 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every vector-memory operation except the most recent N. The counter retires in
// issue order, so this waits for the earlier loads while the last N (the dQ atomics of the
// current tile) stay in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_except() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D>
constexpr size_t bwd_smem_bytes() {
  using T = BwdTile<D>;
  return (size_t)(2 * T::K_ELEMS + 4 * T::Q_ELEMS + T::S_ELEMS) * 2 + 4 * T::BM * sizeof(float);
}

// LDS read at a per-lane byte address plus a compile-time byte offset (the offset folds into
// the instruction's immediate field).
template <class V>
__device__ __forceinline__ V lds_at(const unsigned char* base, int imm) {
  return *reinterpret_cast<const V*>(base + imm);
}
__device__ __forceinline__ bf16x4 tr_at(const unsigned char* base, int imm) {
  return lds_read_tr4(reinterpret_cast<const bf16*>(base + imm));
}

template <int D, bool CAUSAL, int MASK, bool VARLEN>
__global__ void __launch_bounds__(256) bwd_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int RB = D * 2;                      // bytes per swizzled row
  constexpr int QBYTES = T::Q_ELEMS * 2;         // one Q or dO buffer
  constexpr int KBYTES = T::K_ELEMS * 2;
  constexpr int DO_OFF = 2 * QBYTES;             // dO buffers follow the two Q buffers
  constexpr int V_OFF = KBYTES;                  // V follows K
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* k_b = smem;                     // K then V
  unsigned char* q_b = smem + 2 * KBYTES;        // Q[2] then dO[2]
  unsigned char* ds_b = q_b + 4 * QBYTES;        // dS [BM][SLD]
  float* lse2_l = reinterpret_cast<float*>(ds_b + T::S_ELEMS * 2);  // [2][BM]
  float* del_l = lse2_l + 2 * T::BM;                                // [2][BM]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, j16 = lane & 15;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int kbi = blk % a.num_k_blocks;
  const int ug = blk / a.num_k_blocks;
  const int g = ug % a.Hkv, unit = ug / a.Hkv;

  int Sq, Sk;
  int64_t qrow0, krow0, qb_off, kb_off, vb_off, dob_off, st_unit;
  if constexpr (VARLEN) {
    const int qs = a.cu_q[unit], ks = a.cu_k[unit];
    Sq = a.cu_q[unit + 1] - qs;
    Sk = a.cu_k[unit + 1] - ks;
    qrow0 = qs;
    krow0 = ks;
    qb_off = (int64_t)qs * a.q_ss;
    kb_off = (int64_t)ks * a.k_ss;
    vb_off = (int64_t)ks * a.v_ss;
    dob_off = (int64_t)qs * a.do_ss;
    st_unit = qs;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
    qrow0 = (int64_t)unit * a.Sq;
    krow0 = (int64_t)unit * a.Sk;
    qb_off = (int64_t)unit * a.q_sb;
    kb_off = (int64_t)unit * a.k_sb;
    vb_off = (int64_t)unit * a.v_sb;
    dob_off = (int64_t)unit * a.do_sb;
    st_unit = 0;
  }
  const int kb0 = kbi * T::BN;
  if (kb0 >= Sk) return;
  const int krows = min(T::BN, Sk - kb0);

  // The block's K and V, row-major and swizzled, zero past the last key.
  {
    const bf16* K = reinterpret_cast<const bf16*>(a.k) + kb_off + (int64_t)g * a.k_sh +
                    (int64_t)kb0 * a.k_ss;
    const bf16* V = reinterpret_cast<const bf16*>(a.v) + vb_off + (int64_t)g * a.v_sh +
                    (int64_t)kb0 * a.v_ss;
    copy_tile_to_lds<D, T::BN, T::NW>(reinterpret_cast<bf16*>(k_b),
                                     make_rsrc(K, (uint32_t)((krows - 1) * a.k_ss + D) * 2u),
                                     (int)a.k_ss, wave, lane);
    copy_tile_to_lds<D, T::BN, T::NW>(reinterpret_cast<bf16*>(k_b + V_OFF),
                                     make_rsrc(V, (uint32_t)((krows - 1) * a.v_ss + D) * 2u),
                                     (int)a.v_ss, wave, lane);
  }
  const int kl_w = wave * 32 + l32;          // block-local key of this lane
  const int kw = kb0 + kl_w;

  // ---- per-lane LDS base addresses; everything else is an immediate offset ----------------
  // Row-operand reads (row & 7 == l32 & 7 for Q/dO rows qb*32+l32 and K/V rows kl_w): the
  // swizzle only permutes d-slab pairs within groups of four, so four bases cover all slabs.
  const int fa_hi = l32 & 3, fa_lo = (l32 >> 2) & 1;
  const unsigned char* aq[4];   // Q buffer 0 (+QBYTES for buffer 1, +DO_OFF for dO)
  const unsigned char* ak[4];   // K (+V_OFF for V)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = 32 * (i ^ fa_hi) + 16 * (half ^ fa_lo);
    aq[i] = q_b + l32 * RB + off;
    ak[i] = k_b + kl_w * RB + off;
  }
  // Transposed reads of Q/dO for dV/dK: rows 16kk + 4*half + (j16>>2) (+8), columns
  // db*32 + 16*(grp&1) + 4*(j16&3). Two bases, for db even and odd.
  const int tr_row = j16 >> 2;
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  const unsigned char* tq[2];
  {
    const int row = 4 * half + tr_row;
    const int f = swz_f(row);
#pragma unroll
    for (int b = 0; b < 2; ++b) tq[b] = q_b + row * RB + 16 * ((4 * b + clow) ^ f) + 8 * (j16 & 1);
  }
  // Transposed reads of K for dQ: rows 16kk + 8*half + (j16>>2) and 4 rows below.
  const unsigned char* tk[2][2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 8 * half + tr_row + 4 * sec;
    const int f = swz_f(row);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      tk[sec][b] = k_b + row * RB + 16 * ((4 * b + clow) ^ f) + 8 * (j16 & 1);
  }
  // dS written as [query][key] from the C layout, read back as 8 consecutive keys per lane.
  unsigned char* dsw = ds_b + (4 * half * T::SLD + kl_w) * 2;
  const unsigned char* dsr = ds_b + (l32 * T::SLD + 8 * half) * 2;
  const unsigned char* st_rd = reinterpret_cast<const unsigned char*>(lse2_l) + 16 * half;

  f32x16 dk[T::DB], dv[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) dk[db] = dv[db] = f32x16{};

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);
  const int qstart = CAUSAL ? min(kb0 / T::BM * T::BM, Sq) : 0;
  const int n_qt = (Sq - qstart + T::BM - 1) / T::BM;
  const int n_iter = a.group * n_qt;

  // Staging of one query tile: Q and dO straight into LDS, lse2 and Delta via registers.
  float st_v = 0.f;
  auto tile_head = [&](int it) { return g * a.group + it / n_qt; };
  auto tile_q0 = [&](int it) { return qstart + (it % n_qt) * T::BM; };
  auto load_q = [&](int it, int buf) {
    const int head = tile_head(it), qt0 = tile_q0(it);
    const int rows = min(T::BM, Sq - qt0);
    const bf16* Qp = reinterpret_cast<const bf16*>(a.q) + qb_off + (int64_t)head * a.q_sh +
                     (int64_t)qt0 * a.q_ss;
    const bf16* Dp = reinterpret_cast<const bf16*>(a.dout) + dob_off + (int64_t)head * a.do_sh +
                     (int64_t)qt0 * a.do_ss;
    copy_tile_to_lds<D, T::BM, T::NW>(reinterpret_cast<bf16*>(q_b + buf * QBYTES),
                                     make_rsrc(Qp, (uint32_t)((rows - 1) * a.q_ss + D) * 2u),
                                     (int)a.q_ss, wave, lane);
    copy_tile_to_lds<D, T::BM, T::NW>(reinterpret_cast<bf16*>(q_b + DO_OFF + buf * QBYTES),
                                     make_rsrc(Dp, (uint32_t)((rows - 1) * a.do_ss + D) * 2u),
                                     (int)a.do_ss, wave, lane);
    const int64_t st = VARLEN ? (int64_t)head * a.lse_row + st_unit
                              : ((int64_t)unit * a.H + head) * a.Sq;
    if (tid < 2 * T::BM) {
      const int r = tid & (T::BM - 1);
      const bool ok = r < rows;
      st_v = tid < T::BM ? (ok ? a.lse2[st + qt0 + r] : INFINITY) : (ok ? a.delta[st + qt0 + r] : 0.f);
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < T::BM) lse2_l[buf * T::BM + tid] = st_v;
    else if (tid < 2 * T::BM) del_l[buf * T::BM + tid - T::BM] = st_v;
  };

  if (n_iter > 0) {
    load_q(0, 0);
    store_stats(0);
  }
  wait_vmem();
  __syncthreads();

  // One query tile. BUF (0/1) selects the staging buffer at compile time.
  auto iteration = [&](int it, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr int QO = BUF * QBYTES;
    if (it + 1 < n_iter) load_q(it + 1, BUF ^ 1);
    const int head = tile_head(it), qt0 = tile_q0(it);
    const bool edge = (kb0 + T::BN > Sk) || (qt0 + T::BM > Sq) || (MASK != kMaskNone) ||
                      (CAUSAL && kb0 + T::BN - 1 > qt0);
    const int64_t m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;

    // P = exp2(min(S*c + bias - lse2, 0)) and dS = P * (dP - Delta), in place.
    auto softmax_grad = [&](f32x16& s, f32x16& dp, int qb, auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int soff = BUF * T::BM * 4 + (qb * 32 + 8 * rg) * 4;
        const f32x4 l2 = lds_at<f32x4>(st_rd, soff);
        const f32x4 dd = lds_at<f32x4>(st_rd, soff + 2 * T::BM * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float p;
          if constexpr (!EDGE) {
            p = fast_exp2(fminf(fmaf(s[r], c2, -l2[e]), 0.f));
          } else {
            // Branch-free visibility: mask reads use indices clamped into range.
            const int qi = qt0 + qb * 32 + 8 * rg + 4 * half + e;
            bool vis = (qi < Sq) && (kw < Sk);
            if (CAUSAL) vis = vis && (kw <= qi);
            float b2 = 0.f;
            if (MASK != kMaskNone) {
              const int64_t mi = m_base + (int64_t)min(qi, Sq - 1) * a.m_si + min(kw, Sk - 1);
              if (MASK == kMaskBool) {
                vis = vis && (mask_u8[mi] != 0);
              } else {
                const float bias = (float)mask_bf[mi];
                vis = vis && (bias != -INFINITY);
                b2 = vis ? bias * kLog2e : 0.f;
              }
            }
            const float e2 = fast_exp2(fminf(fmaf(s[r], c2, b2 - l2[e]), 0.f));
            p = vis ? e2 : 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - dd[e]);
        }
      }
    };

#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 query rows: rows = queries, columns = keys.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ds = 0; ds < T::DS; ++ds) {
        const int i = ds & 3, m = (ds >> 2) * 128;
        const bf16x8 kf = lds_at<bf16x8>(ak[i], m);
        const bf16x8 vf = lds_at<bf16x8>(ak[i], m + V_OFF);
        s = mfma32(lds_at<bf16x8>(aq[i], QO + qb * 32 * RB + m), kf, s);
        dp = mfma32(lds_at<bf16x8>(aq[i], DO_OFF + QO + qb * 32 * RB + m), vf, dp);
      }
      if (edge) softmax_grad(s, dp, qb, bool_c<true>{});
      else softmax_grad(s, dp, qb, bool_c<false>{});
      // dV += P^T dO and dK += dS^T Q over the two 16-row slabs of these 32 rows.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kk = 2 * qb + ks, hs = ks * 8;
        const bf16x8 pa = cvt8(s[hs + 0], s[hs + 1], s[hs + 2], s[hs + 3], s[hs + 4], s[hs + 5],
                               s[hs + 6], s[hs + 7]);
        const bf16x8 sa = cvt8(dp[hs + 0], dp[hs + 1], dp[hs + 2], dp[hs + 3], dp[hs + 4],
                               dp[hs + 5], dp[hs + 6], dp[hs + 7]);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const unsigned char* tb = tq[db & 1];
          const int o = QO + 16 * kk * RB + 128 * (db >> 1);
          const bf16x8 ob = cat44(tr_at(tb, DO_OFF + o), tr_at(tb, DO_OFF + o + 8 * RB));
          const bf16x8 qv = cat44(tr_at(tb, o), tr_at(tb, o + 8 * RB));
          dv[db] = mfma32(pa, ob, dv[db]);
          dk[db] = mfma32(sa, qv, dk[db]);
        }
      }
      // dS -> LDS as [query][key] for the dQ product.
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<bf16*>(dsw + (qb * 32 + 8 * (r >> 2) + (r & 3)) * T::SLD * 2) = (bf16)dp[r];
    }
    __syncthreads();  // dS complete; every wave is done with this tile's Q and dO

    // dQ tiles: rows = queries, columns = d; k = the block's 128 keys.
    const int qrows = min(T::BM, Sq - qt0);
    float* dqp = a.dq_acc + ((qrow0 + qt0) * a.H + head) * D;
    const auto rdq = make_rsrc(dqp, (uint32_t)((qrows - 1) * a.H * D + D) * 4u);
#pragma unroll
    for (int tt = 0; tt < T::DQ_PER_WAVE; ++tt) {
      const int tile = wave * T::DQ_PER_WAVE + tt;
      const int qb = tile / T::DB, db = tile % T::DB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < T::BN / 16; ++kk) {
        const bf16x8 sv = lds_at<bf16x8>(dsr, (qb * 32 * T::SLD + kk * 16) * 2);
        const int o = 16 * kk * RB + 128 * (db >> 1);
        const bf16x8 kv = cat44(tr_at(tk[0][db & 1], o), tr_at(tk[1][db & 1], o));
        acc = mfma32(sv, kv, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qb * 32 + acc_row(r, half);
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
            acc[r], rdq, (int)((row * a.H * D + db * 32 + l32) * 4), 0, 0);
      }
    }
    if (it + 1 < n_iter) store_stats(BUF ^ 1);
    wait_vmem_except<16 * T::DQ_PER_WAVE>();  // the next tile's Q and dO have landed in LDS
    __syncthreads();  // ... for every wave, and every wave is done reading dS
  };

  int it = 0;
  for (; it + 1 < n_iter; it += 2) {
    iteration(it, std::integral_constant<int, 0>{});
    iteration(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < n_iter) iteration(it, std::integral_constant<int, 0>{});

  // Epilogue: dK (times scale) and dV as bf16 into contiguous [rows_k, Hkv, D]; rows past
  // the sequence end are dropped by the buffer range.
  const float sc = a.scale;
  const int64_t kv_off = ((krow0 + kb0) * a.Hkv + g) * D;
  const uint32_t kv_bytes = (uint32_t)((krows - 1) * a.Hkv * D + D) * 2u;
  const auto rdk = make_rsrc(reinterpret_cast<bf16*>(a.dk) + kv_off, kv_bytes);
  const auto rdv = make_rsrc(reinterpret_cast<bf16*>(a.dv) + kv_off, kv_bytes);
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = wave * 32 + acc_row(r, half);
      const int off = (key * a.Hkv * D + db * 32 + l32) * 2;
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)(dk[db][r] * sc)),
                                            rdk, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)dv[db][r]),
                                            rdv, off, 0, 0);
    }
  }
}

// ----------------------------------------------------------------------------------------
// 3. dq = bf16(dq_acc * scale), 8 elements per thread.
// ----------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) dq_reduce_kernel(BwdArgs a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.dq_acc) + 2 * i;
  const f32x4 x0 = src[0], x1 = src[1];
  const float sc = a.scale;
  reinterpret_cast<bf16x8*>(a.dq)[i] = cvt8(x0[0] * sc, x0[1] * sc, x0[2] * sc, x0[3] * sc,
                                            x1[0] * sc, x1[1] * sc, x1[2] * sc, x1[3] * sc);
}

// ----------------------------------------------------------------------------------------
// 4. Packed layouts: key rows past cu_seqlens_k[num_seqs] get dk = dv = 0.
// ----------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kv_tail_kernel(BwdArgs a, int64_t row_chunks, int chunks_per_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= row_chunks) return;
  const int64_t row = i / chunks_per_row;
  if (row < a.cu_k[a.num_units]) return;
  reinterpret_cast<u32x4*>(a.dk)[i] = u32x4{0, 0, 0, 0};
  reinterpret_cast<u32x4*>(a.dv)[i] = u32x4{0, 0, 0, 0};
}

// Zero-fill of a buffer, 16 bytes per thread (used instead of a memset node so that the
// call stays capturable into a graph).
__global__ void __launch_bounds__(256) zero16_kernel(u32x4* p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = u32x4{0, 0, 0, 0};
}

// ----------------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------------
hipError_t launch_zero16(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  dim3 grid((unsigned)((n16 + 255) / 256)), block(256);
  hipLaunchKernelGGL(zero16_kernel, grid, block, 0, s, reinterpret_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

int bwd_block_n(int head_dim) { return BwdTile<128>::BN; }

hipError_t launch_delta(const BwdArgs& a, int head_dim, bool varlen, hipStream_t s) {
  const int64_t nrows = (int64_t)a.rows_q * a.H;
  if (nrows <= 0) return hipSuccess;
  const int rpb = 256 / (head_dim / 8);
  dim3 grid((unsigned)((nrows + rpb - 1) / rpb)), block(256);
  if (head_dim == 64) {
    if (varlen) hipLaunchKernelGGL((delta_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<64, false>), grid, block, 0, s, a);
  } else {
    if (varlen) hipLaunchKernelGGL((delta_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<128, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  const int64_t nblk = (int64_t)a.num_units * a.Hkv * a.num_k_blocks;
  if (nblk <= 0) return hipSuccess;
  constexpr size_t smem = bwd_smem_bytes<D>();
  dim3 grid((unsigned)nblk), block(256);
#define EXATTN_BWD(C, M, V)                                                                    \
  do {                                                                                         \
    auto kfn = bwd_kernel<D, C, M, V>;                                                         \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL(kfn, grid, block, smem, s, a);                                          \
  } while (0)
  if (varlen) {
    if (causal) EXATTN_BWD(true, kMaskNone, true);
    else EXATTN_BWD(false, kMaskNone, true);
  } else if (causal) {
    if (mask == kMaskBool) EXATTN_BWD(true, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_BWD(true, kMaskAdd, false);
    else EXATTN_BWD(true, kMaskNone, false);
  } else {
    if (mask == kMaskBool) EXATTN_BWD(false, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_BWD(false, kMaskAdd, false);
    else EXATTN_BWD(false, kMaskNone, false);
  }
#undef EXATTN_BWD
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool causal, int mask, bool varlen,
                      hipStream_t s) {
  if (head_dim == 64) return launch_bwd_d<64>(a, causal, mask, varlen, s);
  return launch_bwd_d<128>(a, causal, mask, varlen, s);
}

hipError_t launch_dq_reduce(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t n8 = (int64_t)a.rows_q * a.H * head_dim / 8;
  if (n8 <= 0) return hipSuccess;
  dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  hipLaunchKernelGGL(dq_reduce_kernel, grid, block, 0, s, a, n8);
  return hipGetLastError();
}

hipError_t launch_kv_tail(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int cpr = a.Hkv * head_dim / 8;
  const int64_t n = (int64_t)a.rows_k * cpr;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  hipLaunchKernelGGL(kv_tail_kernel, grid, block, 0, s, a, n, cpr);
  return hipGetLastError();
}

}  // namespace exattn
