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

#include "common.hpp"
#include "params.hpp"

namespace exattn {

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
// and keeps their K and V fragments (B-operand layout, k-slots = d) in registers, plus
// fp32 dK and dV accumulators (C layout: rows = keys, columns = d).
// Per query tile of 64 rows, staged in LDS both row-major (A operand, k = d) and
// row-interleaved Q[row/4][d][row%4] (B operand with k = rows):
//   S  = Q K^T and dP = dO V^T          (lane = key column, registers = query rows)
//   P  = exp2(min(S*c - lse2, 0)), dS = P * (dP - Delta), masked entries 0
//   dV += P^T dO, dK += dS^T Q          (P and dS feed the A operand from registers)
//   dS -> LDS [query][key]; dQ tile = dS K over all 128 keys, K read from an interleaved
//   copy K[key/4][d][key%4]; each wave adds its dQ tiles with fp32 atomics.
// ----------------------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int NW = 4;
  static constexpr int BN = 128;
  static constexpr int BM = 64;
  static constexpr int QB = BM / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QLD = D + 8;        // row-major pitch
  static constexpr int TG = D * 4 + 8;     // interleaved 4-row group pitch
  static constexpr int SLD = BN + 8;       // dS pitch
  static constexpr int Q_ELEMS = BM * QLD;
  static constexpr int QT_ELEMS = (BM / 4) * TG;
  static constexpr int KT_ELEMS = (BN / 4) * TG;
  static constexpr int S_ELEMS = BM * SLD;
  static constexpr int QGR = (BM / 4) * (D / 8);   // 4x8 blocks per Q tile
  static constexpr int KGR = (BN / 4) * (D / 8);   // 4x8 blocks of the K tile
  static constexpr int DQ_TILES = QB * DB;         // 32x32 dQ tiles per query tile
  static constexpr int DQ_PER_WAVE = DQ_TILES / NW;
};

template <int D, bool CAUSAL, int MASK, bool VARLEN>
__global__ void __launch_bounds__(256) bwd_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* q_l = reinterpret_cast<bf16*>(smem);
  bf16* qt_l = q_l + T::Q_ELEMS;
  bf16* do_l = qt_l + T::QT_ELEMS;
  bf16* dot_l = do_l + T::Q_ELEMS;
  bf16* kt_l = dot_l + T::QT_ELEMS;
  bf16* ds_l = kt_l + T::KT_ELEMS;
  float* lse2_l = reinterpret_cast<float*>(ds_l + T::S_ELEMS);
  float* del_l = lse2_l + T::BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int kbi = blk % a.num_k_blocks;
  const int ug = blk / a.num_k_blocks;
  const int g = ug % a.Hkv, unit = ug / a.Hkv;

  int Sq, Sk;
  int64_t qrow0, krow0;              // first row of the unit in the token dimension
  int64_t qb_off, kb_off, vb_off, ob_off, dob_off, st_base_unit;
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
    ob_off = 0;
    st_base_unit = qs;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
    qrow0 = (int64_t)unit * a.Sq;
    krow0 = (int64_t)unit * a.Sk;
    qb_off = (int64_t)unit * a.q_sb;
    kb_off = (int64_t)unit * a.k_sb;
    vb_off = (int64_t)unit * a.v_sb;
    dob_off = (int64_t)unit * a.do_sb;
    ob_off = 0;
    st_base_unit = 0;
  }
  (void)ob_off;
  const int kb0 = kbi * T::BN;
  if (kb0 >= Sk) return;

  const bf16* K = reinterpret_cast<const bf16*>(a.k) + kb_off + (int64_t)g * a.k_sh;
  const bf16* V = reinterpret_cast<const bf16*>(a.v) + vb_off + (int64_t)g * a.v_sh;

  // This wave's key fragments (B operand: column = key, k-slots = d).
  const int kw = kb0 + wave * 32 + l32;
  bf16x8 kf[T::DS], vf[T::DS];
  if (kw < Sk) {
    const bf16* kr = K + (int64_t)kw * a.k_ss + 8 * half;
    const bf16* vr = V + (int64_t)kw * a.v_ss + 8 * half;
#pragma unroll
    for (int s = 0; s < T::DS; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
      vf[s] = *reinterpret_cast<const bf16x8*>(vr + 16 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < T::DS; ++s) kf[s] = vf[s] = bf16x8{};
  }

  // Interleaved copy of the whole 128-key K block for the dQ product.
  for (int gi = tid; gi < T::KGR; gi += 256) {
    const int g4 = gi / (D / 8), d8 = gi % (D / 8);
    u32x4 rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb0 + 4 * g4 + i;
      rr[i] = key < Sk ? ldg16(K + (int64_t)key * a.k_ss + d8 * 8) : u32x4{0, 0, 0, 0};
    }
    store_4x8_transposed(kt_l + g4 * T::TG + d8 * 32, rr[0], rr[1], rr[2], rr[3]);
  }

  f32x16 dk[T::DB], dv[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) dk[db] = dv[db] = f32x16{};

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);
  const int qstart = CAUSAL ? (kb0 / T::BM) * T::BM : 0;
  const bool q_thread = (T::QGR >= 256) || (tid < T::QGR);
  const int sg4 = tid / (D / 8), sd8 = tid % (D / 8);

  for (int hh = 0; hh < a.group; ++hh) {
    const int head = g * a.group + hh;
    const bf16* Q = reinterpret_cast<const bf16*>(a.q) + qb_off + (int64_t)head * a.q_sh;
    const bf16* DO = reinterpret_cast<const bf16*>(a.dout) + dob_off + (int64_t)head * a.do_sh;
    const int64_t st_base = VARLEN ? (int64_t)head * a.lse_row + st_base_unit
                                   : ((int64_t)unit * a.H + head) * a.Sq;
    const int64_t m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;

    for (int qt0 = qstart; qt0 < Sq; qt0 += T::BM) {
      __syncthreads();  // previous tile's LDS reads are complete
      if (q_thread) {
        u32x4 rq[4], rd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = qt0 + 4 * sg4 + i;
          const bool ok = qi < Sq;
          rq[i] = ok ? ldg16(Q + (int64_t)qi * a.q_ss + sd8 * 8) : u32x4{0, 0, 0, 0};
          rd[i] = ok ? ldg16(DO + (int64_t)qi * a.do_ss + sd8 * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<u32x4*>(q_l + (4 * sg4 + i) * T::QLD + sd8 * 8) = rq[i];
          *reinterpret_cast<u32x4*>(do_l + (4 * sg4 + i) * T::QLD + sd8 * 8) = rd[i];
        }
        store_4x8_transposed(qt_l + sg4 * T::TG + sd8 * 32, rq[0], rq[1], rq[2], rq[3]);
        store_4x8_transposed(dot_l + sg4 * T::TG + sd8 * 32, rd[0], rd[1], rd[2], rd[3]);
      }
      if (tid < T::BM) {
        const int qi = qt0 + tid;
        lse2_l[tid] = qi < Sq ? a.lse2[st_base + qi] : INFINITY;
      } else if (tid < 2 * T::BM) {
        const int qi = qt0 + tid - T::BM;
        del_l[tid - T::BM] = qi < Sq ? a.delta[st_base + qi] : 0.f;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T: rows = queries, columns = this wave's keys.
      f32x16 s[T::QB], dp[T::QB];
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < T::DS; ++ds) {
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb) {
          const int off = (qb * 32 + l32) * T::QLD + ds * 16 + 8 * half;
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(q_l + off);
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(do_l + off);
          s[qb] = mfma32(qa, kf[ds], s[qb]);
          dp[qb] = mfma32(da, vf[ds], dp[qb]);
        }
      }

      // P and dS in place.
      const bool edge = (kb0 + T::BN > Sk) || (qt0 + T::BM > Sq) || (MASK != kMaskNone) ||
                        (CAUSAL && kb0 + T::BN - 1 > qt0);
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int rl = qb * 32 + 8 * rg + 4 * half;  // local row of register 4*rg
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(lse2_l + rl);
          const f32x4 dl = *reinterpret_cast<const f32x4*>(del_l + rl);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            float x = s[qb][r] * c2;
            bool vis = true;
            if (edge) {
              const int qi = qt0 + rl + e;
              vis = (qi < Sq) && (kw < Sk);
              if (CAUSAL) vis = vis && (kw <= qi);
              if (MASK == kMaskBool) {
                if (vis) vis = mask_u8[m_base + (int64_t)qi * a.m_si + kw] != 0;
              }
              if (MASK == kMaskAdd) {
                if (vis) x = x + (float)mask_bf[m_base + (int64_t)qi * a.m_si + kw] * kLog2e;
              }
            }
            const float p = vis ? fast_exp2(fminf(x - l2[e], 0.f)) : 0.f;
            s[qb][r] = p;
            dp[qb][r] = p * (dp[qb][r] - dl[e]);
          }
        }
      }

      // dV += P^T dO and dK += dS^T Q over 16-row slabs of the query tile.
#pragma unroll
      for (int kk = 0; kk < T::BM / 16; ++kk) {
        const int qb = kk >> 1, hs = (kk & 1) * 8;
        const bf16x8 pa = cvt8(s[qb][hs + 0], s[qb][hs + 1], s[qb][hs + 2], s[qb][hs + 3],
                               s[qb][hs + 4], s[qb][hs + 5], s[qb][hs + 6], s[qb][hs + 7]);
        const bf16x8 sa = cvt8(dp[qb][hs + 0], dp[qb][hs + 1], dp[qb][hs + 2], dp[qb][hs + 3],
                               dp[qb][hs + 4], dp[qb][hs + 5], dp[qb][hs + 6], dp[qb][hs + 7]);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const int off = (4 * kk + half) * T::TG + (db * 32 + l32) * 4;
          const bf16x8 ob = cat44(*reinterpret_cast<const bf16x4*>(dot_l + off),
                                  *reinterpret_cast<const bf16x4*>(dot_l + off + 2 * T::TG));
          const bf16x8 qbv = cat44(*reinterpret_cast<const bf16x4*>(qt_l + off),
                                   *reinterpret_cast<const bf16x4*>(qt_l + off + 2 * T::TG));
          dv[db] = mfma32(pa, ob, dv[db]);
          dk[db] = mfma32(sa, qbv, dk[db]);
        }
      }

      // dS -> LDS as [query][key] for the dQ product.
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ds_l[(qb * 32 + acc_row(r, half)) * T::SLD + wave * 32 + l32] = (bf16)dp[qb][r];
      __syncthreads();

      // dQ tiles: rows = queries, columns = d; k = the block's 128 keys.
#pragma unroll
      for (int tt = 0; tt < T::DQ_PER_WAVE; ++tt) {
        const int tile = wave * T::DQ_PER_WAVE + tt;
        const int qb = tile / T::DB, db = tile % T::DB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < T::BN / 16; ++kk) {
          const bf16x8 sa =
              *reinterpret_cast<const bf16x8*>(ds_l + (qb * 32 + l32) * T::SLD + kk * 16 + 8 * half);
          const int off = (4 * kk + 2 * half) * T::TG + (db * 32 + l32) * 4;
          const bf16x8 kbv = cat44(*reinterpret_cast<const bf16x4*>(kt_l + off),
                                   *reinterpret_cast<const bf16x4*>(kt_l + off + T::TG));
          acc = mfma32(sa, kbv, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qt0 + qb * 32 + acc_row(r, half);
          if (qi < Sq)
            unsafeAtomicAdd(a.dq_acc + ((qrow0 + qi) * a.H + head) * D + db * 32 + l32, acc[r]);
        }
      }
    }
  }

  // Epilogue: dK (times scale) and dV, bf16, contiguous [rows_k, Hkv, D].
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb0 + wave * 32 + acc_row(r, half);
      if (key < Sk) {
        const int64_t off = ((krow0 + key) * a.Hkv + g) * D + db * 32 + l32;
        reinterpret_cast<bf16*>(a.dk)[off] = (bf16)(dk[db][r] * sc);
        reinterpret_cast<bf16*>(a.dv)[off] = (bf16)dv[db][r];
      }
    }
  }
}

template <int D>
constexpr size_t bwd_smem_bytes() {
  using T = BwdTile<D>;
  return (size_t)(2 * T::Q_ELEMS + 2 * T::QT_ELEMS + T::KT_ELEMS + T::S_ELEMS) * 2 +
         2 * T::BM * sizeof(float);
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
