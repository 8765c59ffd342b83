// Forward kernel: tiled exact softmax attention with an online softmax and an LSE output.
//
// What it computes follows FlyDSL PR #1033 ("[Bugfix][Kernel] Fix NaN from the lazy rescale
// on a wide score range", sections "Root cause" and "The fix"): a running row max m and
// row sum l; for each key tile the new max is max(m_row, m_tile) taken per row before any
// exp2, so every exponent is <= 0 and the rescale factor of the output accumulator is <= 1.
// Masked keys (partial last tile, causal, bool/additive mask, packed-sequence bounds) are
// removed inside the kernel (OpenWAM PR #64, "Summary"/"Fix").
//
// Work decomposition (gfx950, 64-wide waves):
//   one workgroup = 4 waves = one (unit, head, query tile of 128*QB rows);
//   each wave owns 32*QB query rows and keeps their Q fragments in registers;
//   K and V tiles of 64 keys are staged through LDS, double-buffered through registers.
// S^T = K Q^T is computed with 32x32x16 bf16 MFMAs so that a lane's accumulator holds one
// query column: row statistics are per lane plus one exchange with the partner lane
// (l ^ 32), the output rescale is a per-lane scalar, and the exponentiated scores feed
// the O^T += V^T P^T MFMA as its B operand straight from registers. V is stored in LDS
// as V[key/4][d][key%4] so one 8-byte read gives a lane four consecutive keys of one d.

#include "common.hpp"
#include "params.hpp"

namespace exattn {

template <int D, int QB>
struct FwdTile {
  static constexpr int NW = 4;
  static constexpr int BM = NW * 32 * QB;
  static constexpr int BN = 64;
  static constexpr int KB = BN / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KLD = D + 8;          // K row pitch (elements), breaks bank aliasing
  static constexpr int VG = D * 4 + 8;       // pitch of one 4-key group of V
  static constexpr int K_ELEMS = BN * KLD;
  static constexpr int V_ELEMS = (BN / 4) * VG;
  static constexpr int KCH = BN * D / 8 / 256;   // 16-byte K chunks per thread
  static constexpr int VGR = (BN / 4) * (D / 8); // 4x8 V blocks per tile
};

template <int D, int QB, bool CAUSAL, int MASK, bool VARLEN>
__global__ void __launch_bounds__(256) fwd_kernel(FwdArgs a) {
  using T = FwdTile<D, QB>;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2 * T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2 * T::V_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qtile = blk % a.num_q_tiles;
  const int uh = blk / a.num_q_tiles;
  const int head = uh % a.H, unit = uh / a.H, g = head / a.group;
  if (CAUSAL) qtile = a.num_q_tiles - 1 - qtile;  // longest rows first

  int Sq, Sk;
  int64_t q_base, k_base, v_base, o_base, lse_base, m_base = 0;
  if constexpr (VARLEN) {
    const int qs = a.cu_q[unit], ks = a.cu_k[unit];
    Sq = a.cu_q[unit + 1] - qs;
    Sk = a.cu_k[unit + 1] - ks;
    q_base = (int64_t)qs * a.q_ss + (int64_t)head * a.q_sh;
    k_base = (int64_t)ks * a.k_ss + (int64_t)g * a.k_sh;
    v_base = (int64_t)ks * a.v_ss + (int64_t)g * a.v_sh;
    o_base = (int64_t)qs * a.o_ss + (int64_t)head * a.o_sh;
    lse_base = (int64_t)head * a.lse_row + qs;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
    q_base = (int64_t)unit * a.q_sb + (int64_t)head * a.q_sh;
    k_base = (int64_t)unit * a.k_sb + (int64_t)g * a.k_sh;
    v_base = (int64_t)unit * a.v_sb + (int64_t)g * a.v_sh;
    o_base = (int64_t)unit * a.o_sb + (int64_t)head * a.o_sh;
    lse_base = ((int64_t)unit * a.H + head) * a.Sq;
    m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;
  }
  const int qt0 = qtile * T::BM;
  if (qt0 >= Sq) return;

  const bf16* Q = reinterpret_cast<const bf16*>(a.q) + q_base;
  const bf16* K = reinterpret_cast<const bf16*>(a.k) + k_base;
  const bf16* V = reinterpret_cast<const bf16*>(a.v) + v_base;

  // Q fragments of this wave's rows, B-operand layout (column = query, k-slots = d).
  const int qw0 = qt0 + wave * 32 * QB;
  bf16x8 qf[QB][T::DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + qb * 32 + l32;
    if (qi < Sq) {
      const bf16* row = Q + (int64_t)qi * a.q_ss + 8 * half;
#pragma unroll
      for (int s = 0; s < T::DS; ++s) qf[qb][s] = *reinterpret_cast<const bf16x8*>(row + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < T::DS; ++s) qf[qb][s] = bf16x8{};
    }
  }

  const int kend = CAUSAL ? min(Sk, qt0 + T::BM) : Sk;
  const int ntiles = (kend + T::BN - 1) / T::BN;

  // Register staging of the next K/V tile.
  u32x4 kr[T::KCH];
  u32x4 vr[4];
  const bool v_thread = (T::VGR >= 256) || (tid < T::VGR);
  const int vg4 = tid / (D / 8), vd8 = tid % (D / 8);

  auto load_tile = [&](int t) {
    const int kb0 = t * T::BN;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + i * 256;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = kb0 + row;
      kr[i] = key < Sk ? ldg16(K + (int64_t)key * a.k_ss + col) : u32x4{0, 0, 0, 0};
    }
    if (v_thread) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb0 + 4 * vg4 + i;
        vr[i] = key < Sk ? ldg16(V + (int64_t)key * a.v_ss + vd8 * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16* kl = k_lds + buf * T::K_ELEMS;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + i * 256;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(kl + row * T::KLD + col) = kr[i];
    }
    if (v_thread)
      store_4x8_transposed(v_lds + buf * T::V_ELEMS + vg4 * T::VG + vd8 * 32, vr[0], vr[1], vr[2],
                           vr[3]);
  };

  f32x16 o[T::DB][QB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) o[db][qb] = f32x16{};
  }

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const bf16* kl = k_lds + buf * T::K_ELEMS;
    const bf16* vl = v_lds + buf * T::V_ELEMS;

    // S^T tile: rows = keys, columns = this wave's queries.
    f32x16 s[T::KB][QB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < T::DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(kl + (kb * 32 + l32) * T::KLD + ds * 16 + 8 * half);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(af, qf[qb][ds], s[kb][qb]);
      }
    }

    const int kb0 = t * T::BN;
    const bool edge = (kb0 + T::BN > Sk) || (MASK != kMaskNone) || (CAUSAL && kb0 + T::BN - 1 > qw0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw0 + qb * 32 + l32;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][qb][r] * c2;
          if (edge) {
            const int kj = kb0 + kb * 32 + acc_row(r, half);
            bool vis = kj < Sk;
            if (CAUSAL) vis = vis && (kj <= qi);
            if (MASK == kMaskBool) {
              if (vis && qi < Sq) vis = mask_u8[m_base + (int64_t)qi * a.m_si + kj] != 0;
            }
            if (MASK == kMaskAdd) {
              if (vis && qi < Sq)
                x = x + (float)mask_bf[m_base + (int64_t)qi * a.m_si + kj] * kLog2e;
            }
            x = vis ? x : -INFINITY;
          }
          s[kb][qb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, wave_xor32(mx));
      // Per-row max first, then exp2: exponents are never positive.
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float corr = fast_exp2(m_run[qb] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[kb][qb][r] - m_use);
          s[kb][qb][r] = p;
          rs += p;
        }
      }
      l_run[qb] = l_run[qb] * corr + rs;
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) o[db][qb] *= corr;
    }

    // O^T += V^T P^T over 16-key slabs.
#pragma unroll
    for (int kk = 0; kk < T::BN / 16; ++kk) {
      const int kb = kk >> 1, hs = (kk & 1) * 8;
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        pf[qb] = cvt8(s[kb][qb][hs + 0], s[kb][qb][hs + 1], s[kb][qb][hs + 2], s[kb][qb][hs + 3],
                      s[kb][qb][hs + 4], s[kb][qb][hs + 5], s[kb][qb][hs + 6], s[kb][qb][hs + 7]);
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const bf16* vp = vl + (4 * kk + half) * T::VG + (db * 32 + l32) * 4;
        const bf16x8 af = cat44(*reinterpret_cast<const bf16x4*>(vp),
                                *reinterpret_cast<const bf16x4*>(vp + 2 * T::VG));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma32(af, pf[qb], o[db][qb]);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: normalise, write out (bf16, RNE) and lse (natural log).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + qb * 32 + l32;
    const float l = l_run[qb] + wave_xor32(l_run[qb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qi < Sq) {
      bf16* orow = reinterpret_cast<bf16*>(a.out) + o_base + (int64_t)qi * a.o_ss;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d = db * 32 + 8 * rg + 4 * half;
          f32x4 vv = {o[db][qb][4 * rg + 0] * inv, o[db][qb][4 * rg + 1] * inv,
                      o[db][qb][4 * rg + 2] * inv, o[db][qb][4 * rg + 3] * inv};
          *reinterpret_cast<bf16x4*>(orow + d) = __builtin_convertvector(vv, bf16x4);
        }
      }
      if (half == 0) {
        const float mu = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
        a.lse[lse_base + qi] = l > 0.f ? (mu + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

// Rows of a packed output past cu_seqlens_q[num_seqs]: out = 0, lse = -inf.
template <int D>
__global__ void __launch_bounds__(256) fwd_tail_kernel(FwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.Sq * a.H) return;
  const int row = (int)(idx / a.H), head = (int)(idx % a.H);
  if (row < a.cu_q[a.num_units]) return;
  bf16* o = reinterpret_cast<bf16*>(a.out) + (int64_t)row * a.o_ss + (int64_t)head * a.o_sh;
#pragma unroll
  for (int d = 0; d < D; d += 8) *reinterpret_cast<u32x4*>(o + d) = u32x4{0, 0, 0, 0};
  a.lse[(int64_t)head * a.lse_row + row] = -INFINITY;
}

int fwd_block_m(int head_dim) { return FwdTile<128, 1>::BM; }

template <int D, int QB>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  const int64_t nblk = (int64_t)a.num_units * a.H * a.num_q_tiles;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(256);
#define EXATTN_FWD(C, M, V) hipLaunchKernelGGL((fwd_kernel<D, QB, C, M, V>), grid, block, 0, s, a)
  if (varlen) {
    if (causal) EXATTN_FWD(true, kMaskNone, true);
    else EXATTN_FWD(false, kMaskNone, true);
  } else if (causal) {
    if (mask == kMaskBool) EXATTN_FWD(true, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_FWD(true, kMaskAdd, false);
    else EXATTN_FWD(true, kMaskNone, false);
  } else {
    if (mask == kMaskBool) EXATTN_FWD(false, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_FWD(false, kMaskAdd, false);
    else EXATTN_FWD(false, kMaskNone, false);
  }
#undef EXATTN_FWD
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool causal, int mask, bool varlen,
                      hipStream_t s) {
  if (head_dim == 64) return launch_fwd_d<64, 1>(a, causal, mask, varlen, s);
  return launch_fwd_d<128, 1>(a, causal, mask, varlen, s);
}

hipError_t launch_fwd_tail(const FwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t n = (int64_t)a.Sq * a.H;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (head_dim == 64) hipLaunchKernelGGL((fwd_tail_kernel<64>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((fwd_tail_kernel<128>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace exattn
