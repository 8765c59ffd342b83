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
//   one workgroup = NW waves = one (unit, head, query tile of 32*QB*NW rows);
//   each wave owns 32*QB query rows and keeps their Q fragments in registers;
//   K and V tiles of 64 keys are staged through LDS, double-buffered through registers,
//   loaded with buffer loads that return zero past the last key (no per-row branches).
// S^T = K Q^T is computed with 32x32x16 bf16 MFMAs so that a lane's accumulator holds one
// query column: row statistics are per lane plus one exchange with the partner lane
// (l ^ 32), the output rescale is a per-lane scalar, and the exponentiated scores feed
// the O^T += V^T P^T MFMA as its B operand straight from registers. V stays row-major in
// LDS; its A-operand fragments (four consecutive keys of one d per lane) come from
// transposed LDS reads.
//
// Rescaling: EAGER takes m_new = max(m_row, m_tile) on every tile. The lazy form keeps the
// running max while every row's tile max exceeds it by at most kLazyTau (log2 units), so
// exponentials are bounded by 2^kLazyTau and the accumulator is left alone; as soon as one
// row exceeds it, every lane takes max(m_row, m_tile) before exp2 (the FlyDSL PR #1033
// fix: a lane dragged into the rescale by the wave-wide decision gets a factor <= 1).

#include <type_traits>

#include "common.hpp"
#include "params.hpp"

namespace exattn {

constexpr float kLazyTau = 8.f;

template <int D, int NW, int QB>
struct FwdTile {
  static constexpr int NT = 64 * NW;         // threads per workgroup
  static constexpr int BM = NW * 32 * QB;    // query rows per workgroup
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KB = BN / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KLD = D + 8;          // K row pitch: 16 B mod 128 B, conflict-free b128
  static constexpr int VLD = D + 16;         // V row pitch: 32 B mod 128 B, conflict-free tr reads
  static constexpr int K_ELEMS = BN * KLD;
  static constexpr int V_ELEMS = BN * VLD;
  static constexpr int CH = BN * D / 8 / NT; // 16-byte chunks per thread, per tensor
  static_assert(CH * NT * 8 == BN * D, "tiles must split evenly over the threads");
};

template <bool B>
using bool_c = std::integral_constant<bool, B>;

template <int D, int NW, int QB, bool CAUSAL, int MASK, bool VARLEN, bool LAZY>
__global__ void __launch_bounds__(64 * NW) fwd_kernel(FwdArgs a) {
  using T = FwdTile<D, NW, QB>;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2 * T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2 * T::V_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform across the wave
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
  // Leading tiles that need no masking for any row of this workgroup.
  int n_plain = 0;
  if (MASK == kMaskNone) {
    int lim = Sk / T::BN;
    if (CAUSAL) lim = min(lim, (qt0 + 1) / T::BN);
    n_plain = min(lim, ntiles);
  }

  // Per-thread 16-byte chunks of a tile: row and column are fixed, the tile base moves.
  uint32_t k_off[T::CH], v_off[T::CH];
  int lds_k[T::CH], lds_v[T::CH];
#pragma unroll
  for (int i = 0; i < T::CH; ++i) {
    const int c = tid + i * T::NT;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    k_off[i] = (uint32_t)(row * a.k_ss + col) * 2u;
    v_off[i] = (uint32_t)(row * a.v_ss + col) * 2u;
    lds_k[i] = row * T::KLD + col;
    lds_v[i] = row * T::VLD + col;
  }
  u32x4 kr[T::CH], vr[T::CH];
  auto load_tile = [&](int t) {
    const int kb0 = t * T::BN;
    const int rows = min(T::BN, Sk - kb0);
    const auto rk = make_rsrc(K + (int64_t)kb0 * a.k_ss, (uint32_t)((rows - 1) * a.k_ss + D) * 2u);
    const auto rv = make_rsrc(V + (int64_t)kb0 * a.v_ss, (uint32_t)((rows - 1) * a.v_ss + D) * 2u);
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      kr[i] = buf_load16(rk, k_off[i]);
      vr[i] = buf_load16(rv, v_off[i]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      *reinterpret_cast<u32x4*>(k_lds + buf * T::K_ELEMS + lds_k[i]) = kr[i];
      *reinterpret_cast<u32x4*>(v_lds + buf * T::V_ELEMS + lds_v[i]) = vr[i];
    }
  };
  // Transposed-read address of this lane inside a V tile (16-lane group layout).
  const int grp = lane >> 4, j16 = lane & 15;
  const int v_rd = (4 * half + (j16 >> 2)) * T::VLD + 16 * (grp & 1) + 4 * (j16 & 3);

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

  // Visibility of key kj for this lane's query in block qb, and its additive bias (log2).
  auto visible = [&](int qb, int kj, float& b2) -> bool {
    const int qi = qw0 + qb * 32 + l32;
    bool vis = kj < Sk;
    if (CAUSAL) vis = vis && (kj <= qi);
    b2 = 0.f;
    if (MASK == kMaskBool) {
      if (vis && qi < Sq) vis = mask_u8[m_base + (int64_t)qi * a.m_si + kj] != 0;
    }
    if (MASK == kMaskAdd) {
      if (vis && qi < Sq) {
        const float bias = (float)mask_bf[m_base + (int64_t)qi * a.m_si + kj];
        vis = bias != -INFINITY;
        b2 = vis ? bias * kLog2e : 0.f;
      }
    }
    return vis;
  };

  auto tile = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
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
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Tile max of the scaled scores, mt (log2 units); masked entries become -inf.
      float mt;
      if constexpr (!MASKED) {
        float mx;
        if (c2 >= 0.f) {
          mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
          mx = fmaxf(mx, wave_xor32(mx));
        } else {
          mx = INFINITY;
#pragma unroll
          for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fminf(mx, s[kb][qb][r]);
          mx = fminf(mx, wave_xor32(mx));
        }
        mt = mx * c2;
      } else {
        // Masked tile: a visible entry contributes fma(s, c2, bias2) with bias2 the
        // additive mask in log2 units (0 otherwise), the same rounding as the plain path.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float b2;
            const bool vis = visible(qb, kb0 + kb * 32 + acc_row(r, half), b2);
            mx = fmaxf(mx, vis ? fmaf(s[kb][qb][r], c2, b2) : -INFINITY);
          }
        }
        mt = fmaxf(mx, wave_xor32(mx));
      }
      // Rescale decision, wave-uniform. Eager: whenever some row's max grows (a factor of
      // exactly 1 elsewhere leaves those rows unchanged). Lazy: only when some row's tile
      // max exceeds its running max by more than kLazyTau.
      const float thr = LAZY ? kLazyTau : 0.f;
      if (__builtin_amdgcn_ballot_w64(mt > m_run[qb] + thr) != 0) {
        // Per-row max first, then exp2: the factor is <= 1 on every lane.
        const float m_new = fmaxf(m_run[qb], mt);
        const float corr = fast_exp2(m_run[qb] - ((m_new == -INFINITY) ? 0.f : m_new));
        l_run[qb] *= corr;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) o[db][qb] *= corr;
        m_run[qb] = m_new;
      }
      const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float rs = 0.f;
      if constexpr (!MASKED) {
        const float nm = -m_use;
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[kb][qb][r], c2, nm));
            s[kb][qb][r] = p;
            rs += p;
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float b2;
            const bool vis = visible(qb, kb0 + kb * 32 + acc_row(r, half), b2);
            const float p = vis ? fast_exp2(fmaf(s[kb][qb][r], c2, b2 - m_use)) : 0.f;
            s[kb][qb][r] = p;
            rs += p;
          }
        }
      }
      l_run[qb] += rs;
    }

    // O^T += V^T P^T over 16-key slabs; V^T fragments by transposed reads.
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
        // slots 0-3: keys 16kk + 4h + 0..3, slots 4-7: keys 16kk + 8 + 4h + 0..3
        const bf16* vp = vl + (16 * kk) * T::VLD + db * 32 + v_rd;
        const bf16x8 af = cat44(lds_read_tr4(vp), lds_read_tr4(vp + 8 * T::VLD));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma32(af, pf[qb], o[db][qb]);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  };

  int t = 0;
  for (; t < n_plain; ++t) tile(t, bool_c<false>{});
  for (; t < ntiles; ++t) tile(t, bool_c<true>{});

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

// Variants: 0 = 8 waves x 32 rows, lazy rescale (default); 1 = 8 waves x 32 rows, eager
// rescale; 2 = 4 waves x 64 rows, lazy; 3 = 4 waves x 32 rows, lazy. Variants 2 and 3 are
// compiled for head_dim 128 without a mask; other problems use variant 0 or 1.
static int g_fwd_variant = 0;

void set_fwd_variant(int v) { g_fwd_variant = (v >= 0 && v <= 3) ? v : 0; }
int get_fwd_variant() { return g_fwd_variant; }

static int effective_variant(int head_dim, int mask, bool varlen) {
  const int v = g_fwd_variant;
  if (v >= 2 && (head_dim != 128 || mask != kMaskNone || varlen)) return 0;
  return v;
}

int fwd_block_m(int head_dim, int mask, bool varlen) {
  const int v = effective_variant(head_dim, mask, varlen);
  return v == 2 ? 256 : (v == 3 ? 128 : 256);
}

template <int D, int NW, int QB, bool LAZY>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  const int64_t nblk = (int64_t)a.num_units * a.H * a.num_q_tiles;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(64 * NW);
#define EXATTN_FWD(C, M, V) \
  hipLaunchKernelGGL((fwd_kernel<D, NW, QB, C, M, V, LAZY>), grid, block, 0, s, a)
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

template <int NW, int QB>
static hipError_t launch_fwd_plain128(const FwdArgs& a, bool causal, hipStream_t s) {
  const int64_t nblk = (int64_t)a.num_units * a.H * a.num_q_tiles;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(64 * NW);
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<128, NW, QB, true, kMaskNone, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<128, NW, QB, false, kMaskNone, false, true>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool causal, int mask, bool varlen,
                      hipStream_t s) {
  const int v = effective_variant(head_dim, mask, varlen);
  if (head_dim == 64) {
    if (v == 1) return launch_fwd_d<64, 8, 1, false>(a, causal, mask, varlen, s);
    return launch_fwd_d<64, 8, 1, true>(a, causal, mask, varlen, s);
  }
  if (v == 1) return launch_fwd_d<128, 8, 1, false>(a, causal, mask, varlen, s);
  if (v == 2) return launch_fwd_plain128<4, 2>(a, causal, s);
  if (v == 3) return launch_fwd_plain128<4, 1>(a, causal, s);
  return launch_fwd_d<128, 8, 1, true>(a, causal, mask, varlen, s);
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
