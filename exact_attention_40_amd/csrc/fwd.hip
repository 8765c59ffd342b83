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
//   one workgroup = NW waves = one (unit, head, query tile of 32*NW rows); each wave owns
//   32 query rows and keeps their Q fragments in registers; K and V tiles of 64 keys are
//   copied straight from global memory into XOR-swizzled LDS (buffer loads with an LDS
//   destination, zero past the last key), K one tile further ahead than V.
// S^T = K Q^T is computed with 32x32x16 MFMAs (bf16 or fp16 inputs) so that a lane's accumulator holds one
// query column: row statistics are per lane plus one exchange with the partner lane
// (l ^ 32), the output rescale is a per-lane scalar, and the exponentiated scores feed
// the O^T += V^T P^T MFMA as its B operand straight from registers. V stays row-major in
// LDS; its A-operand fragments (four consecutive keys of one d per lane) come from
// transposed LDS reads. The swizzle keeps both the K row reads and the V transposed reads
// free of bank conflicts.
//
// Software pipeline: iteration t issues the S MFMAs of tile t+1 next to the exponentials of
// tile t (independent work for the matrix and vector units of the same SIMD), then
// O += V_t P_t next to the row max of tile t+1. The rescale for tile t+1 is decided after
// that, outside the matrix work, so no branch splits the interleaved region.
//
// Rescaling: EAGER takes m_new = max(m_row, m_tile) whenever a row's max grows. The lazy
// form keeps the running max while every row's tile max exceeds it by at most kLazyTau
// (log2 units), so exponentials are bounded by 2^kLazyTau and the accumulator is left
// alone; as soon as one row exceeds it, every lane takes max(m_row, m_tile) before exp2
// (the FlyDSL PR #1033 fix: a lane dragged into the rescale by the wave-wide decision gets
// a factor <= 1).

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
  static constexpr int RB = D * 2;           // bytes per LDS row (swizzled, no padding)
  static constexpr int TBYTES = BN * RB;     // one K or V tile
  static_assert((BN * D / 8) % NT == 0, "tiles must split evenly over the threads");
};

template <bool B>
using bool_c = std::integral_constant<bool, B>;
template <int I>
using int_c = std::integral_constant<int, I>;

// QB = 1: two waves per SIMD (8 waves x 32 rows); QB = 2: one wave per SIMD (4 waves x 64
// rows), which halves the LDS reads per MFMA and relies on the in-stream interleave alone.
template <class E, int D, int NW, int QB, bool CAUSAL, int MASK, bool VARLEN, bool LAZY>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(QB == 1 ? 2 : 1)))
fwd_kernel(FwdArgs a) {
  using T = FwdTile<D, NW, QB>;
  using V8 = typename Ty<E>::v8;
  using V4 = typename Ty<E>::v4;
  constexpr int RB = T::RB;
  constexpr int V_OFF = 2 * T::TBYTES;           // V buffers follow the two K buffers
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * T::TBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform across the wave
  const int half = lane >> 5, l32 = lane & 31;
  const uint32_t lds0 = lds_addr(smem);                        // LDS byte address of smem

  // Dense: consecutive blocks are the query tiles of one (unit, head), which share K/V in
  // one XCD's L2. Packed: query-tile index outermost, highest first, so that the longest
  // blocks of every sequence (whatever its length) start before the short ones; without
  // the XCD remap, so that each tile layer (heavy high layers, light low ones) is spread
  // over all XCDs instead of one XCD taking the heavy layers.
  // Dense causal: block j of a (unit, head) runs query tiles n-1-j and j one after the
  // other (tile i sees i+1 key tiles), so every block has the same amount of work and no
  // long tile is left for the end of the grid.
  const int blk = VARLEN ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  int qtile, qtile2 = -1, uh;
  if constexpr (VARLEN) {
    const int nuh = a.num_units * a.H;
    qtile = a.num_q_tiles - 1 - blk / nuh;
    uh = blk % nuh;
  } else if constexpr (CAUSAL) {
    const int npair = (a.num_q_tiles + 1) / 2;
    const int j = blk % npair;
    uh = blk / npair;
    qtile = a.num_q_tiles - 1 - j;
    if (j != qtile) qtile2 = j;
  } else {
    qtile = blk % a.num_q_tiles;
    uh = blk / a.num_q_tiles;
  }
  const int head = uh % a.H, unit = uh / a.H, g = head / a.group;

  int Sq, Sk;
  int64_t q_base, k_base, v_base, o_base, lse_base, m_base = 0;
  if constexpr (VARLEN) {
    const SeqRows rq = seq_rows(a.cu_q, unit, a.Sq, a.max_sq);
    const SeqRows rk = seq_rows(a.cu_k, unit, a.Sk, a.max_sk);
    const int qs = rq.beg, ks = rk.beg;
    Sq = rq.len;
    Sk = rk.len;
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
  // One query tile of BM rows; the workgroup runs one or two of them.
  auto run_tile = [&](const int qtile) __attribute__((always_inline)) {
  const int qt0 = qtile * T::BM;
  if (qt0 >= Sq) return;

  const E* Q = reinterpret_cast<const E*>(a.q) + q_base;
  const E* K = reinterpret_cast<const E*>(a.k) + k_base;
  const E* V = reinterpret_cast<const E*>(a.v) + v_base;

  // A negative scale is folded into the sign of Q: (-q).k * |c| equals q.k * c exactly
  // (negation commutes with every rounding), so the row max is always a max.
  const float c2s = a.scale_log2;
  const float c2 = fabsf(c2s);
  const uint32_t qsign = c2s < 0.f ? 0x80008000u : 0u;

  // Q fragments of this lane's query rows, B-operand layout (column = query, k-slots = d).
  int qi[QB];
  V8 qf[QB][T::DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qi[qb] = qt0 + (wave * QB + qb) * 32 + l32;
    if (qi[qb] < Sq) {
      const E* row = Q + (int64_t)qi[qb] * a.q_ss + 8 * half;
#pragma unroll
      for (int s = 0; s < T::DS; ++s)
        qf[qb][s] = __builtin_bit_cast(V8, ldg16(row + 16 * s) ^ u32x4{qsign, qsign, qsign, qsign});
    } else {
#pragma unroll
      for (int s = 0; s < T::DS; ++s) qf[qb][s] = V8{};
    }
  }
  // Consume the Q loads before the tile loop: otherwise the compiler keeps waiting for them
  // inside the loop, where its vmcnt waits would also wait for the K/V copies in flight.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < T::DS; ++s) asm volatile("" ::"v"(qf[qb][s]));

  const int kend = CAUSAL ? min(Sk, qt0 + T::BM) : Sk;
  const int ntiles = (kend + T::BN - 1) / T::BN;
  // Leading tiles that need no masking for any row of this workgroup.
  int n_plain = 0;
  if (MASK == kMaskNone) {
    int lim = Sk / T::BN;
    if (CAUSAL) lim = min(lim, (qt0 + 1) / T::BN);
    n_plain = min(lim, ntiles);
  }

  auto load_k = [&](int t, int buf) {
    const int kb0 = t * T::BN;
    const int rows = min(T::BN, Sk - kb0);
    copy_tile_async<D, T::BN, NW>(lds0 + buf * T::TBYTES,
                                  copy_rsrc(K + (int64_t)kb0 * a.k_ss, (uint32_t)((rows - 1) * a.k_ss + D) * 2u),
                                  (int)a.k_ss, wave, lane);
  };
  auto load_v = [&](int t, int buf) {
    const int kb0 = t * T::BN;
    const int rows = min(T::BN, Sk - kb0);
    copy_tile_async<D, T::BN, NW>(lds0 + V_OFF + buf * T::TBYTES,
                                  copy_rsrc(V + (int64_t)kb0 * a.v_ss, (uint32_t)((rows - 1) * a.v_ss + D) * 2u),
                                  (int)a.v_ss, wave, lane);
  };
  // Per-lane LDS bases. K row reads: key kb*32 + l32, 16-byte chunk 2*ds + half. V^T
  // transposed reads: keys 16kk + 4*half + (j16>>2) + 8*sec, d = db*32 + 16*(grp&1) +
  // 4*(j16&3). The swizzle depends on the row's low four bits only, so kb, kk and the
  // buffer are immediate offsets.
  const int grp = lane >> 4, j16 = lane & 15;
  const unsigned char* ar[T::DS];
#pragma unroll
  for (int ds = 0; ds < T::DS; ++ds) ar[ds] = smem + l32 * RB + 16 * ((2 * ds + half) ^ swz_f<D>(l32));
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  const unsigned char* tv[T::DB][2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 4 * half + (j16 >> 2) + 8 * sec;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
      tv[db][sec] = smem + V_OFF + row * RB + 16 * ((4 * db + clow) ^ swz_f<D>(row)) + 8 * (j16 & 1);
  }

  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);

  // Visibility of key kj for query row `row` and its additive bias in log2 units.
  // Branch-free: the mask is read at indices clamped into [0, Sq) x [0, Sk), so every read
  // is in range, and the result is used only for in-range pairs.
  auto visible = [&](int row, int kj, float& b2) -> bool {
    bool vis = (kj < Sk) && (row < Sq);
    if (CAUSAL) vis = vis && (kj <= row);
    b2 = 0.f;
    if (MASK != kMaskNone) {
      const int64_t mi = m_base + (int64_t)min(row, Sq - 1) * a.m_si + min(kj, Sk - 1);
      if (MASK == kMaskBool) {
        vis = vis && (mask_u8[mi] != 0);
      } else {
        const float bias = (float)mask_bf[mi];
        vis = vis && (bias != -INFINITY);
        b2 = vis ? bias_log2(bias) : 0.f;
      }
    }
    return vis;
  };

  f32x16 o[QB][T::DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) o[qb][db] = f32x16{};
  }

  // Rescale decision for query block qb whose tile max is mt, wave-uniform. Eager:
  // whenever some row's max grows (a factor of exactly 1 elsewhere leaves those rows
  // unchanged). Lazy: only when some row's tile max exceeds its running max by more than
  // kLazyTau. Per-row max first, then exp2: the factor is <= 1 on every lane.
  auto update_max = [&](int qb, float mt) {
    const float thr = LAZY ? kLazyTau : 0.f;
    if (__builtin_amdgcn_ballot_w64(mt > m_run[qb] + thr) != 0) {
      const float m_new = fmaxf(m_run[qb], mt);
      const float corr = fast_exp2(m_run[qb] - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run[qb] *= corr;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) o[qb][db] *= corr;
      m_run[qb] = m_new;
    }
  };

  // Scores of tile t (cur) and t+1 (nxt): [QB][KB] accumulators, rows = keys, columns =
  // this wave's queries. Element e of a score set is (qb, kb, r) = (e / (16 KB),
  // (e / 16) % KB, e % 16), the order of every sweep below.
  using Scores = f32x16[QB][T::KB];
  constexpr int NE = QB * T::KB * 16;           // score elements per lane

  // Row max of tile t's scores in log2 units (prologue only).
  auto first_max = [&](const Scores& sc, int t, auto masked_tag, float (&mt)[QB]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (!MASKED) {
            mx = fmaxf(mx, sc[qb][kb][r]);
          } else {
            float b2;
            const bool vis = visible(qi[qb], t * T::BN + kb * 32 + acc_row(r, half), b2);
            mx = fmaxf(mx, vis ? fmaf(sc[qb][kb][r], c2, b2) : -INFINITY);
          }
        }
      }
      mx = pair_max32(mx);
      mt[qb] = MASKED ? mx : mx * c2;
    }
  };

  // Iteration body as one instruction stream:
  //   QK phase: the S MFMAs of tile t+1 (16 K fragments, each used for QB MFMAs; fragments
  //             read three ahead) with two exponentials of tile t per MFMA, and the
  //             transposed V reads for the first two PV slabs over the last 8 fragments;
  //   PV phase: the PV MFMAs of tile t (each V fragment used for QB MFMAs) with two
  //             elements of tile t+1's row max per MFMA and the remaining V reads two slabs
  //             ahead.
  // Scheduling fences (only scalar instructions may cross) keep this order, so the matrix
  // and vector work of one wave overlap. MC / MN: tile t / t+1 needs masking. Unmasked,
  // the row max of s * c2 is c2 * max(s) (c2 >= 0); masked, a visible entry counts as
  // fma(s, c2, bias2), the rounding the exponent uses. Writes tile t+1's row max (log2
  // units) to mt.
  auto body = [&](Scores& nxt, Scores& cur, int t, auto par_tag, auto mc_tag, auto mn_tag,
                  float (&mt)[QB]) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool MC = decltype(mc_tag)::value;
    constexpr bool MN = decltype(mn_tag)::value;
    constexpr int KO = (PAR ^ 1) * T::TBYTES;   // K of tile t + 1
    constexpr int VB = PAR * T::TBYTES;         // V of tile t
    constexpr int NF = T::DS * T::KB;           // K fragments
    constexpr int QSTEPS = NF * QB;             // S MFMAs
    constexpr int NKK = T::BN / 16;             // PV slabs
    constexpr int PSTEPS = NKK * T::DB * QB;    // PV MFMAs
    constexpr int PER = NE / QSTEPS;            // exponentials per S MFMA
    constexpr int MPER = NE / PSTEPS;           // max elements per PV MFMA
    static_assert(NF >= 8 && NKK == 4 && PER * QSTEPS == NE && MPER * PSTEPS == NE &&
                  MPER % 2 == 0 && (16 * T::KB) % MPER == 0, "schedule shape");
    const int kc0 = t * T::BN, kn0 = kc0 + T::BN;
    float m_use[QB], rs[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_use[qb] = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
#pragma unroll
      for (int j = 0; j < 4; ++j) rs[qb][j] = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) nxt[qb][kb] = f32x16{};
    }
    auto kfrag = [&](int f) { return lds_at<V8>(ar[f / T::KB], KO + (f % T::KB) * 32 * RB); };
    auto vfrag = [&](int kk, int db, int sec) { return tr_at<V4>(tv[db][sec], VB + 16 * kk * RB); };
    V8 kf[3] = {kfrag(0), kfrag(1), kfrag(2)};
    V4 vt[2][T::DB][2];
#pragma unroll
    for (int i = 0; i < QSTEPS; ++i) {
      const int f = i / QB, qb = i % QB;
      const int ds = f / T::KB, kb = f % T::KB;
      nxt[qb][kb] = mfma32(kf[f % 3], qf[qb][ds], nxt[qb][kb]);
      if (qb == QB - 1 && f + 3 < NF) kf[f % 3] = kfrag(f + 3);
      // transposed reads of slabs 0 and 1 over the last eight fragments
      const int j = f - (NF - 8);
      if (qb == 0 && j >= 0) {
        const int kk = j / 4, db = j % 4;
        if (db < T::DB) {
          vt[kk][db][0] = vfrag(kk, db, 0);
          vt[kk][db][1] = vfrag(kk, db, 1);
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = PER * i + u;
        const int eq = e / (16 * T::KB), cb = (e / 16) % T::KB, r = e % 16;
        float pe;
        if constexpr (!MC) {
          pe = fast_exp2(fmaf(cur[eq][cb][r], c2, -m_use[eq]));
        } else {
          float b2;
          const bool vis = visible(qi[eq], kc0 + cb * 32 + acc_row(r, half), b2);
          pe = vis ? fast_exp2(fmaf(cur[eq][cb][r], c2, b2 - m_use[eq])) : 0.f;
        }
        cur[eq][cb][r] = pe;
        asm volatile("" : "+v"(cur[eq][cb][r]));   // pin this step's exponential here
      }
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int kb = kk >> 1, hs = (kk & 1) * 8;
      V8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
      {
        pf[qb] = cvt8<V8>(cur[qb][kb][hs + 0], cur[qb][kb][hs + 1], cur[qb][kb][hs + 2],
                      cur[qb][kb][hs + 3], cur[qb][kb][hs + 4], cur[qb][kb][hs + 5],
                      cur[qb][kb][hs + 6], cur[qb][kb][hs + 7]);
        // the row sum adds the exponentials as the P.V product sees them (rounded to the
        // input format), two per instruction, so the output's weights sum to exactly 1
        const u32x4 pw = __builtin_bit_cast(u32x4, pf[qb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[qb][j] = add_pair<E>(pw[j], rs[qb][j]);
      }
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          o[qb][db] = mfma32(cat44(vt[kk & 1][db][0], vt[kk & 1][db][1]), pf[qb], o[qb][db]);
          if (qb == QB - 1 && kk + 2 < NKK) {
            vt[kk & 1][db][0] = vfrag(kk + 2, db, 0);
            vt[kk & 1][db][1] = vfrag(kk + 2, db, 1);
          }
          const int step = (kk * T::DB + db) * QB + qb;
#pragma unroll
          for (int u = 0; u < MPER; u += 2) {
            // a pair never straddles two query blocks (16 KB is a multiple of MPER)
            const int e0 = MPER * step + u, e1 = e0 + 1;
            const int q0 = e0 / (16 * T::KB), b0i = (e0 / 16) % T::KB, r0 = e0 % 16;
            const int b1i = (e1 / 16) % T::KB, r1 = e1 % 16;
            float x0 = nxt[q0][b0i][r0], x1 = nxt[q0][b1i][r1];
            if constexpr (MN) {
              float bb0, bb1;
              const bool v0 = visible(qi[q0], kn0 + b0i * 32 + acc_row(r0, half), bb0);
              const bool v1 = visible(qi[q0], kn0 + b1i * 32 + acc_row(r1, half), bb1);
              x0 = v0 ? fmaf(x0, c2, bb0) : -INFINITY;
              x1 = v1 ? fmaf(x1, c2, bb1) : -INFINITY;
            }
            mx[q0] = fmaxf(fmaxf(mx[q0], x0), x1);
            asm volatile("" : "+v"(mx[q0]));   // pin this step's part of the max chain here
          }
          __builtin_amdgcn_sched_barrier(0x0004);
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      asm volatile("" : "+v"(mx[qb]));   // keep the max chain inside the stream
      mt[qb] = MN ? pair_max32(mx[qb]) : pair_max32(mx[qb]) * c2;
      l_run[qb] += (rs[qb][0] + rs[qb][1]) + (rs[qb][2] + rs[qb][3]);
    }
  };

  // Tile j's K lives in K buffer j & 1 and its V in V buffer j & 1.
  Scores sa, sb;
  if (ntiles > 0) {
    load_k(0, 0);
    load_v(0, 0);
  }
  if (ntiles > 1) load_k(1, 1);
  sync_copies<0>();
  if (ntiles > 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) sa[qb][kb] = f32x16{};
    }
#pragma unroll
    for (int ds = 0; ds < T::DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const V8 kfr = lds_at<V8>(ar[ds], kb * 32 * RB);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sa[qb][kb] = mfma32(kfr, qf[qb][ds], sa[qb][kb]);
      }
    }
    float mt[QB];
    if (n_plain > 0) first_max(sa, 0, bool_c<false>{}, mt);
    else first_max(sa, 0, bool_c<true>{}, mt);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) update_max(qb, mt[qb]);
  }
  __syncthreads();  // every wave has read K_0 before K_2 replaces it

  // Iteration t. Buffers: K tile t (parity PAR) was consumed by the previous iteration and
  // is refilled with K_{t+2}; V buffer PAR ^ 1 (V_{t-1}) is refilled with V_{t+1}. When
  // t + 1 == ntiles the S MFMAs read a stale K buffer and their result is discarded.
  auto iteration = [&](int t, Scores& cur, Scores& nxt, auto par_tag, auto mask_cur,
                       auto mask_nxt) {
    constexpr int PAR = decltype(par_tag)::value;
    if (t + 2 < ntiles) load_k(t + 2, PAR);
    if (t + 1 < ntiles) load_v(t + 1, PAR ^ 1);
    float mt[QB];
    body(nxt, cur, t, par_tag, mask_cur, mask_nxt, mt);
    if (t + 1 < ntiles) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) update_max(qb, mt[qb]);
    }
    sync_copies<0>();  // every wave's part of K_{t+2} and V_{t+1} has landed in LDS; every
                       // wave is done with K_{t+1} and V_t
  };

  using F = bool_c<false>;
  using Tr = bool_c<true>;
  int t = 0;
  for (; t + 2 < n_plain; t += 2) {
    iteration(t, sa, sb, int_c<0>{}, F{}, F{});
    iteration(t + 1, sb, sa, int_c<1>{}, F{}, F{});
  }
  // Remaining tiles (the masked ones and at most two unmasked ones before them) take the
  // masked form, still in pairs so that the pending scores of the next tile live in sa at
  // the top of the loop. One form per loop keeps the register allocation of the two loops
  // independent (a run-time choice between forms inside one loop costs spills).
  for (; t < ntiles; t += 2) {
    iteration(t, sa, sb, int_c<0>{}, Tr{}, Tr{});
    if (t + 1 < ntiles) iteration(t + 1, sb, sa, int_c<1>{}, Tr{}, Tr{});
  }

  // Epilogue: normalise, write out (input format, RNE) through this wave's slice of LDS (every wave
  // has passed the last barrier, so the K/V buffers are free) and lse (natural log).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = l_run[qb] + wave_xor32(l_run[qb]);
    const float inv = l != 0.f ? 1.f / l : 0.f;   // NaN propagates
    const int r0 = qt0 + (wave * QB + qb) * 32;
    E* orow = reinterpret_cast<E*>(a.out) + o_base + (int64_t)r0 * a.o_ss;
    static_assert(NW * QB * 32 * D * 2 <= 4 * T::TBYTES, "epilogue staging fits the tile buffers");
    wave_store_rows<D, E>(smem + (wave * QB + qb) * 32 * D * 2, o[qb], inv, orow, a.o_ss,
                       Sq - r0, lane);
    if (qi[qb] < Sq && half == 0) {
      const float mu = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      a.lse[lse_base + qi[qb]] = l != 0.f ? (mu + log2f(l)) * kLn2 : -INFINITY;
    }
  }
  };

  run_tile(qtile);
  if (qtile2 >= 0) {
    __syncthreads();  // the first tile's epilogue is done with LDS
    run_tile(qtile2);
  }
}

// Rows of a packed output that no sequence computes (past cu_seqlens_q[num_seqs], or past
// max_seqlen_q rows of their sequence): out = 0, lse = -inf.
template <int D>
__global__ void __launch_bounds__(256) fwd_tail_kernel(FwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.Sq * a.H) return;
  const int row = (int)(idx / a.H), head = (int)(idx % a.H);
  if (!row_uncovered(a.cu_q, a.num_units, row, a.Sq, a.max_sq)) return;
  uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (int64_t)row * a.o_ss + (int64_t)head * a.o_sh;
#pragma unroll
  for (int d = 0; d < D; d += 8) *reinterpret_cast<u32x4*>(o + d) = u32x4{0, 0, 0, 0};
  a.lse[(int64_t)head * a.lse_row + row] = -INFINITY;
}

// Variants: 0 = 8 waves x 32 rows, lazy rescale (default); 1 = 8 waves x 32 rows, eager
// rescale; 2 = 4 waves x 64 rows (lazy), one wave per SIMD. Variant 2 is compiled for bf16,
// head_dim 128, without a mask or cu_seqlens; other problems use variant 0.
static int effective_variant(int v, int head_dim, int dtype, int mask, bool varlen) {
  if (v == 2 && (head_dim != 128 || dtype != kDtypeBf16 || mask != kMaskNone || varlen)) return 0;
  return (v >= 0 && v <= 2) ? v : 0;
}

int fwd_block_m(int head_dim, int mask, bool varlen) { return 256; }

// Blocks per (unit, head): one per query tile, or one per pair of tiles (dense causal).
static int64_t fwd_blocks(const FwdArgs& a, bool causal, bool varlen) {
  const int per = (causal && !varlen) ? (a.num_q_tiles + 1) / 2 : a.num_q_tiles;
  return (int64_t)a.num_units * a.H * per;
}

template <class E, int D, int NW, int QB, bool LAZY>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  const int64_t nblk = fwd_blocks(a, causal, varlen);
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(64 * NW);
#define EXATTN_FWD(C, M, V) \
  hipLaunchKernelGGL((fwd_kernel<E, D, NW, QB, C, M, V, LAZY>), grid, block, 0, s, a)
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
  const int64_t nblk = fwd_blocks(a, causal, false);
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(64 * NW);
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<bf16, 128, NW, QB, true, kMaskNone, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<bf16, 128, NW, QB, false, kMaskNone, false, true>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fwd_e(const FwdArgs& a, int head_dim, int v, bool causal, int mask,
                               bool varlen, hipStream_t s) {
  if (head_dim == 64) {
    if (v == 1) return launch_fwd_d<E, 64, 8, 1, false>(a, causal, mask, varlen, s);
    return launch_fwd_d<E, 64, 8, 1, true>(a, causal, mask, varlen, s);
  }
  if (v == 1) return launch_fwd_d<E, 128, 8, 1, false>(a, causal, mask, varlen, s);
  return launch_fwd_d<E, 128, 8, 1, true>(a, causal, mask, varlen, s);
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, bool causal, int mask,
                      bool varlen, int variant, hipStream_t s) {
  const int v = effective_variant(variant, head_dim, dtype, mask, varlen);
  if (v == 2) return launch_fwd_plain128<4, 2>(a, causal, s);
  if (dtype == kDtypeF16) return launch_fwd_e<f16>(a, head_dim, v, causal, mask, varlen, s);
  return launch_fwd_e<bf16>(a, head_dim, v, causal, mask, varlen, s);
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
