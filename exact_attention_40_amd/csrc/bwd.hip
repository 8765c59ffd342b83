// Backward kernels: recompute P from the stored LSE and produce dQ, dK, dV.
//
// Pass order on the caller's stream (default, deterministic variant):
//   0. unit_order_kernel  packed layouts only: rank the sequences by query length.
//   1. delta_kernel    Delta_i = sum_d dO_id * O_id (fp32), lse2_i = lse_i * log2(e)
//                      (+inf for empty rows so exp2(s - lse2) = 0).
//   2. bwd_kernel      per (unit, kv head, block of 128 keys): dK and dV accumulate in
//      <DQ=false>      registers over every query head of the group and every query tile.
//   3. bwd_dq_kernel   per (unit, head, block of 256 query rows): dQ accumulates in
//                      registers over every key tile, recomputing S and dP.
//   4. q_tail_kernel / kv_tail_kernel  packed layouts only: query rows past
//                      cu_seqlens_q[num_seqs] get dq = 0, key rows past cu_seqlens_k[num_seqs]
//                      get dk = dv = 0.
// Fused variant: delta_kernel also clears an fp32 dQ accumulator, bwd_kernel<DQ=true> adds
// dQ partial products into it with atomics, and dq_reduce converts it (dq = bf16(acc*scale)).
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

// ----------------------------------------------------------------------------------------
// 1. Delta / lse2 / dQ-accumulator clear. One block = 64 consecutive rows (tokens) of one
// head; D/8 lanes per row read that row's O and dO once (whole 2*D-byte rows), and the 64
// row results are stored together, so Delta and lse2 go out as whole contiguous runs (a
// dense run may straddle two batch entries).
// ----------------------------------------------------------------------------------------
constexpr int kDeltaRows = 64;

template <class E, int D, bool VARLEN>
__global__ void __launch_bounds__(256) delta_kernel(BwdArgs a) {
  using V8 = typename Ty<E>::v8;
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPP = 256 / LPR;        // rows per pass
  __shared__ float part[kDeltaRows];
  const int head = (int)(blockIdx.x % a.H);
  const int64_t tok0 = (int64_t)(blockIdx.x / a.H) * kDeltaRows;
  const int sub = threadIdx.x % LPR;
  // row index of token `tok` in the lse layout
  auto st_index = [&](int64_t tok) -> int64_t {
    if constexpr (VARLEN) {
      return (int64_t)head * a.lse_row + tok;
    } else {
      const int64_t b = tok / a.Sq, s = tok % a.Sq;
      return (b * a.H + head) * a.Sq + s;
    }
  };
#pragma unroll
  for (int pass = 0; pass < kDeltaRows / RPP; ++pass) {
    const int lr = pass * RPP + (int)threadIdx.x / LPR;
    const int64_t tok = tok0 + lr;
    float acc = 0.f;
    if (tok < a.rows_q) {
      int64_t o_off, do_off;
      if constexpr (VARLEN) {
        o_off = tok * a.o_ss + (int64_t)head * a.o_sh;
        do_off = tok * a.do_ss + (int64_t)head * a.do_sh;
      } else {
        const int64_t b = tok / a.Sq, s = tok % a.Sq;
        o_off = b * a.o_sb + s * a.o_ss + (int64_t)head * a.o_sh;
        do_off = b * a.do_sb + s * a.do_ss + (int64_t)head * a.do_sh;
      }
      const V8 o = *reinterpret_cast<const V8*>(reinterpret_cast<const E*>(a.out) + o_off + sub * 8);
      const V8 g = *reinterpret_cast<const V8*>(reinterpret_cast<const E*>(a.dout) + do_off + sub * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (float)o[i] * (float)g[i];
      if (a.dq_acc != nullptr) {
        float* dqa = a.dq_acc + (tok * a.H + head) * D + sub * 8;
        reinterpret_cast<f32x4*>(dqa)[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<f32x4*>(dqa)[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (sub == 0) part[lr] = acc;
  }
  __syncthreads();
  if (threadIdx.x < kDeltaRows) {
    const int64_t tok = tok0 + threadIdx.x;
    if (tok < a.rows_q) {
      const int64_t st = st_index(tok);
      const float l = a.lse[st];
      a.delta[st] = part[threadIdx.x];
      a.lse2[st] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
  }
}

// ----------------------------------------------------------------------------------------
// 2. Main backward kernel.
//
// One workgroup = 8 waves = 128 keys (four groups of 32) of one (unit, kv head), looping
// over every query head of the group and every 64-row query tile that can see the block.
// The waves come in pairs per key group, with two waves per SIMD:
//   wave A (0..3): S = Q K^T, P = exp2(min(S*c + bias - lse2, 0)) (hidden entries 0),
//                  P -> LDS (fp32), dV += P^T dO;  keeps K fragments and dV in registers;
//   wave B (4..7): dP = dO V^T, dS = P * (dP - Delta) with P from LDS, dS -> LDS (bf16,
//                  [query][key]), dK += dS^T Q;   keeps V fragments and dK in registers.
// Then all eight waves form the 64 x D dQ tile from dS and the block's K (32x32 tiles, the
// k dimension over all 128 keys) and add it to the fp32 accumulator with buffer atomics,
// which drop rows past the end of the sequence.
// Both roles issue their matrix products from registers (P, dS as the A operand from the C
// layout; lane = key) and LDS (Q, dO row reads; transposed reads for the k = query
// operands and for K in the dQ product). Q and dO tiles are copied straight from global
// memory into swizzled LDS, double-buffered, one tile ahead; two barriers per tile.
// Row-major LDS tiles without padding use an XOR swizzle of their 16-byte chunks (swz_f),
// which keeps both the 16-byte row reads and the 8-byte transposed reads free of bank
// conflicts.
// ----------------------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int BN = 128;
  static constexpr int KG = BN / 32;             // key groups (wave pairs)
  static constexpr int BM = 64;
  static constexpr int QB = BM / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int SLD = BN + 8;             // dS pitch (16 B mod 128 B)
  static constexpr int Q_ELEMS = BM * D;
  static constexpr int K_ELEMS = BN * D;
  static constexpr int S_ELEMS = BM * SLD;
  static constexpr int P_BYTES = KG * QB * 4 * 64 * 16;   // fp32 P hand-over, C layout
  static constexpr int DQ_TILES = QB * DB;       // 32x32 dQ tiles per query tile
  static_assert((BM * CPR) % (64 * NW) == 0 && (BN * CPR) % (64 * NW) == 0, "even copy split");
  static_assert(DQ_TILES <= NW, "one dQ tile per wave at most");
};

// LDS bytes: [K block | Q x2 | dO x2 | dS | P | lse2 x2 | Delta x2]; K block and dS only
// when the kernel forms dQ.
template <int D, bool DQ>
constexpr size_t bwd_smem_bytes() {
  using T = BwdTile<D>;
  return (size_t)((DQ ? T::K_ELEMS + T::S_ELEMS : 0) + 4 * T::Q_ELEMS) * 2 + T::P_BYTES +
         4 * T::BM * sizeof(float);
}

template <class E, int D, bool CAUSAL, int MASK, bool VARLEN, bool DQ>
__global__ void __launch_bounds__(512) bwd_kernel(BwdArgs a) {
  nan_passing_clamp();   // NaN passes the clamped exponential below (no NaN is cleaned)
  using T = BwdTile<D>;
  using V8 = typename Ty<E>::v8;
  using V4 = typename Ty<E>::v4;
  constexpr int kDqAtomics = 16;                 // buffer atomics per wave per dQ phase
  constexpr int RB = D * 2;                      // bytes per swizzled row
  constexpr int QBYTES = T::Q_ELEMS * 2;         // one Q or dO buffer
  constexpr int KBYTES = DQ ? T::K_ELEMS * 2 : 0;
  constexpr int SBYTES = DQ ? T::S_ELEMS * 2 : 0;
  constexpr int DO_OFF = 2 * QBYTES;             // dO buffers follow the two Q buffers
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* k_b = smem;                     // K block (dQ only)
  unsigned char* q_b = smem + KBYTES;            // Q[2] then dO[2]
  unsigned char* ds_b = q_b + 4 * QBYTES;        // dS [BM][SLD] bf16 (dQ only)
  unsigned char* p_b = ds_b + SBYTES;            // P hand-over, fp32
  float* lse2_l = reinterpret_cast<float*>(p_b + T::P_BYTES);  // [2][BM]
  float* del_l = lse2_l + 2 * T::BM;                           // [2][BM]

  // The wave index is uniform across a wave; readfirstlane tells the compiler so, which keeps
  // role branches scalar and buffer descriptors in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, j16 = lane & 15;
  const bool role_a = wave < T::KG;
  const int kg = role_a ? wave : wave - T::KG;   // key group of this wave

  // Consecutive blocks are the key blocks of one (unit, kv head): they re-read the same
  // Q/dO tiles, which then stay in one XCD's L2 (also for packed layouts, where ordering
  // by key block across sequences was measured slower).
  // Dense: consecutive logical blocks share an XCD (xcd_remap). Packed with a ranking of
  // the sequences (unit_order: largest q_len * k_len first): the dispatcher sends block b to
  // XCD b % 8, and XCD x takes the sequences of rank 8s + x (s even) or 8s + 7 - x (s odd),
  // a snake deal that gives every XCD a similar share of the work; each sequence's blocks
  // stay on one XCD (its Q/dO re-reads hit that XCD's L2), largest sequences first.
  int kbi, g, unit;
  if (VARLEN && a.unit_order) {
    const int per_unit = a.Hkv * a.num_k_blocks;
    const int x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
    const int slot = k / per_unit, within = k - slot * per_unit;
    const int r = 8 * slot + ((slot & 1) ? 7 - x : x);
    if (r >= a.num_units) return;
    unit = a.unit_order[r];
    g = within / a.num_k_blocks;
    kbi = within - g * a.num_k_blocks;
  } else {
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    kbi = blk % a.num_k_blocks;
    const int ug = blk / a.num_k_blocks;
    g = ug % a.Hkv;
    unit = ug / a.Hkv;
  }

  int Sq, Sk;
  int64_t qrow0, krow0, qb_off, kb_off, vb_off, dob_off, st_unit;
  if constexpr (VARLEN) {
    const SeqRows rq = seq_rows(a.cu_q, unit, a.Sq, a.max_sq);
    const SeqRows rk = seq_rows(a.cu_k, unit, a.Sk, a.max_sk);
    const int qs = rq.beg, ks = rk.beg;
    Sq = rq.len;
    Sk = rk.len;
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
  const int kl_w = kg * 32 + l32;            // block-local key of this lane
  const int kw = kb0 + kl_w;

  // The block's K (swizzled LDS, zero past the last key) and this pair's operand
  // fragments in registers: K for wave A (S = Q K^T), V for wave B (dP = dO V^T).
  const E* K = reinterpret_cast<const E*>(a.k) + kb_off + (int64_t)g * a.k_sh +
                  (int64_t)kb0 * a.k_ss;
  const E* V = reinterpret_cast<const E*>(a.v) + vb_off + (int64_t)g * a.v_sh +
                  (int64_t)kb0 * a.v_ss;
  const auto rk = make_rsrc(K, (uint32_t)((krows - 1) * a.k_ss + D) * 2u);
  const auto rv = make_rsrc(V, (uint32_t)((krows - 1) * a.v_ss + D) * 2u);
  if (DQ) copy_tile_to_lds<D, T::BN, T::NW>(k_b, rk, (int)a.k_ss, wave, lane);
  V8 kv[T::DS];
  {
    const auto r = role_a ? rk : rv;
    const int st = role_a ? (int)a.k_ss : (int)a.v_ss;
#pragma unroll
    for (int s = 0; s < T::DS; ++s)
      kv[s] = __builtin_bit_cast(V8, buf_load16(r, (uint32_t)(kl_w * st + 16 * s + 8 * half) * 2u));
  }

  // ---- per-lane LDS base addresses; everything else is an immediate offset ----------------
  // Row-operand reads of Q/dO rows qb*32 + l32, d-slab ds: one base per slab (the swizzle
  // depends on the row's low four bits only, so qb, the buffer and Q/dO are immediates).
  // Wave A reads Q (S = Q K^T), wave B reads dO (dP = dO V^T).
  const unsigned char* aq[T::DS];   // buffer 0; +QBYTES for buffer 1
#pragma unroll
  for (int ds = 0; ds < T::DS; ++ds)
    aq[ds] = q_b + (role_a ? 0 : DO_OFF) + l32 * RB + 16 * ((2 * ds + half) ^ swz_f<D>(l32));
  // Transposed reads of dO (wave A) or Q (wave B): rows 16kk + 4*half + (j16>>2) + 8*sec,
  // columns db*32 + 16*(grp&1) + 4*(j16&3); one base per (db, sec), kk is an immediate.
  const int tr_row = j16 >> 2;
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  const unsigned char* tq[T::DB][2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 4 * half + tr_row + 8 * sec;
    const unsigned char* base = q_b + (role_a ? DO_OFF : 0) + row * RB + 8 * (j16 & 1);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) tq[db][sec] = base + 16 * ((4 * db + clow) ^ swz_f<D>(row));
  }
  // Transposed reads of K for this wave's dQ column block: rows 16kk + 8*half + (j16>>2)
  // and 4 rows below.
  const int dq_db = wave % T::DB;
  const unsigned char* tk[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 8 * half + tr_row + 4 * sec;
    tk[sec] = k_b + row * RB + 16 * ((4 * dq_db + clow) ^ swz_f<D>(row)) + 8 * (j16 & 1);
  }
  unsigned char* dsw = ds_b + (4 * half * T::SLD + kl_w) * 2;         // dS write (wave B)
  const unsigned char* dsr = ds_b + (l32 * T::SLD + 8 * half) * 2;   // dS read (dQ)
  unsigned char* pp = p_b + kg * (T::QB * 4 * 1024) + lane * 16;    // P hand-over
  const unsigned char* st_rd = reinterpret_cast<const unsigned char*>(lse2_l) + 16 * half;

  f32x16 acc[T::DB];   // dV (wave A) or dK (wave B)
#pragma unroll
  for (int db = 0; db < T::DB; ++db) acc[db] = f32x16{};

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);
  const int qstart = CAUSAL ? min(kb0 / T::BM * T::BM, Sq) : 0;
  const int n_qt = (Sq - qstart + T::BM - 1) / T::BM;
  const int n_iter = a.group * n_qt;

  // Staging of one query tile: Q and dO straight into LDS, lse2 and Delta via registers.
  float st_v = 0.f;
  // Workgroups of neighbouring key blocks run at the same time on one XCD; starting each
  // at a different query tile spreads their dQ atomics over different rows.
  const int rot = n_iter == 0 ? 0
                : a.rotate == 1 ? (int)(((int64_t)kbi * n_iter) / a.num_k_blocks) % n_iter
                : a.rotate == 2 ? (kbi & 7) % n_iter : 0;
  // Tile positions advance incrementally (query tile fastest, then head, wrapping), so the
  // loop needs no integer division.
  struct TilePos { int head, q0; };
  const int h_beg = g * a.group, h_end = h_beg + a.group;
  const int q_end = qstart + n_qt * T::BM;
  auto advance = [&](TilePos& p) {
    p.q0 += T::BM;
    if (p.q0 >= q_end) {
      p.q0 = qstart;
      if (++p.head == h_end) p.head = h_beg;
    }
  };
  TilePos cur = {h_beg + (n_iter ? rot / n_qt : 0), qstart + (n_iter ? rot % n_qt : 0) * T::BM};
  auto load_q = [&](const TilePos& tp, int buf) {
    const int head = tp.head, qt0 = tp.q0;
    const int rows = min(T::BM, Sq - qt0);
    const E* Qp = reinterpret_cast<const E*>(a.q) + qb_off + (int64_t)head * a.q_sh +
                     (int64_t)qt0 * a.q_ss;
    const E* Dp = reinterpret_cast<const E*>(a.dout) + dob_off + (int64_t)head * a.do_sh +
                     (int64_t)qt0 * a.do_ss;
    copy_tile_to_lds<D, T::BM, T::NW>(q_b + buf * QBYTES,
                                     make_rsrc(Qp, (uint32_t)((rows - 1) * a.q_ss + D) * 2u),
                                     (int)a.q_ss, wave, lane);
    copy_tile_to_lds<D, T::BM, T::NW>(q_b + DO_OFF + buf * QBYTES,
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

  // Prefetch distance two: tiles 0 and 1 now; tile it + 2 is requested during the dQ phase
  // of tile it, before that phase's atomics, so waiting for it never waits for atomics.
  if (n_iter > 0) {
    load_q(cur, 0);
    store_stats(0);
  }
  if (n_iter > 1) {
    wait_vmem();
    TilePos nx = cur;
    advance(nx);
    load_q(nx, 1);
    store_stats(1);
  }
  wait_vmem();
  __syncthreads();

  // One query tile. BUF (0/1) selects the staging buffer at compile time.
  TilePos ahead = cur;   // position of tile it + 2
  advance(ahead);
  advance(ahead);
  auto iteration = [&](int it, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr int QO = BUF * QBYTES;
    const int head = cur.head, qt0 = cur.q0;
    const bool edge = (kb0 + T::BN > Sk) || (qt0 + T::BM > Sq) || (MASK != kMaskNone) ||
                      (CAUSAL && kb0 + T::BN - 1 > qt0);
    const int64_t m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;

    // P = exp2(min(S*c + bias - lse2, 0)) in place (wave A).
    auto softmax_p = [&](f32x16& s, int qb, auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 l2 = lds_at<f32x4>(st_rd, BUF * T::BM * 4 + (qb * 32 + 8 * rg) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          if constexpr (!EDGE) {
            s[r] = exp2_le1(fmaf(s[r], c2, -l2[e]));
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
                b2 = vis ? bias_log2(bias) : 0.f;
              }
            }
            const float e2 = exp2_le1(fmaf(s[r], c2, b2 - l2[e]));
            s[r] = vis ? e2 : 0.f;
          }
        }
      }
    };

    // ---- phase 1: S and P (A) / dP (B) ----
    // Row fragments are read four MFMAs ahead; the fences keep the reads where they are
    // placed so the LDS latency overlaps the preceding MFMAs.
    f32x16 sp[T::QB];
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) sp[qb] = f32x16{};
    {
      constexpr int NF = T::DS * T::QB;
      auto frag = [&](int f) { return lds_at<V8>(aq[f / T::QB], QO + (f % T::QB) * 32 * RB); };
      V8 fr[4] = {frag(0), frag(1), frag(2), frag(3)};
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int ds = f / T::QB, qb = f % T::QB;
        sp[qb] = mfma32(fr[f % 4], kv[ds], sp[qb]);
        if (f + 4 < NF) fr[f % 4] = frag(f + 4);
        __builtin_amdgcn_sched_barrier(0x0004);
      }
    }
    if (role_a) {
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) {
        if (edge) softmax_p(sp[qb], qb, bool_c<true>{});
        else softmax_p(sp[qb], qb, bool_c<false>{});
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<f32x4*>(pp + (qb * 4 + rg) * 1024) =
              f32x4{sp[qb][4 * rg], sp[qb][4 * rg + 1], sp[qb][4 * rg + 2], sp[qb][4 * rg + 3]};
      }
    }
    __syncthreads();  // P visible to wave B

    // ---- phase 2: dV += P^T dO (A) / dS, dK += dS^T Q (B) ----
    if (!role_a) {
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 pv = *reinterpret_cast<const f32x4*>(pp + (qb * 4 + rg) * 1024);
          const f32x4 dd =
              lds_at<f32x4>(st_rd, 2 * T::BM * 4 + BUF * T::BM * 4 + (qb * 32 + 8 * rg) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sp[qb][4 * rg + e] = pv[e] * (sp[qb][4 * rg + e] - dd[e]);
        }
        if (DQ) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *reinterpret_cast<E*>(dsw + (qb * 32 + 8 * (r >> 2) + (r & 3)) * T::SLD * 2) =
                (E)sp[qb][r];
        }
      }
    }
    // Transposed fragments of the next 16-row slab are read while this slab's MFMAs run.
    {
      constexpr int NKK = T::BM / 16;
      V4 tb[2][T::DB][2];
      auto tload = [&](int kk, int slot) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          tb[slot][db][0] = tr_at<V4>(tq[db][0], QO + 16 * kk * RB);
          tb[slot][db][1] = tr_at<V4>(tq[db][1], QO + 16 * kk * RB);
        }
      };
      tload(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int qb = kk >> 1, hs = (kk & 1) * 8;
        const V8 pa = cvt8<V8>(sp[qb][hs + 0], sp[qb][hs + 1], sp[qb][hs + 2], sp[qb][hs + 3],
                               sp[qb][hs + 4], sp[qb][hs + 5], sp[qb][hs + 6], sp[qb][hs + 7]);
        if (kk + 1 < NKK) tload(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          acc[db] = mfma32(pa, cat44(tb[kk & 1][db][0], tb[kk & 1][db][1]), acc[db]);
          __builtin_amdgcn_sched_barrier(0x0004);
        }
      }
    }
    // Tile it + 1 was requested during the previous dQ phase; only the newest memory
    // operations (that phase's atomics) may still be in flight.
    if (DQ && wave < T::DQ_TILES) wait_vmem_except<kDqAtomics>();
    else wait_vmem();
    if (it >= 1 && it + 1 < n_iter) store_stats(BUF ^ 1);
    __syncthreads();  // dS complete; next tile's staging visible; P consumed

    // ---- phase 3: request tile it + 2, then the dQ tile of this wave over 128 keys ----
    if (it + 2 < n_iter) load_q(ahead, BUF);
    advance(ahead);
    if (DQ && wave < T::DQ_TILES) {
      const int qb = wave / T::DB, db = dq_db;
      const int qrows = min(T::BM, Sq - qt0);
      float* dqp = a.dq_acc + ((qrow0 + qt0) * a.H + head) * D;
      const auto rdq = make_rsrc(dqp, (uint32_t)((qrows - 1) * a.H * D + D) * 4u);
      f32x16 dq = f32x16{};
#pragma unroll
      for (int kk = 0; kk < T::BN / 16; ++kk) {
        const V8 sv = lds_at<V8>(dsr, (qb * 32 * T::SLD + kk * 16) * 2);
        const int o = 16 * kk * RB;
        const V8 kvv = cat44(tr_at<V4>(tk[0], o), tr_at<V4>(tk[1], o));
        dq = mfma32(sv, kvv, dq);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qb * 32 + acc_row(r, half);
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
            dq[r], rdq, (int)((row * a.H * D + db * 32 + l32) * 4), 0, 0);
      }
    }
    advance(cur);
  };

  int it = 0;
  for (; it + 1 < n_iter; it += 2) {
    iteration(it, std::integral_constant<int, 0>{});
    iteration(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < n_iter) iteration(it, std::integral_constant<int, 0>{});

  // Epilogue: dV (wave A) or dK times scale (wave B) in the input format into contiguous
  // [rows_k, Hkv, D], whole rows staged through this wave's slice of LDS (free after the
  // last barrier); rows past the sequence end are not written.
  __syncthreads();
  static_assert(T::NW * 32 * D * 2 <= bwd_smem_bytes<D, DQ>(), "epilogue staging fits the LDS");
  const float sc = role_a ? 1.f : a.scale;
  E* dst = reinterpret_cast<E*>(role_a ? a.dv : a.dk) + ((krow0 + kb0 + kg * 32) * a.Hkv + g) * D;
  wave_store_cols<D, E>(smem + wave * 32 * D * 2, acc, sc, dst, (int64_t)a.Hkv * D,
                        krows - kg * 32, lane);
}

// ----------------------------------------------------------------------------------------
// 2b. dQ kernel (deterministic, no atomics).
//
// One workgroup = 8 waves = 256 query rows of one (unit, head); each wave owns 32 rows and
// keeps their Q and dO fragments (B operand: column = query, k-slots = d) and their lse2
// and Delta (one per lane) in registers. Key tiles of 64 (K and V, row-major, swizzled) are
// copied straight into LDS, double-buffered. Per tile:
//   S^T = K Q^T and dP^T = V dO^T        (lane = query column, registers = keys)
//   P = exp2(min(S*c + bias - lse2, 0)), dS = P * (dP - Delta); hidden entries are 0
//   dQ^T += K^T dS^T                     (K^T fragments by transposed LDS reads; dS^T is the
//                                          B operand straight from registers)
// dQ accumulates over every key tile in registers and is written once, times the scale, as
// bf16: the sum order is fixed, so dQ is bitwise reproducible.
// ----------------------------------------------------------------------------------------
template <int D>
struct DqTile {
  static constexpr int NW = 8;
  static constexpr int BM = NW * 32;
  static constexpr int BN = 64;
  static constexpr int KB = BN / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TBYTES = BN * D * 2;      // one K or V tile
  static_assert((BN * D / 8) % (64 * NW) == 0, "even copy split");
};

template <class E, int D, bool CAUSAL, int MASK, bool VARLEN>
__global__ void __launch_bounds__(512) bwd_dq_kernel(BwdArgs a) {
  nan_passing_clamp();   // NaN passes the clamped exponential below (no NaN is cleaned)
  using T = DqTile<D>;
  using V8 = typename Ty<E>::v8;
  using V4 = typename Ty<E>::v4;
  constexpr int RB = D * 2;
  constexpr int V_OFF = 2 * T::TBYTES;           // V buffers follow the two K buffers
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * T::TBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, j16 = lane & 15;

  // Block order as in the forward: packed layouts take the query-tile index outermost
  // (and no XCD remap). Dense causal: tiles n-1-j and j in one workgroup (equal work).
  const int blk = VARLEN ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int n_qtiles = a.num_q_blocks;
  int qtile, qtile2 = -1, uh;
  if constexpr (VARLEN) {
    const int nuh = a.num_units * a.H;
    qtile = n_qtiles - 1 - blk / nuh;
    uh = blk % nuh;
  } else if constexpr (CAUSAL) {
    const int npair = (n_qtiles + 1) / 2;
    const int j = blk % npair;
    uh = blk / npair;
    qtile = n_qtiles - 1 - j;
    if (j != qtile) qtile2 = j;
  } else {
    qtile = blk % n_qtiles;
    uh = blk / n_qtiles;
  }
  const int head = uh % a.H, unit = uh / a.H, g = head / a.group;

  int Sq, Sk;
  int64_t qrow0, q_base, k_base, v_base, do_base, st_base, m_base = 0;
  if constexpr (VARLEN) {
    const SeqRows rq = seq_rows(a.cu_q, unit, a.Sq, a.max_sq);
    const SeqRows rk = seq_rows(a.cu_k, unit, a.Sk, a.max_sk);
    const int qs = rq.beg, ks = rk.beg;
    Sq = rq.len;
    Sk = rk.len;
    qrow0 = qs;
    q_base = (int64_t)qs * a.q_ss + (int64_t)head * a.q_sh;
    do_base = (int64_t)qs * a.do_ss + (int64_t)head * a.do_sh;
    k_base = (int64_t)ks * a.k_ss + (int64_t)g * a.k_sh;
    v_base = (int64_t)ks * a.v_ss + (int64_t)g * a.v_sh;
    st_base = (int64_t)head * a.lse_row + qs;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
    qrow0 = (int64_t)unit * a.Sq;
    q_base = (int64_t)unit * a.q_sb + (int64_t)head * a.q_sh;
    do_base = (int64_t)unit * a.do_sb + (int64_t)head * a.do_sh;
    k_base = (int64_t)unit * a.k_sb + (int64_t)g * a.k_sh;
    v_base = (int64_t)unit * a.v_sb + (int64_t)g * a.v_sh;
    st_base = ((int64_t)unit * a.H + head) * a.Sq;
    m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;
  }
  // One query tile of BM rows; the workgroup runs one or two of them.
  auto run_tile = [&](const int qtile) __attribute__((always_inline)) {
  const int qt0 = qtile * T::BM;
  if (qt0 >= Sq) return;
  const E* K = reinterpret_cast<const E*>(a.k) + k_base;
  const E* V = reinterpret_cast<const E*>(a.v) + v_base;

  // This lane's query row: Q and dO fragments, lse2 and Delta (zero / +inf past the end).
  const int qw0 = qt0 + wave * 32;
  const int qi = qw0 + l32;
  V8 qf[T::DS], df[T::DS];
  float l2 = INFINITY, dl = 0.f;
  if (qi < Sq) {
    const E* qr = reinterpret_cast<const E*>(a.q) + q_base + (int64_t)qi * a.q_ss + 8 * half;
    const E* dr = reinterpret_cast<const E*>(a.dout) + do_base + (int64_t)qi * a.do_ss + 8 * half;
#pragma unroll
    for (int s = 0; s < T::DS; ++s) {
      qf[s] = *reinterpret_cast<const V8*>(qr + 16 * s);
      df[s] = *reinterpret_cast<const V8*>(dr + 16 * s);
    }
    l2 = a.lse2[st_base + qi];
    dl = a.delta[st_base + qi];
  } else {
#pragma unroll
    for (int s = 0; s < T::DS; ++s) qf[s] = df[s] = V8{};
  }

  const int kend = CAUSAL ? min(Sk, qt0 + T::BM) : Sk;
  const int ntiles = (kend + T::BN - 1) / T::BN;
  int n_plain = 0;
  if (MASK == kMaskNone) {
    int lim = Sk / T::BN;
    if (CAUSAL) lim = min(lim, (qt0 + 1) / T::BN);
    n_plain = min(lim, ntiles);
  }

  // K/V tiles go straight into LDS through the compiler's direct-to-LDS loads. (The
  // asynchronous copies the forward and dK/dV kernels use measured about 1% slower here.)
  auto load_tile = [&](int t, int buf) {
    const int kb0 = t * T::BN;
    const int rows = min(T::BN, Sk - kb0);
    copy_tile_to_lds<D, T::BN, T::NW>(smem + buf * T::TBYTES,
                                     make_rsrc(K + (int64_t)kb0 * a.k_ss, (uint32_t)((rows - 1) * a.k_ss + D) * 2u),
                                     (int)a.k_ss, wave, lane);
    copy_tile_to_lds<D, T::BN, T::NW>(smem + V_OFF + buf * T::TBYTES,
                                     make_rsrc(V + (int64_t)kb0 * a.v_ss, (uint32_t)((rows - 1) * a.v_ss + D) * 2u),
                                     (int)a.v_ss, wave, lane);
  };

  // Per-lane LDS bases: row reads (keys kb*32 + l32, slab ds) and transposed K reads (keys
  // 16kk + 4*half + (j16>>2) + 8*sec, d = db*32 + 16*(grp&1) + 4*(j16&3)).
  const unsigned char* ar[T::DS];
#pragma unroll
  for (int ds = 0; ds < T::DS; ++ds) ar[ds] = smem + l32 * RB + 16 * ((2 * ds + half) ^ swz_f<D>(l32));
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  const unsigned char* tk[T::DB][2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 4 * half + (j16 >> 2) + 8 * sec;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
      tk[db][sec] = smem + row * RB + 16 * ((4 * db + clow) ^ swz_f<D>(row)) + 8 * (j16 & 1);
  }

  f32x16 dq[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) dq[db] = f32x16{};

  if (ntiles > 0) load_tile(0, 0);
  wait_vmem();
  __syncthreads();

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);

  auto tile = [&](int t, auto buf_tag, auto masked_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int KO = BUF * T::TBYTES;
    if (t + 1 < ntiles) load_tile(t + 1, BUF ^ 1);
    // S^T and dP^T: K and V row fragments read four MFMAs ahead (fences keep the order).
    // Unmasked tiles take the key blocks one after the other, and the VALU work of a block
    // (P and dS) is issued between MFMAs that do not depend on it: block 0's between the S
    // and dP MFMAs of block 1, block 1's between the dQ MFMAs of block 0. Masked tiles
    // (mask reads, boundary tests) keep all VALU work after the S and dP MFMAs.
    f32x16 s[T::KB], dp[T::KB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) s[kb] = dp[kb] = f32x16{};
    const int kb0 = t * T::BN;
    auto ds_elem = [&](int kb, int r) {
      float p;
      if constexpr (!MASKED) {
        p = exp2_le1(fmaf(s[kb][r], c2, -l2));
      } else {
        const int kj = kb0 + kb * 32 + acc_row(r, half);
        bool vis = (kj < Sk) && (qi < Sq);
        if (CAUSAL) vis = vis && (kj <= qi);
        float b2 = 0.f;
        if (MASK != kMaskNone) {
          const int64_t mi = m_base + (int64_t)min(qi, Sq - 1) * a.m_si + min(kj, Sk - 1);
          if (MASK == kMaskBool) {
            vis = vis && (mask_u8[mi] != 0);
          } else {
            const float bias = (float)mask_bf[mi];
            vis = vis && (bias != -INFINITY);
            b2 = vis ? bias_log2(bias) : 0.f;
          }
        }
        const float e2 = exp2_le1(fmaf(s[kb][r], c2, b2 - l2));
        p = vis ? e2 : 0.f;
      }
      dp[kb][r] = p * (dp[kb][r] - dl);
    };
    static_assert(T::KB == 2, "two key blocks per tile");
    {
      constexpr int NF = T::DS * T::KB * 2;    // (kb, ds, K or V) unmasked; (ds, kb, K or V) masked
      constexpr int EPM = 16 / (2 * T::DS);    // block-0 elements per block-1 MFMA
      auto fkb = [](int f) { return MASKED ? (f / 2) % T::KB : f / (2 * T::DS); };
      auto fds = [](int f) { return MASKED ? f / (2 * T::KB) : (f / 2) % T::DS; };
      auto frag = [&](int f) {
        return lds_at<V8>(ar[fds(f)], (f & 1) * V_OFF + KO + fkb(f) * 32 * RB);
      };
      V8 fr[4] = {frag(0), frag(1), frag(2), frag(3)};
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int ds = fds(f), kb = fkb(f);
        if (f & 1) dp[kb] = mfma32(fr[f % 4], df[ds], dp[kb]);
        else s[kb] = mfma32(fr[f % 4], qf[ds], s[kb]);
        if (f + 4 < NF) fr[f % 4] = frag(f + 4);
        if (!MASKED && kb == 1) {
#pragma unroll
          for (int e = 0; e < EPM; ++e) ds_elem(0, (f - 2 * T::DS) * EPM + e);
        }
        __builtin_amdgcn_sched_barrier(0x0004);
      }
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ds_elem(kb, r);
    }
    // dQ^T += K^T dS^T over 16-key slabs; the next slab's transposed K fragments are read
    // while this slab's MFMAs run.
    {
      constexpr int NKK = T::BN / 16;
      constexpr int EPM = 16 / (2 * T::DB);    // block-1 elements per block-0 dQ MFMA
      V4 tb[2][T::DB][2];
      auto tload = [&](int kk, int slot) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          tb[slot][db][0] = tr_at<V4>(tk[db][0], KO + 16 * kk * RB);
          tb[slot][db][1] = tr_at<V4>(tk[db][1], KO + 16 * kk * RB);
        }
      };
      tload(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int kb = kk >> 1, hs = (kk & 1) * 8;
        const V8 sb = cvt8<V8>(dp[kb][hs + 0], dp[kb][hs + 1], dp[kb][hs + 2], dp[kb][hs + 3],
                               dp[kb][hs + 4], dp[kb][hs + 5], dp[kb][hs + 6], dp[kb][hs + 7]);
        if (kk + 1 < NKK) tload(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          dq[db] = mfma32(cat44(tb[kk & 1][db][0], tb[kk & 1][db][1]), sb, dq[db]);
          if (!MASKED && kb == 0) {
#pragma unroll
            for (int e = 0; e < EPM; ++e) ds_elem(1, ((kk & 1) * T::DB + db) * EPM + e);
          }
          __builtin_amdgcn_sched_barrier(0x0004);
        }
      }
    }
    wait_vmem();      // the next tile has landed in LDS
    __syncthreads();  // ... for every wave, and every wave is done with this one
  };

  int t = 0;
  for (; t + 1 < n_plain; t += 2) {
    tile(t, std::integral_constant<int, 0>{}, bool_c<false>{});
    tile(t + 1, std::integral_constant<int, 1>{}, bool_c<false>{});
  }
  if constexpr (CAUSAL || MASK != kMaskNone || VARLEN) {
    // Remaining tiles (at most one unmasked, then the masked ones) in the masked form, in
    // pairs of fixed buffer parity: one form per loop keeps the register allocation of the
    // two loops apart (a run-time choice between forms inside one loop spills).
    for (; t < ntiles; t += 2) {
      tile(t, std::integral_constant<int, 0>{}, bool_c<true>{});
      if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{}, bool_c<true>{});
    }
  } else {
    // Dense, unmasked, non-causal: only an odd last tile and a partial key tile remain.
    // This form measured about 1% faster for the main loop above than the paired one.
    for (; t < ntiles; ++t) {
      const bool plain = t < n_plain;
      if ((t & 1) == 0) {
        if (plain) tile(t, std::integral_constant<int, 0>{}, bool_c<false>{});
        else tile(t, std::integral_constant<int, 0>{}, bool_c<true>{});
      } else {
        if (plain) tile(t, std::integral_constant<int, 1>{}, bool_c<false>{});
        else tile(t, std::integral_constant<int, 1>{}, bool_c<true>{});
      }
    }
  }

  // Epilogue: dq = bf16(dQ * scale), contiguous [rows_q, H, D], through this wave's slice
  // of LDS (free after the last barrier); rows past Sq are not written.
  E* dqw = reinterpret_cast<E*>(a.dq) + ((qrow0 + qw0) * a.H + head) * D;
  static_assert(T::NW * 32 * D * 2 <= 4 * T::TBYTES, "epilogue staging fits the tile buffers");
  wave_store_rows<D, E>(smem + wave * 32 * D * 2, dq, a.scale, dqw, (int64_t)a.H * D, Sq - qw0, lane);
  };

  run_tile(qtile);
  if (qtile2 >= 0) {
    __syncthreads();  // the first tile's epilogue is done with LDS
    run_tile(qtile2);
  }
}

// ----------------------------------------------------------------------------------------
// 3. dq = bf16(dq_acc * scale), 8 elements per thread.
// ----------------------------------------------------------------------------------------
template <class E>
__global__ void __launch_bounds__(256) dq_reduce_kernel(BwdArgs a, int64_t n8) {
  using V8 = typename Ty<E>::v8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.dq_acc) + 2 * i;
  const f32x4 x0 = src[0], x1 = src[1];
  const float sc = a.scale;
  reinterpret_cast<V8*>(a.dq)[i] = cvt8<V8>(x0[0] * sc, x0[1] * sc, x0[2] * sc, x0[3] * sc,
                                            x1[0] * sc, x1[1] * sc, x1[2] * sc, x1[3] * sc);
}

// ----------------------------------------------------------------------------------------
// 4. Packed layouts: key rows that no sequence computes (past cu_seqlens_k[num_seqs], or
// past max_seqlen_k rows of their sequence) get dk = dv = 0.
// ----------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kv_tail_kernel(BwdArgs a, int64_t row_chunks, int chunks_per_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= row_chunks) return;
  const int row = (int)(i / chunks_per_row);
  if (!row_uncovered(a.cu_k, a.num_units, row, a.Sk, a.max_sk)) return;
  reinterpret_cast<u32x4*>(a.dk)[i] = u32x4{0, 0, 0, 0};
  reinterpret_cast<u32x4*>(a.dv)[i] = u32x4{0, 0, 0, 0};
}

// Packed layouts, deterministic dQ: query rows that no sequence computes get dq = 0.
__global__ void __launch_bounds__(256) q_tail_kernel(BwdArgs a, int64_t row_chunks, int chunks_per_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= row_chunks) return;
  const int row = (int)(i / chunks_per_row);
  if (!row_uncovered(a.cu_q, a.num_units, row, a.Sq, a.max_sq)) return;
  reinterpret_cast<u32x4*>(a.dq)[i] = u32x4{0, 0, 0, 0};
}

// Packed layouts: order[rank] = sequence, ranked by q_len * k_len of the clamped, truncated
// sequences (largest first, ties by index). The ranks form a permutation, so every slot is
// written exactly once.
__global__ void __launch_bounds__(256) unit_order_kernel(BwdArgs a, int32_t* order) {
  const int n = a.num_units;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  auto work = [&](int s) {
    return (int64_t)seq_rows(a.cu_q, s, a.Sq, a.max_sq).len * seq_rows(a.cu_k, s, a.Sk, a.max_sk).len;
  };
  const int64_t wi = work(i);
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int64_t wj = work(j);
    rank += (wj > wi) || (wj == wi && j < i);
  }
  order[rank] = i;
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

hipError_t launch_unit_order(const BwdArgs& a, int32_t* order, hipStream_t s) {
  const int n = a.num_units;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  hipLaunchKernelGGL(unit_order_kernel, grid, block, 0, s, a, order);
  return hipGetLastError();
}

int bwd_block_n(int head_dim) { return BwdTile<128>::BN; }

template <class E>
static hipError_t launch_delta_e(const BwdArgs& a, int head_dim, bool varlen, hipStream_t s) {
  const int64_t nblk = ((int64_t)a.rows_q + kDeltaRows - 1) / kDeltaRows * a.H;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(256);
  if (head_dim == 64) {
    if (varlen) hipLaunchKernelGGL((delta_kernel<E, 64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<E, 64, false>), grid, block, 0, s, a);
  } else {
    if (varlen) hipLaunchKernelGGL((delta_kernel<E, 128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<E, 128, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_delta(const BwdArgs& a, int head_dim, int dtype, bool varlen, hipStream_t s) {
  if (dtype == kDtypeF16) return launch_delta_e<f16>(a, head_dim, varlen, s);
  return launch_delta_e<bf16>(a, head_dim, varlen, s);
}

// The fused (atomic) kernel is compiled for bf16 only; fp16 problems always take the
// split backward.
template <class E, int D, bool FUSED>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  // with a sequence ranking (packed): 8 XCDs x ceil(units / 8) slots of whole sequences
  const int64_t units = (varlen && a.unit_order) ? 8 * (((int64_t)a.num_units + 7) / 8) : a.num_units;
  const int64_t nblk = units * a.Hkv * a.num_k_blocks;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(512);
  constexpr int smem = (int)bwd_smem_bytes<D, FUSED>();
#define EXATTN_BWD(C, M, V)                                                                    \
  do {                                                                                         \
    auto kfn = bwd_kernel<E, D, C, M, V, FUSED>;                                               \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);      \
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

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask,
                      bool varlen, bool fused, hipStream_t s) {
  if (dtype == kDtypeF16) {
    if (head_dim == 64) return launch_bwd_d<f16, 64, false>(a, causal, mask, varlen, s);
    return launch_bwd_d<f16, 128, false>(a, causal, mask, varlen, s);
  }
  if (head_dim == 64) {
    if (fused) return launch_bwd_d<bf16, 64, true>(a, causal, mask, varlen, s);
    return launch_bwd_d<bf16, 64, false>(a, causal, mask, varlen, s);
  }
  if (fused) return launch_bwd_d<bf16, 128, true>(a, causal, mask, varlen, s);
  return launch_bwd_d<bf16, 128, false>(a, causal, mask, varlen, s);
}

template <class E, int D>
static hipError_t launch_bwd_dq_d(const BwdArgs& a, bool causal, int mask, bool varlen,
                                  hipStream_t s) {
  const int per = (causal && !varlen) ? (a.num_q_blocks + 1) / 2 : a.num_q_blocks;
  const int64_t nblk = (int64_t)a.num_units * a.H * per;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(512);
#define EXATTN_DQ(C, M, V) hipLaunchKernelGGL((bwd_dq_kernel<E, D, C, M, V>), grid, block, 0, s, a)
  if (varlen) {
    if (causal) EXATTN_DQ(true, kMaskNone, true);
    else EXATTN_DQ(false, kMaskNone, true);
  } else if (causal) {
    if (mask == kMaskBool) EXATTN_DQ(true, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_DQ(true, kMaskAdd, false);
    else EXATTN_DQ(true, kMaskNone, false);
  } else {
    if (mask == kMaskBool) EXATTN_DQ(false, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_DQ(false, kMaskAdd, false);
    else EXATTN_DQ(false, kMaskNone, false);
  }
#undef EXATTN_DQ
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask,
                         bool varlen, hipStream_t s) {
  if (dtype == kDtypeF16) {
    if (head_dim == 64) return launch_bwd_dq_d<f16, 64>(a, causal, mask, varlen, s);
    return launch_bwd_dq_d<f16, 128>(a, causal, mask, varlen, s);
  }
  if (head_dim == 64) return launch_bwd_dq_d<bf16, 64>(a, causal, mask, varlen, s);
  return launch_bwd_dq_d<bf16, 128>(a, causal, mask, varlen, s);
}

int bwd_dq_block_m(int head_dim) { return DqTile<128>::BM; }

hipError_t launch_dq_reduce(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t n8 = (int64_t)a.rows_q * a.H * head_dim / 8;
  if (n8 <= 0) return hipSuccess;
  dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  hipLaunchKernelGGL(dq_reduce_kernel<bf16>, grid, block, 0, s, a, n8);
  return hipGetLastError();
}

hipError_t launch_q_tail(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int cpr = a.H * head_dim / 8;
  const int64_t n = (int64_t)a.rows_q * cpr;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  hipLaunchKernelGGL(q_tail_kernel, grid, block, 0, s, a, n, cpr);
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
