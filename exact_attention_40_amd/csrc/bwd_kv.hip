// Backward dK/dV kernel with the two roles of each wave pair one query tile apart.
//
// Same decomposition as the two-barrier dK/dV kernel in bwd.hip: one workgroup = 8 waves =
// 128 keys (four groups of 32) of one (unit, kv head), looping over every query head of the
// group and every 64-row query tile that can see the block; per key group one wave pair,
// both waves on one SIMD:
//   wave A: S = Q K^T, P = exp2(min(S*c + bias - lse2, 0)) (hidden entries 0), dV += P^T dO;
//           keeps K fragments and dV in registers; P goes to LDS as the bf16 (fp16) operand
//           fragments of its own dV product
//   wave B: dS = P * (dP - Delta) with P from LDS, dK += dS^T Q, dP = dO V^T;
//           keeps V fragments and dK in registers
// Wave B runs one tile behind wave A: in the phase where A forms S and P of tile t and
// adds dV, B forms dS and adds dK of tile t - 1 and computes dP of tile t (held in
// registers into the next phase). So while A spends the VALU on the exponentials, B keeps
// the SIMD's matrix unit busy, and one barrier per tile suffices. The buffers are rings
// sized for that lag and for copies two tiles ahead: Q x4 (B still reads tile t - 1 while
// tiles t + 1 and t + 2 arrive), dO x3, P x2, lse2 / Delta x3. Tiles and their lse2 and
// Delta rows are copied global -> LDS with asynchronous copies; each phase ends with one
// wait that leaves only the copies of tile t + 2 in flight, then the barrier.
//
// Stored dS (SDS, dense layouts): wave B also writes each dS fragment it forms, rounded to
// the input format as for its own dK product, so that a separate pass can form dQ = dS K
// without recomputing S and dP. Chunk (unit, head, 64-row query tile, key block, key group,
// 16-row slab) is 1 KB: 32 bytes per key, the lanes' 16-byte halves side by side, key index
// XOR 4 on odd slabs (the reader's transposed LDS reads then touch every bank once).
//
// Sources: dv = P^T dO and dk = dS^T q (flash-dmattn PR #122 "Fix NaN/Inf values in dV
// gradients during backward pass", section "Solution", item 2); P = exp(s - lse) from the
// stored LSE, with partial key and query tiles masked in the kernel (OpenWAM PR #64,
// "Summary"); every dk/dv row written, including keys no query sees (flash-dmattn PR #122,
// "Root Cause" 1); the exponent bounded above (PFCCLab cudnn-frontend PR #9 "DSA: fix dK
// SMEM handoff race and two latent NaN sources in the dense indexer", item 3).

#include "common.hpp"
#include "params.hpp"

namespace exattn {

template <int D>
struct KvTile {
  static constexpr int NW = 8;
  static constexpr int BN = 128;
  static constexpr int KG = BN / 32;             // key groups (wave pairs)
  static constexpr int BM = 64;                  // query rows per tile
  static constexpr int QB = BM / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int QBYTES = BM * D * 2;      // one Q or dO tile
  static constexpr int NQ = 4, NDO = 3, NP = 2, NST = 3;   // ring depths
  static constexpr int DO_BASE = NQ * QBYTES;
  static constexpr int P_BASE = DO_BASE + NDO * QBYTES;
  static constexpr int P_BYTES = KG * (BM / 16) * 64 * 16;   // bf16 P operand fragments of one tile
  static constexpr int ST_BASE = P_BASE + NP * P_BYTES;
  static constexpr int SMEM = ST_BASE + 2 * NST * BM * 4;  // + lse2 and Delta rings
  static_assert((BM * CPR) % (64 * NW) == 0, "even copy split");
  static_assert(SMEM <= 160 * 1024, "fits the 160 KB of LDS");
};

template <class E, int D, bool CAUSAL, int MASK, bool VARLEN, bool SDS>
__global__ void __launch_bounds__(512) bwd_kv_kernel(BwdArgs a) {
  nan_passing_clamp();   // NaN passes the clamped exponential below (no NaN is cleaned)
  static_assert(!(SDS && VARLEN), "stored dS is laid out for dense problems");
  using T = KvTile<D>;
  using V8 = typename Ty<E>::v8;
  using V4 = typename Ty<E>::v4;
  constexpr int RB = D * 2;                      // bytes per swizzled row
  constexpr int NKK = T::BM / 16;                // 16-row slabs per query tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* lse2_l = reinterpret_cast<float*>(smem + T::ST_BASE);   // [NST][BM]
  float* del_l = lse2_l + T::NST * T::BM;                         // [NST][BM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, j16 = lane & 15;
  const bool role_a = wave < T::KG;
  const int kg = role_a ? wave : wave - T::KG;   // key group of this wave

  // Block order: dense layouts keep the key blocks of one (unit, kv head) on one XCD
  // (xcd_remap), so its Q/dO re-reads hit that XCD's L2. Packed layouts with a ranking of
  // the sequences deal them to the XCDs in snake order (XCD x takes ranks 8s + x on even
  // slots s and 8s + 7 - x on odd ones), largest first, whole sequences per XCD.
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
  int64_t krow0, qb_off, kb_off, vb_off, dob_off, st_unit;
  if constexpr (VARLEN) {
    const SeqRows rq = seq_rows(a.cu_q, unit, a.Sq, a.max_sq);
    const SeqRows rk = seq_rows(a.cu_k, unit, a.Sk, a.max_sk);
    const int qs = rq.beg, ks = rk.beg;
    Sq = rq.len;
    Sk = rk.len;
    krow0 = ks;
    qb_off = (int64_t)qs * a.q_ss;
    kb_off = (int64_t)ks * a.k_ss;
    vb_off = (int64_t)ks * a.v_ss;
    dob_off = (int64_t)qs * a.do_ss;
    st_unit = qs;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
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

  // This pair's operand fragments in registers: K for wave A, V for wave B (zero past the
  // last key through the buffer range).
  const E* K = reinterpret_cast<const E*>(a.k) + kb_off + (int64_t)g * a.k_sh +
               (int64_t)kb0 * a.k_ss;
  const E* V = reinterpret_cast<const E*>(a.v) + vb_off + (int64_t)g * a.v_sh +
               (int64_t)kb0 * a.v_ss;
  V8 kv[T::DS];
  {
    const auto r = role_a ? make_rsrc(K, (uint32_t)((krows - 1) * a.k_ss + D) * 2u)
                          : make_rsrc(V, (uint32_t)((krows - 1) * a.v_ss + D) * 2u);
    const int st = role_a ? (int)a.k_ss : (int)a.v_ss;
#pragma unroll
    for (int s = 0; s < T::DS; ++s)
      kv[s] = __builtin_bit_cast(V8, buf_load16(r, (uint32_t)(kl_w * st + 16 * s + 8 * half) * 2u));
    // Consume the fragments here, so that these loads are complete before the tile loop:
    // otherwise the compiler keeps waiting for them inside the loop, where its vmcnt waits
    // would also wait for the asynchronous copies in flight.
#pragma unroll
    for (int s = 0; s < T::DS; ++s) asm volatile("" ::"v"(kv[s]));
  }

  // ---- per-lane LDS bases for ring slot 0; slots are added as run-time byte offsets ------
  // Row-operand reads (rows qb*32 + l32, d-slab ds): wave A reads Q, wave B reads dO.
  const unsigned char* aq[T::DS];
#pragma unroll
  for (int ds = 0; ds < T::DS; ++ds)
    aq[ds] = smem + (role_a ? 0 : T::DO_BASE) + l32 * RB + 16 * ((2 * ds + half) ^ swz_f<D>(l32));
  // Transposed reads (k = query rows 16kk + 4*half + (j16>>2) + 8*sec, columns db*32 +
  // 16*(grp&1) + 4*(j16&3)): wave A reads dO, wave B reads Q.
  const int tr_row = j16 >> 2;
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  const unsigned char* tq[T::DB][2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 4 * half + tr_row + 8 * sec;
    const unsigned char* base = smem + (role_a ? T::DO_BASE : 0) + row * RB + 8 * (j16 & 1);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) tq[db][sec] = base + 16 * ((4 * db + clow) ^ swz_f<D>(row));
  }
  unsigned char* pp = smem + T::P_BASE + kg * (NKK * 1024) + lane * 16;   // P hand-over
  const unsigned char* st_rd = reinterpret_cast<const unsigned char*>(lse2_l) + 16 * half;
  constexpr int DEL_OFF = T::NST * T::BM * 4;    // Delta ring, bytes after the lse2 ring

  f32x16 acc[T::DB];   // dV (wave A) or dK (wave B)
#pragma unroll
  for (int db = 0; db < T::DB; ++db) acc[db] = f32x16{};

  const float c2 = a.scale_log2;
  const uint8_t* mask_u8 = reinterpret_cast<const uint8_t*>(a.mask);
  const bf16* mask_bf = reinterpret_cast<const bf16*>(a.mask);
  const int qstart = CAUSAL ? min(kb0 / T::BM * T::BM, Sq) : 0;
  const int n_qt = (Sq - qstart + T::BM - 1) / T::BM;
  const int n_iter = a.group * n_qt;

  // Tile positions advance incrementally (query tile fastest, then head).
  struct TilePos { int head, q0; };
  const int h_beg = g * a.group;
  const int q_end = qstart + n_qt * T::BM;
  auto advance = [&](TilePos& p) {
    p.q0 += T::BM;
    if (p.q0 >= q_end) {
      p.q0 = qstart;
      ++p.head;
    }
  };

  // Staging: the Q and dO tiles and the tile's lse2 and Delta rows go straight into LDS
  // ring slots through asynchronous copies; rows past the end read as zero. Zero Q, dO and
  // Delta rows add nothing, and their lse2 of 0 is harmless: those rows are hidden in P (by
  // the boundary fix-up or by the masked form).
  auto load_stats = [&](const TilePos& tp, int slot) {
    if (wave < 2) {
      const int head = tp.head, qt0 = tp.q0;
      const int rows = min(T::BM, Sq - qt0);
      const int64_t st = (VARLEN ? (int64_t)head * a.lse_row + st_unit
                                 : ((int64_t)unit * a.H + head) * a.Sq) + qt0;
      const float* src = wave == 0 ? a.lse2 + st : a.delta + st;
      float* dst = (wave == 0 ? lse2_l : del_l) + slot * T::BM;
      copy4_to_lds(copy_rsrc(src, (uint32_t)rows * 4u), (uint32_t)lane * 4u, lds_addr(dst));
    }
  };
  auto load_tile = [&](const TilePos& tp, int qslot, int dslot) {
    const int head = tp.head, qt0 = tp.q0;
    const int rows = min(T::BM, Sq - qt0);
    const E* Qp = reinterpret_cast<const E*>(a.q) + qb_off + (int64_t)head * a.q_sh +
                  (int64_t)qt0 * a.q_ss;
    const E* Dp = reinterpret_cast<const E*>(a.dout) + dob_off + (int64_t)head * a.do_sh +
                  (int64_t)qt0 * a.do_ss;
    copy_tile_async<D, T::BM, T::NW>(smem + qslot * T::QBYTES,
                                     copy_rsrc(Qp, (uint32_t)((rows - 1) * a.q_ss + D) * 2u),
                                     (int)a.q_ss, wave, lane);
    copy_tile_async<D, T::BM, T::NW>(smem + T::DO_BASE + dslot * T::QBYTES,
                                     copy_rsrc(Dp, (uint32_t)((rows - 1) * a.do_ss + D) * 2u),
                                     (int)a.do_ss, wave, lane);
  };
  constexpr int NCOPY = 2 * (T::BM * T::CPR / 64 / T::NW);   // tile copies per wave

  TilePos prv = {h_beg, qstart};   // tile t - 1 (wave B's dS and dK)
  TilePos cur = {h_beg, qstart};   // tile t (wave A)
  TilePos nxt = cur;               // tile t + 1
  advance(nxt);
  TilePos nx2 = nxt;               // tile t + 2
  advance(nx2);
  if (n_iter > 0) {
    load_tile(cur, 0, 0);
    load_stats(cur, 0);
  }
  if (n_iter > 1) {
    load_tile(nxt, 1, 1);
    sync_copies<NCOPY>();          // tile 0 and its stats landed; tile 1 may be in flight
  } else {
    sync_copies<0>();
  }

  // Wave A: S, then P of tile t. Wave B: dP of tile t, held across the barrier until dS of
  // tile t is formed in the next phase.
  f32x16 sp[T::QB];

  // ---- wave A, one tile: S = Q K^T; P; P -> LDS; dV += P^T dO -------------------------------
  // Without a mask, the exponentials of query block 0 are issued between the MFMAs of block
  // 1, and those of block 1 between the dV MFMAs of block 0, so the wave itself overlaps
  // VALU and MFMA work. With a mask they follow the S product, so the mask reads of a tile
  // go out together.
  constexpr bool ILV = MASK == kMaskNone;
  auto phase_a = [&](int qslot, int dslot, int sslot, int pslot, bool edge, auto copy_next) {
    const int head = cur.head, qt0 = cur.q0;
    if (!ILV) copy_next();
    const int qo = qslot * T::QBYTES, dqo = dslot * T::QBYTES;
    const int64_t m_base = (int64_t)unit * a.m_sb + (int64_t)head * a.m_sh;
    // P for register r of query block qb, in place; the lse2 of four rows is read with the
    // first of them (the calls come in register order). With a mask every tile takes the
    // masked form; without one, the plain form runs everywhere and boundary tiles (partial
    // key or query tile, causal diagonal) then zero the hidden entries (hide_p), which gives
    // the same values: the masked form differs only by that select.
    f32x4 l2v;
    auto pexp = [&](int qb, int r) {
      if ((r & 3) == 0) l2v = lds_at<f32x4>(st_rd, sslot * T::BM * 4 + (qb * 32 + 8 * (r >> 2)) * 4);
      const float lv = l2v[r & 3];
      if constexpr (MASK == kMaskNone) {
        sp[qb][r] = exp2_le1(fmaf(sp[qb][r], c2, -lv));
      } else {
        // Branch-free visibility: mask reads use indices clamped into range.
        const int qi = qt0 + qb * 32 + acc_row(r, half);
        bool vis = (qi < Sq) && (kw < Sk);
        if (CAUSAL) vis = vis && (kw <= qi);
        float b2 = 0.f;
        const int64_t mi = m_base + (int64_t)min(qi, Sq - 1) * a.m_si + min(kw, Sk - 1);
        if (MASK == kMaskBool) {
          vis = vis && (mask_u8[mi] != 0);
        } else {
          const float bias = (float)mask_bf[mi];
          vis = vis && (bias != -INFINITY);
          b2 = vis ? bias_log2(bias) : 0.f;
        }
        const float e2 = exp2_le1(fmaf(sp[qb][r], c2, b2 - lv));
        sp[qb][r] = vis ? e2 : 0.f;
      }
    };
    auto hide_p = [&](int qb) {
      if (MASK == kMaskNone && edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qt0 + qb * 32 + acc_row(r, half);
          bool vis = (qi < Sq) && (kw < Sk);
          if (CAUSAL) vis = vis && (kw <= qi);
          sp[qb][r] = vis ? sp[qb][r] : 0.f;
        }
      }
    };
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) sp[qb] = f32x16{};
    {
      // S MFMAs query block first; Q row fragments read four MFMAs ahead.
      constexpr int NF = T::QB * T::DS;
      constexpr int EPM = 16 / T::DS;            // block-0 exponentials per block-1 MFMA
      auto frag = [&](int f) { return lds_at<V8>(aq[f % T::DS] + qo, (f / T::DS) * 32 * RB); };
      V8 fr[4] = {frag(0), frag(1), frag(2), frag(3)};
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int qb = f / T::DS, ds = f % T::DS;
        sp[qb] = mfma32(fr[f % 4], kv[ds], sp[qb]);
        if (f + 4 < NF) fr[f % 4] = frag(f + 4);
        if (ILV && qb == 1) {
#pragma unroll
          for (int e = 0; e < EPM; ++e) pexp(0, ds * EPM + e);
        }
        __builtin_amdgcn_sched_barrier(0x0004);
      }
    }
    if (!ILV) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pexp(0, r);
#pragma unroll
      for (int r = 0; r < 16; ++r) pexp(1, r);
    }
    if (ILV) copy_next();
    hide_p(0);
    {
      // dV += P^T dO over 16-row slabs; transposed dO fragments read one slab ahead.
      constexpr int EPM = 16 / (2 * T::DB);      // block-1 exponentials per block-0 MFMA
      V4 tb[2][T::DB][2];
      auto tload = [&](int kk, int slot) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          tb[slot][db][0] = tr_at<V4>(tq[db][0] + dqo, 16 * kk * RB);
          tb[slot][db][1] = tr_at<V4>(tq[db][1] + dqo, 16 * kk * RB);
        }
      };
      tload(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int qb = kk >> 1, hs = (kk & 1) * 8;
        const V8 pa = cvt8<V8>(sp[qb][hs + 0], sp[qb][hs + 1], sp[qb][hs + 2], sp[qb][hs + 3],
                               sp[qb][hs + 4], sp[qb][hs + 5], sp[qb][hs + 6], sp[qb][hs + 7]);
        *reinterpret_cast<V8*>(pp + pslot * T::P_BYTES + kk * 1024) = pa;
        if (kk + 1 < NKK) tload(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          acc[db] = mfma32(pa, cat44(tb[kk & 1][db][0], tb[kk & 1][db][1]), acc[db]);
          if (ILV && qb == 0) {
#pragma unroll
            for (int e = 0; e < EPM; ++e) pexp(1, ((kk & 1) * T::DB + db) * EPM + e);
          }
          __builtin_amdgcn_sched_barrier(0x0004);
        }
        if (kk == 1) hide_p(1);
      }
    }
  };

  // ---- wave B, previous tile: dS = P * (dP - Delta); dK += dS^T Q ----------------------------
  auto dk_step = [&](int qslot, int pslot, int sslot, const TilePos& tp) {
    const int tro = qslot * T::QBYTES;
    const unsigned char* pr = pp + pslot * T::P_BYTES;
    E* dsw = nullptr;   // this wave's four dS chunks of the tile (SDS)
    if constexpr (SDS) {
      const int64_t chunk = ((((int64_t)unit * a.H + tp.head) * a.ds_nqt + tp.q0 / T::BM) *
                                 a.num_k_blocks + kbi) * 16 + kg * 4;
      dsw = reinterpret_cast<E*>(a.ds) + chunk * 512 + half * 8;
    }
    V4 tb[2][T::DB][2];
    auto tload = [&](int kk, int slot) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        tb[slot][db][0] = tr_at<V4>(tq[db][0] + tro, 16 * kk * RB);
        tb[slot][db][1] = tr_at<V4>(tq[db][1] + tro, 16 * kk * RB);
      }
    };
    tload(0, 0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int qb = kk >> 1, hs = (kk & 1) * 8, rg0 = 2 * (kk & 1);
      float d[8];
      const V8 p8 = *reinterpret_cast<const V8*>(pr + kk * 1024);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 pv = {(float)p8[4 * h], (float)p8[4 * h + 1], (float)p8[4 * h + 2], (float)p8[4 * h + 3]};
        const f32x4 dd =
            lds_at<f32x4>(st_rd, DEL_OFF + sslot * T::BM * 4 + (qb * 32 + 8 * (rg0 + h)) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[4 * h + e] = pv[e] * (sp[qb][hs + 4 * h + e] - dd[e]);
      }
      const V8 sa = cvt8<V8>(d[0], d[1], d[2], d[3], d[4], d[5], d[6], d[7]);
      if constexpr (SDS)   // streaming store: dS is read back once, by the dQ pass
        __builtin_nontemporal_store(sa, reinterpret_cast<V8*>(dsw + kk * 512 + (l32 ^ (4 * (kk & 1))) * 16));
      if (kk + 1 < NKK) tload(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        acc[db] = mfma32(sa, cat44(tb[kk & 1][db][0], tb[kk & 1][db][1]), acc[db]);
        __builtin_amdgcn_sched_barrier(0x0004);
      }
    }
  };

  // ---- wave B, this tile: dP = dO V^T into sp ---------------------------------------------------
  auto dp_step = [&](int dslot) {
    const int ro = dslot * T::QBYTES;
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) sp[qb] = f32x16{};
    constexpr int NF = T::QB * T::DS;
    auto frag = [&](int f) { return lds_at<V8>(aq[f % T::DS] + ro, (f / T::DS) * 32 * RB); };
    V8 fr[4] = {frag(0), frag(1), frag(2), frag(3)};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int qb = f / T::DS, ds = f % T::DS;
      sp[qb] = mfma32(fr[f % 4], kv[ds], sp[qb]);
      if (f + 4 < NF) fr[f % 4] = frag(f + 4);
      __builtin_amdgcn_sched_barrier(0x0004);
    }
  };

  // Phase t (0 .. n_iter): A works on tile t (t < n_iter), B finishes tile t - 1 (t >= 1)
  // and starts tile t (t < n_iter). Ring slots: Q and the stats t % 3, dO and P t % 2.
  // Each role runs its own copy of the phase loop, so that the register allocation of one
  // role does not constrain the other's; both copies pass the same n_iter + 1 barriers.
  auto run_phases = [&](auto work) {
    int s3 = 0, s2 = 0, q4 = 0, d3 = 0;
    for (int t = 0; t <= n_iter; ++t) {
      const int n3 = s3 == 2 ? 0 : s3 + 1;
      const int p3 = s3 == 0 ? 2 : s3 - 1;
      const int q4n = (q4 + 2) & 3, q4p = (q4 + 3) & 3;
      const int d3n = d3 == 0 ? 2 : d3 - 1;
      if (t + 1 < n_iter) load_stats(nxt, n3);
      // The copies of tile t + 2 are issued mid-phase (by wave A after its S product, by
      // wave B between its dK and dP products), not at the start of the phase: issued by all
      // waves at once, they arrived in LDS together with the phase's first operand reads and
      // stalled them (measured 8-10% slower).
      auto copy_next = [&]() { if (t + 2 < n_iter) load_tile(nx2, q4n, d3n); };
      work(t, s3, s2, p3, q4, q4p, d3, copy_next);
      // tile t + 1 and its stats have landed (and P of tile t is written); the copies of
      // tile t + 2 may still be in flight
      if (t + 2 < n_iter) sync_copies<NCOPY>();
      else sync_copies<0>();
      prv = cur;
      cur = nxt;
      nxt = nx2;
      advance(nx2);
      s3 = n3;
      s2 ^= 1;
      q4 = (q4 + 1) & 3;
      d3 = d3 == 2 ? 0 : d3 + 1;
    }
  };
  if (role_a) {
    run_phases([&](int t, int s3, int s2, int, int q4, int, int d3, auto copy_next) {
      if (t < n_iter) {
        const int qt0 = cur.q0;
        const bool edge = (kb0 + T::BN > Sk) || (qt0 + T::BM > Sq) ||
                          (CAUSAL && kb0 + T::BN - 1 > qt0);
        phase_a(q4, d3, s3, s2, edge, copy_next);
      } else {
        copy_next();
      }
    });
  } else {
    run_phases([&](int t, int, int s2, int p3, int, int q4p, int d3, auto copy_next) {
      if (t >= 1) dk_step(q4p, s2 ^ 1, p3, prv);
      copy_next();
      if (t < n_iter) dp_step(d3);
    });
  }

  // Epilogue: dV (wave A) or dK times scale (wave B) in the input format into contiguous
  // [rows_k, Hkv, D], staged through this wave's slice of LDS (every wave has passed the
  // last barrier) so that whole rows are stored; rows past the sequence end are not
  // written. Keys that no query sees are written as exact zeros.
  static_assert(T::NW * 32 * D * 2 <= T::SMEM, "epilogue staging fits the LDS");
  const float sc = role_a ? 1.f : a.scale;
  E* dst = reinterpret_cast<E*>(role_a ? a.dv : a.dk) + ((krow0 + kb0 + kg * 32) * a.Hkv + g) * D;
  wave_store_cols<D, E>(smem + wave * 32 * D * 2, acc, sc, dst, (int64_t)a.Hkv * D,
                        krows - kg * 32, lane);
}

template <class E, int D, bool SDS>
static hipError_t launch_bwd_kv_d(const BwdArgs& a, bool causal, int mask, bool varlen, hipStream_t s) {
  // with a sequence ranking (packed): 8 XCDs x ceil(units / 8) slots of whole sequences
  const int64_t units = (varlen && a.unit_order) ? 8 * (((int64_t)a.num_units + 7) / 8) : a.num_units;
  const int64_t nblk = units * a.Hkv * a.num_k_blocks;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(512);
  constexpr int smem = KvTile<D>::SMEM;
#define EXATTN_BWD_KV(C, M, V)                                                                 \
  do {                                                                                         \
    auto kfn = bwd_kv_kernel<E, D, C, M, V, SDS && !V>;                                        \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);      \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL(kfn, grid, block, smem, s, a);                                          \
  } while (0)
  if (varlen) {
    if (causal) EXATTN_BWD_KV(true, kMaskNone, true);
    else EXATTN_BWD_KV(false, kMaskNone, true);
  } else if (causal) {
    if (mask == kMaskBool) EXATTN_BWD_KV(true, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_BWD_KV(true, kMaskAdd, false);
    else EXATTN_BWD_KV(true, kMaskNone, false);
  } else {
    if (mask == kMaskBool) EXATTN_BWD_KV(false, kMaskBool, false);
    else if (mask == kMaskAdd) EXATTN_BWD_KV(false, kMaskAdd, false);
    else EXATTN_BWD_KV(false, kMaskNone, false);
  }
#undef EXATTN_BWD_KV
  return hipGetLastError();
}

template <bool SDS>
static hipError_t launch_bwd_kv_s(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask,
                                  bool varlen, hipStream_t s) {
  if (dtype == kDtypeF16) {
    if (head_dim == 64) return launch_bwd_kv_d<f16, 64, SDS>(a, causal, mask, varlen, s);
    return launch_bwd_kv_d<f16, 128, SDS>(a, causal, mask, varlen, s);
  }
  if (head_dim == 64) return launch_bwd_kv_d<bf16, 64, SDS>(a, causal, mask, varlen, s);
  return launch_bwd_kv_d<bf16, 128, SDS>(a, causal, mask, varlen, s);
}

hipError_t launch_bwd_kv(const BwdArgs& a, int head_dim, int dtype, bool causal, int mask,
                         bool varlen, bool store_ds, hipStream_t s) {
  if (store_ds && !varlen) return launch_bwd_kv_s<true>(a, head_dim, dtype, causal, mask, false, s);
  return launch_bwd_kv_s<false>(a, head_dim, dtype, causal, mask, varlen, s);
}

}  // namespace exattn
