// fp8 forward: attention over OCP e4m3 q, k, v with per-tensor descales, an online softmax
// with a lazy rescale whose rebase lowers the base by at most a fixed bound, bf16 output
// and an fp32 LSE.
//
// What it computes follows FlyDSL PR #1033 ("[Bugfix][Kernel] Fix NaN from the lazy rescale
// on a wide score range", section "The fp8 helper, second commit"):
//   * scores enter the softmax already multiplied by the logit scale
//     c2 = scale * q_descale * k_descale * log2(e), and the rescale test compares the tile
//     max with the running max on that scale (threshold kFp8Tau, log2 units);
//   * the test is wave-wide: when any of the wave's 32 rows has a tile max more than the
//     threshold above its base, every row of the wave is rebased onto its own tile max,
//     also when that is lower than its base (this keeps the tile's exponentials near 1,
//     where e4m3 resolves them best), but never more than kFp8Bound below the row's
//     running max, so the row's sums stay within 2^kFp8Bound of their max-based values
//     however many rebases other rows cause (a cap per rebase would let drops compound
//     past the fp32 range);
//   * between rebases the exponentials are p = 2^(s * c2 - m) <= 2^kFp8Tau = 256, inside
//     the e4m3 range (448); P is rounded to e4m3 (nearest even) for the P.V product, while
//     the row sum adds the unrounded p.
//
// Work decomposition: one workgroup = 8 waves = one (batch, head, 256-row query tile);
// each wave owns 32 query rows (lane l and l ^ 32 share a row and split its keys). K and V
// tiles of 64 keys x 128 bytes are copied straight into LDS (buffer loads with an LDS
// destination, zero past the last key), K one tile further ahead than V.
// Software pipeline: iteration t issues the S MFMAs of tile t+1 next to the exponentials
// of tile t, then the PV MFMAs of tile t next to the row max of tile t+1; the rescale test
// for tile t+1 follows, outside the interleaved region.
//   S^T = K Q^T: 32x32x64 fp8 MFMAs, A = K rows from LDS (32 contiguous bytes per lane),
//     B = Q^T from registers; a lane's accumulators hold one query column.
//   O^T += V^T P^T: A = V^T from transposed byte reads of the row-major V tile
//     (ds_read_b64_tr_b8), B = the lane's 32 exponentials of its query, packed to e4m3.
// The 64 keys of a tile reach the PV operands in the order the S^T accumulator layout
// gives them: byte j of lane-half h is key 32*(j/16) + 8*((j%16)/4) + 4*h + j%4, and the
// transposed V reads fetch the same keys (read t of 8 bytes covers keys 16t + {4h..4h+3,
// 8+4h..8+4h+3}).

#include <type_traits>

#include "common.hpp"
#include "params.hpp"

namespace exattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kFp8Tau = 8.f;     // rescale threshold (log2 units)
constexpr float kFp8Bound = 16.f;  // largest distance of the base below the running max (log2)

// D[32x32] += A[32x64] * B[64x32], e4m3 in, fp32 accumulate. Lane l holds row (A) or column
// (B) l % 32 and 32 k-slots (bytes) for k-half l / 32; A's and B's slots pair up, so any
// slot-to-k assignment shared by A and B gives the same product. Result layout as the
// 16-bit form: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Transposed byte read: within each 16-lane group, lanes 2m and 2m+1 point at bytes 0-7 and
// 8-15 of row m's 16-column slice; lane i receives column i of the eight rows (byte m =
// row m).
__device__ __forceinline__ i32x2 lds_read_tr8(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(const_cast<unsigned char*>(p)));
}

struct Fp8Tile {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;      // query rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int D = 128;
  static constexpr int RB = D;            // bytes per LDS row
  static constexpr int TB = BN * RB;      // bytes per K or V tile
  static_assert(BN * RB / 16 == NT, "one 16-byte chunk per thread fills a tile");
};

// 16-byte chunk permutations of a 128-byte LDS row (8 chunks). K: reads of 16 rows of one
// parity at one chunk cover the 8 chunk positions, so every 16-lane phase touches all 64
// banks once. V: the transposed reads of a half-wave cover rows {4h..4h+3, 8+4h..8+4h+3}
// (+16t) at chunks 2db and 2db+1; the four rows of one parity land on distinct chunk pairs.
__device__ __forceinline__ int kswz8(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int vswz8(int row) { return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1)); }

// Stage one 64 x 128-byte tile: thread t of the workgroup fills LDS chunk t (row t/8,
// position t%8) with the global chunk that the swizzle places there. Rows past the
// buffer resource's range read as zero.
template <bool IS_V>
__device__ __forceinline__ void copy_fp8_tile(unsigned char* dst, __amdgpu_buffer_rsrc_t rs,
                                              int64_t stride, int wave, int lane) {
  const int pos = wave * 64 + lane;
  const int row = pos >> 3, slot = pos & 7;
  const int c = slot ^ (IS_V ? vswz8(row) : kswz8(row));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(dst + wave * 64 * 16), 16,
      (int)(row * stride + c * 16), 0, 0, 0);
}

template <bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
fwd_fp8_kernel(FwdArgs a) {
  using T = Fp8Tile;
  constexpr int V_OFF = 2 * T::TB;
  // K[2], V[2] tiles (32 KB); the epilogue stages each wave's 32 x 128 bf16 rows (64 KB).
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::NW * 32 * T::D * 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // Dense causal: block j of a (batch, head) runs query tiles n-1-j and j (equal work).
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qtile, qtile2 = -1, uh;
  if constexpr (CAUSAL) {
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
  const int Sq = a.Sq, Sk = a.Sk;
  const unsigned char* Q = reinterpret_cast<const unsigned char*>(a.q) + (int64_t)unit * a.q_sb + (int64_t)head * a.q_sh;
  const unsigned char* K = reinterpret_cast<const unsigned char*>(a.k) + (int64_t)unit * a.k_sb + (int64_t)g * a.k_sh;
  const unsigned char* V = reinterpret_cast<const unsigned char*>(a.v) + (int64_t)unit * a.v_sb + (int64_t)g * a.v_sh;
  const int64_t o_base = (int64_t)unit * a.o_sb + (int64_t)head * a.o_sh;
  const int64_t lse_base = ((int64_t)unit * a.H + head) * a.Sq;

  // A negative logit scale is folded into the sign of Q (bit 7 of each e4m3 byte).
  const float c2s = a.scale_log2;
  const float c2 = fabsf(c2s);
  const int qsign = c2s < 0.f ? (int)0x80808080u : 0;

  // Per-lane LDS read bases. K: row l32 (+32 per S tile, immediate), chunks 4kk + 2*half
  // and +1. V: lane group G = lane / 16 reads rows 8*(m/4) + 4*(G/2) + m%4 (m = (lane%16)/2,
  // +16 per read, immediate) at columns 32db + 16*(G%2) + 8*(lane%2).
  const unsigned char* kb[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
      kb[kk][sub] = smem + l32 * T::RB + 16 * ((4 * kk + 2 * half + sub) ^ kswz8(l32));
  const int grp = lane >> 4, i16 = lane & 15, m8 = i16 >> 1;
  const int vrow = 8 * (m8 >> 2) + 4 * (grp >> 1) + (m8 & 3);
  const unsigned char* vb[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vb[db] = smem + V_OFF + vrow * T::RB + 16 * ((2 * db + (grp & 1)) ^ vswz8(vrow)) + 8 * (i16 & 1);

  auto run_tile = [&](const int qtile) __attribute__((always_inline)) {
    const int qt0 = qtile * T::BM;
    if (qt0 >= Sq) return;
    const int qi = qt0 + wave * 32 + l32;

    // Q^T fragments: k-chunk kk holds bytes 64kk + 32*half .. +31 of the lane's query row.
    i32x8 qf[2];
    if (qi < Sq) {
      const unsigned char* row = Q + (int64_t)qi * a.q_ss + 32 * half;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 lo = ldg16(row + 64 * kk), hi = ldg16(row + 64 * kk + 16);
        qf[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]} ^ qsign;
      }
    } else {
      qf[0] = qf[1] = i32x8{};
    }

    const int kend = CAUSAL ? min(Sk, qt0 + T::BM) : Sk;
    const int ntiles = (kend + T::BN - 1) / T::BN;
    // Tiles that need no key masking for any row of the workgroup.
    int n_plain = Sk / T::BN;
    if (CAUSAL) n_plain = min(n_plain, (qt0 + 1) / T::BN);
    n_plain = min(n_plain, ntiles);

    auto load_k = [&](int t, int buf) {
      const int kb0 = t * T::BN;
      const int rows = min(T::BN, Sk - kb0);
      copy_fp8_tile<false>(smem + buf * T::TB,
                           make_rsrc(K + (int64_t)kb0 * a.k_ss, (uint32_t)((rows - 1) * a.k_ss + T::D)),
                           a.k_ss, wave, lane);
    };
    auto load_v = [&](int t, int buf) {
      const int kb0 = t * T::BN;
      const int rows = min(T::BN, Sk - kb0);
      copy_fp8_tile<true>(smem + V_OFF + buf * T::TB,
                          make_rsrc(V + (int64_t)kb0 * a.v_ss, (uint32_t)((rows - 1) * a.v_ss + T::D)),
                          a.v_ss, wave, lane);
    };
    // Key kj visible to this lane's row (tiles that need masking only).
    auto visible = [&](int kj) -> bool {
      bool vis = kj < Sk && qi < Sq;
      if (CAUSAL) vis = vis && kj <= qi;
      return vis;
    };
    // K fragment i = 2*kk + st (k-chunk kk, keys 32st..32st+31) of the tile at byte kofs.
    auto kfrag = [&](int kofs, int i) -> i32x8 {
      const u32x4 lo = lds_at<u32x4>(kb[i >> 1][0], kofs + (i & 1) * 32 * T::RB);
      const u32x4 hi = lds_at<u32x4>(kb[i >> 1][1], kofs + (i & 1) * 32 * T::RB);
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // V^T fragment of d-block db of the V tile at byte vofs: four transposed 8-byte reads.
    auto vfrag = [&](int vofs, int db) -> i32x8 {
      const i32x2 r0 = lds_read_tr8(vb[db] + vofs + 0 * 16 * T::RB);
      const i32x2 r1 = lds_read_tr8(vb[db] + vofs + 1 * 16 * T::RB);
      const i32x2 r2 = lds_read_tr8(vb[db] + vofs + 2 * 16 * T::RB);
      const i32x2 r3 = lds_read_tr8(vb[db] + vofs + 3 * 16 * T::RB);
      return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    };

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m_run = -INFINITY, m_max = -INFINITY, l_run = 0.f;   // base, running max, sum

    // After tile t's max mt (log2 units) is known: the wave-wide test, and the rebase onto
    // the tile max at most kFp8Bound below the running max.
    auto update = [&](float mt) {
      m_max = fmaxf(m_max, mt);
      if (__builtin_amdgcn_ballot_w64(mt - m_run > kFp8Tau) != 0) {
        const float m_new = fmaxf(mt, m_max - kFp8Bound);
        const float corr = (m_run == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= corr;
        m_run = m_new;
      }
    };

    // Scores of one tile: [st] accumulators, rows = keys 32st + acc_row, column = query.
    using Scores = f32x16[2];

    // Iteration body as one instruction stream: the four S MFMAs of tile t+1, each with
    // eight exponentials of tile t, then the four PV MFMAs of tile t, each with eight
    // elements of tile t+1's row max. Scheduling fences (only scalar instructions may
    // cross) keep the matrix and vector work of the wave interleaved. MC / MN: tile t /
    // t+1 needs masking. Returns tile t+1's row max in log2 units.
    auto body = [&](Scores& nxt, Scores& cur, int t, auto par_tag, auto mc_tag, auto mn_tag) -> float {
      constexpr int PAR = decltype(par_tag)::value;
      constexpr bool MC = decltype(mc_tag)::value;
      constexpr bool MN = decltype(mn_tag)::value;
      constexpr int KO = (PAR ^ 1) * T::TB;       // K of tile t + 1
      constexpr int VO = PAR * T::TB;             // V of tile t (vb[] includes V_OFF)
      const int kc0 = t * T::BN, kn0 = kc0 + T::BN;
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      nxt[0] = f32x16{};
      nxt[1] = f32x16{};
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
      i32x8 kf = kfrag(KO, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        i32x8 kn;
        if (i + 1 < 4) kn = kfrag(KO, i + 1);
        nxt[i & 1] = mfma32_e4m3(kf, qf[i >> 1], nxt[i & 1]);
        kf = kn;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = 8 * i + u, st = e >> 4, r = e & 15;
          float pe;
          if constexpr (!MC) {
            pe = fast_exp2(fmaf(cur[st][r], c2, -m_use));
          } else {
            pe = visible(kc0 + 32 * st + acc_row(r, half)) ? fast_exp2(fmaf(cur[st][r], c2, -m_use)) : 0.f;
          }
          cur[st][r] = pe;
          rs[r & 3] += pe;
          asm volatile("" : "+v"(rs[r & 3]));   // pin this step's exponential and sum here
        }
        __builtin_amdgcn_sched_barrier(0x0004);
      }
      asm volatile("" : "+v"(rs[0]), "+v"(rs[1]), "+v"(rs[2]), "+v"(rs[3]));
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      // e4m3 B operand: byte 16*st + r holds the exponential of key 32st + acc_row(r, half)
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int st = w >> 2, r = 4 * (w & 3);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(cur[st][r], cur[st][r + 1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(cur[st][r + 2], cur[st][r + 3], word, true);
        pf[w] = word;
      }
      float mx = -INFINITY;
      i32x8 vf = vfrag(VO, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        i32x8 vn;
        if (db + 1 < 4) vn = vfrag(VO, db + 1);
        o[db] = mfma32_e4m3(vf, pf, o[db]);
        vf = vn;
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          const int e0 = 8 * db + u, e1 = e0 + 1;
          float x0 = nxt[e0 >> 4][e0 & 15], x1 = nxt[e1 >> 4][e1 & 15];
          if constexpr (MN) {
            x0 = visible(kn0 + 32 * (e0 >> 4) + acc_row(e0 & 15, half)) ? x0 * c2 : -INFINITY;
            x1 = visible(kn0 + 32 * (e1 >> 4) + acc_row(e1 & 15, half)) ? x1 * c2 : -INFINITY;
          }
          mx = fmaxf(fmaxf(mx, x0), x1);
          asm volatile("" : "+v"(mx));   // pin this step's part of the max chain here
        }
        __builtin_amdgcn_sched_barrier(0x0004);
      }
      asm volatile("" : "+v"(mx));
      return MN ? pair_max32(mx) : pair_max32(mx) * c2;
    };

    // Tile j's K lives in K buffer j & 1 and its V in V buffer j & 1.
    Scores sa, sb;
    if (ntiles > 0) {
      load_k(0, 0);
      load_v(0, 0);
    }
    if (ntiles > 1) load_k(1, 1);
    wait_vmem();
    __syncthreads();
    if (ntiles > 0) {
      sa[0] = f32x16{};
      sa[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i & 1] = mfma32_e4m3(kfrag(0, i), qf[i >> 1], sa[i & 1]);
      float mx = -INFINITY;
      const bool masked = n_plain == 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int st = e >> 4, r = e & 15;
        const float x = sa[st][r] * c2;
        mx = fmaxf(mx, (!masked || visible(32 * st + acc_row(r, half))) ? x : -INFINITY);
      }
      update(pair_max32(mx));
    }
    __syncthreads();  // every wave has read K_0 before K_2 replaces it

    // Iteration t. K buffer PAR (K_t, read by the previous iteration) is refilled with
    // K_{t+2}; V buffer PAR ^ 1 (V_{t-1}) with V_{t+1}. When t + 1 == ntiles the S MFMAs
    // read a stale K buffer and their result is discarded.
    auto iteration = [&](int t, Scores& cur, Scores& nxt, auto par_tag, auto mask_cur, auto mask_nxt) {
      constexpr int PAR = decltype(par_tag)::value;
      if (t + 2 < ntiles) load_k(t + 2, PAR);
      if (t + 1 < ntiles) load_v(t + 1, PAR ^ 1);
      const float mt = body(nxt, cur, t, par_tag, mask_cur, mask_nxt);
      if (t + 1 < ntiles) update(mt);
      wait_vmem();      // this thread's chunks of K_{t+2} and V_{t+1} are in LDS
      __syncthreads();  // ... everyone's; every wave is done with K_{t+1} and V_t
    };

    using F = std::integral_constant<bool, false>;
    using Tr = std::integral_constant<bool, true>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int t = 0;
    for (; t + 2 < n_plain; t += 2) {
      iteration(t, sa, sb, P0{}, F{}, F{});
      iteration(t + 1, sb, sa, P1{}, F{}, F{});
    }
    // Remaining tiles in the masked form, still in pairs (the pending scores of the next
    // tile are in sa at the top of each trip); one form per loop keeps the register
    // allocation of the two loops apart.
    for (; t < ntiles; t += 2) {
      iteration(t, sa, sb, P0{}, Tr{}, Tr{});
      if (t + 1 < ntiles) iteration(t + 1, sb, sa, P1{}, Tr{}, Tr{});
    }

    // Epilogue: out = O * v_descale / l as bf16 rows (through this wave's LDS slice; the
    // tile buffers are free after the last barrier), lse in natural-log units.
    const float l = l_run + wave_xor32(l_run);
    const float inv = l != 0.f ? a.v_descale / l : 0.f;   // NaN propagates
    const int r0 = qt0 + wave * 32;
    bf16* orow = reinterpret_cast<bf16*>(a.out) + o_base + (int64_t)r0 * a.o_ss;
    wave_store_rows<T::D, bf16>(smem + wave * 32 * T::D * 2, o, inv, orow, a.o_ss, Sq - r0, lane);
    if (qi < Sq && half == 0) {
      const float mu = (m_run == -INFINITY) ? 0.f : m_run;
      a.lse[lse_base + qi] = l != 0.f ? (mu + log2f(l)) * kLn2 : -INFINITY;
    }
  };

  run_tile(qtile);
  if (qtile2 >= 0) {
    __syncthreads();  // the first tile's epilogue is done with LDS
    run_tile(qtile2);
  }
}

int fwd_fp8_block_m() { return Fp8Tile::BM; }

hipError_t launch_fwd_fp8(const FwdArgs& a, bool causal, hipStream_t s) {
  const int per = causal ? (a.num_q_tiles + 1) / 2 : a.num_q_tiles;
  const int64_t nblk = (int64_t)a.num_units * a.H * per;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(Fp8Tile::NT);
  if (causal) hipLaunchKernelGGL((fwd_fp8_kernel<true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((fwd_fp8_kernel<false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace exattn
