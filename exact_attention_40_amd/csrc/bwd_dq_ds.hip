// dQ from the stored dS: dQ = dS K over the key tiles, for the backward whose dK/dV kernel
// writes every dS fragment it forms (dense layouts). This replaces the dQ kernel that
// recomputes S, P, dP and dS per key tile (6 D FLOP per pair) by the bare product (2 D FLOP
// per pair) over 2 bytes of dS per pair read from HBM: the pass is bound by that read.
//
// One workgroup = 8 waves = 256 query rows of one (unit, head); each wave owns 32 rows.
// Per tile of 64 keys the K tile (row-major, swizzled as in the other kernels) and the
// 256 x 64 dS tile go global -> LDS through asynchronous copies, three stages deep, two
// tiles ahead; the dS copies are streaming loads (each chunk is read once), which keeps
// the K tiles, re-read by every query block of the head, in L2. Per 16-key slab the wave forms
//   dQ^T += K^T dS^T
// with both operands read transposed from LDS: K^T as in the recomputing dQ kernel, and
// dS^T from the stored chunks (32 bytes per key, each 8-byte piece four consecutive query
// rows of one key), so that lane = query column and the k order (keys 4*half + 0..3, then
// 8 + 4*half + 0..3) is the same for both. dQ accumulates in registers over every key tile
// in a fixed order and is written once, times the scale, in the input format: bitwise
// reproducible.
//
// Blocks the dK/dV kernel never wrote (causal: query tiles that end before the key block
// starts; query tiles past the end) are fetched through an empty buffer range, so they read
// as zero and no byte outside the written chunks is touched.
//
// Sources: dq = dS k (flash-dmattn PR #122 "Fix NaN/Inf values in dV gradients during
// backward pass", section "Solution", item 2, which names the three gradient products);
// deterministic dQ without atomics (the backward's dQ accumulation in NVIDIA cudnn-frontend
// PR #429, "Fix stream-ordering and input-validation holes in the SM100 DSA backward
// interface", is the atomic alternative).

#include "common.hpp"
#include "params.hpp"

namespace exattn {

template <int D>
struct DqsTile {
  static constexpr int NW = 8;
  static constexpr int BM = NW * 32;             // query rows per workgroup
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int DB = D / 32;
  static constexpr int NBUF = 3;                 // ring stages
  static constexpr int KBYTES = BN * D * 2;      // K tile
  static constexpr int SBYTES = BM * BN * 2;     // dS tile: 4 query tiles x 8 KB
  static constexpr int STAGE = KBYTES + SBYTES;
  static constexpr int SMEM = NBUF * STAGE;
  static constexpr int KCOPY = BN * (D / 8) / 64 / NW;   // K copies per wave per tile
  static constexpr int NCOPY = KCOPY + 4;                // + four 1 KB dS chunks
  static_assert((BN * (D / 8)) % (64 * NW) == 0, "even K copy split");
  static_assert(SMEM <= 160 * 1024, "fits the 160 KB of LDS");
  static_assert(NW * 32 * D * 2 <= SMEM, "epilogue staging fits");
};

size_t stored_ds_bytes(int64_t batch, int64_t heads, int64_t sq, int64_t sk) {
  return (size_t)batch * heads * ((sq + 63) / 64) * ((sk + 127) / 128) * 16384;
}

template <class E, int D, bool CAUSAL>
__global__ void __launch_bounds__(512) bwd_dq_ds_kernel(BwdArgs a) {
  using T = DqsTile<D>;
  using V4 = typename Ty<E>::v4;
  constexpr int RB = D * 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, grp = lane >> 4, j16 = lane & 15;

  // Block order as in the recomputing dQ kernel: consecutive blocks of one (unit, head) on
  // one XCD; dense causal pairs query tiles n-1-j and j in one workgroup (equal work).
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int n_qtiles = a.num_q_blocks;
  int qtile, qtile2 = -1, uh;
  if constexpr (CAUSAL) {
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
  const int Sq = a.Sq, Sk = a.Sk;
  const E* K = reinterpret_cast<const E*>(a.k) + (int64_t)unit * a.k_sb + (int64_t)g * a.k_sh;
  // dS chunks of this (unit, head): [64-row query tile][key block][16 chunks of 1 KB]
  const unsigned char* dsu = reinterpret_cast<const unsigned char*>(a.ds) +
                             ((int64_t)unit * a.H + head) * a.ds_nqt * a.num_k_blocks * 16384;
  const uint32_t lds0 = lds_addr(smem);

  // Per-lane LDS offsets (stage 0, slab 0). K^T: keys 4*half + (j16>>2) + 8*sec, d = db*32 +
  // 16*(grp&1) + 4*(j16&3). dS^T: this wave's query tile (wave>>1) and 16-row slab
  // 2*(wave&1) + (grp&1); key 4*half + (j16>>2) + 8*sec (XOR 4 on odd slabs); the 8-byte
  // piece holding query rows 4*(j16&3) .. +3 of the slab.
  const int clow = 2 * (grp & 1) + ((j16 & 3) >> 1);
  int tk[T::DB][2], ts[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 4 * half + (j16 >> 2) + 8 * sec;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
      tk[db][sec] = row * RB + 16 * ((4 * db + clow) ^ swz_f<D>(row)) + 8 * (j16 & 1);
    ts[sec] = T::KBYTES + (wave >> 1) * 8192 + (2 * (wave & 1) + (grp & 1)) * 1024 +
              ((row ^ (4 * (grp & 1))) * 32) + (j16 & 1) * 16 + ((j16 >> 1) & 1) * 8;
  }

  auto run_tile = [&](const int qtile) __attribute__((always_inline)) {
    const int qt0 = qtile * T::BM;
    if (qt0 >= Sq) return;
    const int kend = CAUSAL ? min(Sk, qt0 + T::BM) : Sk;
    const int ntiles = (kend + T::BN - 1) / T::BN;
    // This wave's share of a tile's dS copies: 4 KB of query tile qt0/64 + (wave>>1), key
    // groups 2*((k0 % 128) / 64) + (wave&1), all four slabs.
    const int qt64 = qt0 / 64 + (wave >> 1);
    auto load_tile = [&](int t, int stage) {
      const int k0 = t * T::BN;
      const int rows = min(T::BN, Sk - k0);
      const uint32_t st = lds0 + (uint32_t)(stage * T::STAGE);
      copy_tile_async<D, T::BN, T::NW>(st, copy_rsrc(K + (int64_t)k0 * a.k_ss,
                                                     (uint32_t)((rows - 1) * a.k_ss + D) * 2u),
                                       (int)a.k_ss, wave, lane);
      const int kb = k0 / 128;
      const bool written = qt64 < a.ds_nqt && (!CAUSAL || qt64 >= 2 * kb);
      const unsigned char* src = dsu + ((int64_t)qt64 * a.num_k_blocks + kb) * 16384 +
                                 (((k0 & 127) >> 6) * 2 + (wave & 1)) * 4096;
      const u32x4 rs = copy_rsrc(written ? src : reinterpret_cast<const unsigned char*>(a.ds),
                                 written ? 4096u : 0u);
      const uint32_t dst = st + (uint32_t)(T::KBYTES + (wave >> 1) * 8192 + (wave & 1) * 4096);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        copy16_to_lds_nt(rs, (uint32_t)(i * 1024 + lane * 16), sgpr(dst + (uint32_t)i * 1024u));
    };

    f32x16 dq[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db) dq[db] = f32x16{};

    if (ntiles > 0) load_tile(0, 0);
    if (ntiles > 1) {
      load_tile(1, 1);
      sync_copies<T::NCOPY>();   // tile 0 landed; tile 1 may be in flight
    } else {
      sync_copies<0>();
    }
    int stage = 0;
    for (int t = 0; t < ntiles; ++t) {
      const int nst = stage == 0 ? 2 : stage - 1;   // (t + 2) % 3
      if (t + 2 < ntiles) load_tile(t + 2, nst);
      const unsigned char* sb = smem + stage * T::STAGE;
      // Four 16-key slabs; the next slab's fragments are read while this slab's MFMAs run.
      V4 fk[2][T::DB][2], fs[2][2];
      auto fload = [&](int s, int slot) {
        const int ko = 16 * s * RB;
        const int so = (s >> 1) * 4096 + (s & 1) * 512;
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
          fs[slot][sec] = tr_at<V4>(sb + ts[sec], so);
#pragma unroll
          for (int db = 0; db < T::DB; ++db) fk[slot][db][sec] = tr_at<V4>(sb + tk[db][sec], ko);
        }
      };
      fload(0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s + 1 < 4) fload(s + 1, (s + 1) & 1);
        const auto bop = cat44(fs[s & 1][0], fs[s & 1][1]);
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
          dq[db] = mfma32(cat44(fk[s & 1][db][0], fk[s & 1][db][1]), bop, dq[db]);
      }
      // tile t + 1 has landed for every wave, and every wave is done with tile t's stage
      if (t + 2 < ntiles) sync_copies<T::NCOPY>();
      else sync_copies<0>();
      stage = stage == 2 ? 0 : stage + 1;
    }

    // Epilogue: dq = E(dQ * scale), contiguous [rows_q, H, D], through this wave's slice of
    // LDS (free after the last barrier); rows past Sq are not written.
    const int qw0 = qt0 + wave * 32;
    E* dqw = reinterpret_cast<E*>(a.dq) + (((int64_t)unit * Sq + qw0) * a.H + head) * D;
    wave_store_rows<D, E>(smem + wave * 32 * D * 2, dq, a.scale, dqw, (int64_t)a.H * D, Sq - qw0, lane);
  };

  run_tile(qtile);
  if (qtile2 >= 0) {
    __syncthreads();  // the first tile's epilogue is done with LDS
    run_tile(qtile2);
  }
}

template <class E, int D>
static hipError_t launch_dq_ds_d(const BwdArgs& a, bool causal, hipStream_t s) {
  const int nq = a.num_q_blocks;
  const int64_t per = causal ? (nq + 1) / 2 : nq;
  const int64_t nblk = (int64_t)a.num_units * a.H * per;
  if (nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)nblk), block(512);
  constexpr int smem = DqsTile<D>::SMEM;
  auto kfn = causal ? bwd_dq_ds_kernel<E, D, true> : bwd_dq_ds_kernel<E, D, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, grid, block, smem, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, int dtype, bool causal, hipStream_t s) {
  if (dtype == kDtypeF16) {
    if (head_dim == 64) return launch_dq_ds_d<f16, 64>(a, causal, s);
    return launch_dq_ds_d<f16, 128>(a, causal, s);
  }
  if (head_dim == 64) return launch_dq_ds_d<bf16, 64>(a, causal, s);
  return launch_dq_ds_d<bf16, 128>(a, causal, s);
}

}  // namespace exattn
