// bf16 attention forward (prefill) for head sizes 192 and 256 on gfx950.
//
// Same algorithm as fa_fwd.hip (the FA2 loop of "Flash Attention on the 5090
// in CUDA C++", "Flash Attention 2 algorithm" pseudocode, with the online
// softmax of its "v1 -- basic version" bullets in unnormalised form and the
// guarded exponent reference). Head sizes above 128 are that page's "What
// next" item: the page's note that head_dim 128 fits in registers no longer
// holds, so the work split changes.
//
// Mapping to CDNA4 for d = 192, 256:
//  * A workgroup owns 128 query rows, 32 per wave. Q stays in registers as
//    the B operand of S^T = K Q^T (d / 4 VGPRs), O^T is accumulated in d / 2
//    VGPRs, so a wave has at most 256 registers and a SIMD runs two waves,
//    whose MFMA and VALU work overlap without a fixed phase order. The two
//    waves come from one of two layouts (template NG):
//    - NG = 2: 8 waves; waves 0-3 (group 0) and 4-7 (group 1) hold the same
//      rows and take the even and the odd 32-key tiles, merged through LDS at
//      the end; one workgroup per CU. Used when the grid has fewer than two
//      workgroups per CU (the pages' shape: 256).
//    - NG = 1: 4 waves walking every tile; two workgroups per CU, which also
//      hide each other's prologue and epilogue. Used for grids of at least
//      512 workgroups (measured at d = 256: 1047 vs 925 TFLOP/s at B4 H16
//      2048^2, while NG = 2 gives 1058 vs 757 at the pages' shape).
//  * Each group double-buffers its own K and V tiles (32 rows x 2 d bytes).
//    Per tile: scores in d / 16 MFMAs (32x32x16 bf16), the online softmax on
//    16 scores per lane, P.V in d / 16 MFMAs; the group's next tile is copied
//    meanwhile (global -> LDS), one workgroup barrier per step.
//  * Operand layouts are those of the d = 128 kernel: kappa() row order of
//    the K operand puts P straight into the B-operand layout of O^T += V^T P^T;
//    V^T comes from transposing LDS reads. The 16-byte chunks of a row are
//    XOR-swizzled so that both the K reads (16 rows at one chunk per pass) and
//    the transposing V reads (4 rows x 4 chunks per pass) hit distinct banks:
//    512-byte rows (d = 256) start on bank 0 and take a bijection of the row's
//    low 4 bits on chunk bits 0..3; 384-byte rows (d = 192, 24 chunks) start
//    on bank 0 or 32 (by row parity) and take, within each group of 8
//    chunks, an XOR with a row function that is a bijection over the 8 even
//    and over the 8 odd rows of a 16-row block whose bit 2 differs between
//    rows r and r + 2 of a 4-row group.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int k2WavesPerGroup = 4;
constexpr int k2BM = 128;
constexpr int k2BN = 32;
template <int D, int NG>
struct WideLayout {
  static constexpr int kRowB = D * 2;                        // bytes per row
  static constexpr int kTile = k2BN * kRowB;                 // 12 or 16 KiB
  static constexpr int kCopies = kTile / 1024 / k2WavesPerGroup;  // copy instructions per wave per tile
  static constexpr int kThreads = 64 * k2WavesPerGroup * NG;
  static constexpr int kVBase = 2 * NG * kTile;  // two K slots per group, then two V slots per group
  static constexpr int kMergeBytes = NG == 2 ? 4 * (D / 32) * 16 * 64 * 4 + 2048 : 0;
  // O staging (per wave, 32 rows x 64 columns at a time, rows padded by 16
  // bytes): after the exchange area with two groups, at the start of LDS with
  // one (the tile slots are free by then).
  static constexpr int kStageRow = 64 * 2 + 16;
  static constexpr int kStageBytes = 32 * kStageRow;
  static constexpr int kStageBase = kMergeBytes;
  static constexpr int kLdsTiles = 2 * kVBase + (NG == 2 ? 2048 : 0);
  static constexpr int kLdsMerge = kMergeBytes + (NG == 2 ? 4 : 4) * kStageBytes;
  static constexpr int kLds = kLdsMerge > kLdsTiles ? kLdsMerge : kLdsTiles;
  // Lane offsets kept per wave: at d = 256 copy instructions i and i + 2
  // cover rows 16 apart with the same swizzle, so two offsets serve all four
  // (the other two through a scalar base 16 rows further on).
  static constexpr int kGoff = D == 256 ? 2 : kCopies;
  static_assert(kTile % (1024 * k2WavesPerGroup) == 0, "tile must split evenly over the group's waves");
};
constexpr float k2SumHi = 18446744073709551616.0f;  // 2^64, as in the d = 128 kernel

// Stored chunk of logical chunk c in row `row` (an involution for fixed row).
template <int D>
__device__ __forceinline__ int swz_wide(int row, int c) {
  if constexpr (D == 256) {
    return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    const int f = ((row >> 2) & 3) | (((row >> 1) & 1) << 2);
    return c ^ f;  // f < 8: stays within c's group of 8 chunks
  }
}

// Copy one tile (32 rows x 2 d bytes): copy instruction blk writes LDS chunks
// 64 blk .. 64 blk + 63 of the tile (lane l: chunk 64 blk + l, i.e. row
// (64 blk + l) / (d / 8), stored chunk the remainder), fetched from the
// logical chunk whose swizzled position that is. Wave w issues blk = w + 4 i.
// Rows at or past nvalid fetch row nvalid - 1 (finite data, masked later).
template <int D>
__device__ __forceinline__ void tile_wide_to_lds(uint32_t slot_lds, const uint16_t* src, int nvalid,
                                                 const uint32_t (&goff)[WideLayout<D, 1>::kGoff], int wave,
                                                 int lane) {
  constexpr int CH = D / 8;
  constexpr int NC = WideLayout<D, 1>::kCopies;
  if (nvalid >= k2BN) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if constexpr (D == 256) {
        dma16_sbase(src + (i >> 1) * 16 * D, goff[i & 1], slot_lds + (wave + 4 * i) * 1024);
      } else {
        dma16_sbase(src, goff[i], slot_lds + (wave + 4 * i) * 1024);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int blk = wave + 4 * i;
      const int flat = blk * 64 + lane;
      const int row = flat / CH, ch = flat - row * CH;
      const int srow = row < nvalid ? row : nvalid - 1;
      dma16_sbase(src, (uint32_t)(srow * D * 2 + swz_wide<D>(row, ch) * 16), slot_lds + blk * 1024);
    }
  }
}

template <int D, int NG>
__global__ __launch_bounds__(64 * k2WavesPerGroup * NG, 2 / NG) void fwd_bf16_wide_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float sl2, int causal,
    int n_qt, int n_wg) {
  using L = WideLayout<D, NG>;
  constexpr int BN = k2BN;
  constexpr int KS = D / 16;  // k-steps of the score product
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int k2RowB = L::kRowB;
  constexpr int k2Tile = L::kTile;
  constexpr int k2VBase = L::kVBase;
  // Four tile slots per group; with two groups the merge then reuses them
  // and the 2 KiB after them.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[L::kLds / sizeof(uint16_t)];
  const char* lds_c = reinterpret_cast<const char*>(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NG == 2 ? wave >> 2 : 0, rw = wave & 3;
  const int hl = lane >> 5;

  int wg = blockIdx.x;
  if ((n_wg & 7) == 0) wg = (wg & 7) * (n_wg >> 3) + (wg >> 3);
  const int bh = wg / n_qt;
  int qt = wg - bh * n_qt;
  if (causal) qt = n_qt - 1 - qt;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const uint16_t* Qh = Q + (size_t)bh * Nq * D;
  const uint16_t* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const uint16_t* Vh = V + (size_t)(b * Hkv + g) * Nk * D;

  const int qw0 = qt * k2BM + rw * 32;
  const int qrow = qw0 + (lane & 31);
  const int diag = Nk - Nq;

  // Q rows as B operands: k-step s covers d = 16 s .. 16 s + 15.
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qrow < Nq ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + s * 16 + hl * 8) : bf16x8{};

  // K operand of k-step s: row kappa(lane % 32), chunk 2 s + hl, i.e. byte
  // krow + ((2 s) ^ kx) * 16 with kx = hl ^ (the row's swizzle); computed per
  // read (two VALU) to keep registers for Q and O.
  const uint32_t krow = kappa(lane & 31) * k2RowB + 2 * grp * k2Tile;  // + the group's slots
  const uint32_t kx = (uint32_t)swz_wide<D>(kappa(lane & 31), hl);
  // V^T operand (two transposing reads r = 0, 1 per MFMA): lane reads row
  // hl*8 + e + 4 r, chunk 4 db + 2 q16 + j/2, byte half j % 2, i.e. byte
  // vrow[r] + ((4 db) ^ vx[r]) * 16 with vx[r] = (2 q16 + j/2) ^ (the row's
  // swizzle); the 16-key half of the tile is an immediate.
  uint32_t vrow[2], vx[2];
  {
    const int w = lane & 15, e = w >> 2, j = w & 3, q16 = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = hl * 8 + e + 4 * r;
      vrow[r] = k2VBase + 2 * grp * k2Tile + row * k2RowB + (j & 1) * 8;
      vx[r] = (uint32_t)swz_wide<D>(row, q16 * 2 + (j >> 1));
    }
  }
  uint32_t goff[L::kGoff];
#pragma unroll
  for (int i = 0; i < L::kGoff; ++i) {
    const int flat = (rw + 4 * i) * 64 + lane;
    const int row = flat / (D / 8), ch = flat - row * (D / 8);
    goff[i] = (uint32_t)(row * k2RowB + swz_wide<D>(row, ch) * 16);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

  int kv_end = Nk;
  if (causal) {
    const long last = (long)qt * k2BM + k2BM - 1 + diag;
    kv_end = last < 0 ? 0 : (int)(last + 1 < (long)Nk ? last + 1 : Nk);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;
  int n_vis = n_tiles;
  if (causal) {
    const long lastw = (long)qw0 + 31 + diag;
    const long nv = lastw < 0 ? 0 : lastw / BN + 1;
    n_vis = nv < n_tiles ? (int)nv : n_tiles;
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = 0.f, l_run = 0.f;

  // Group g takes tiles g, g + NG, g + 2 NG, ...; its u-th tile
  // (t = NG u + g) lives in slot 2 g + u % 2 of the K and of the V slots.
  auto load = [&](int t, int slot) __attribute__((always_inline)) {
    tile_wide_to_lds<D>(lds0 + slot * k2Tile, Kh + (size_t)t * BN * D, Nk - t * BN, goff, rw, lane);
    tile_wide_to_lds<D>(lds0 + k2VBase + slot * k2Tile, Vh + (size_t)t * BN * D, Nk - t * BN, goff, rw, lane);
  };

  // One tile from the group's K/V slot PAR (the group's base is in krow and
  // vrow): scores, online softmax, P.V.
  auto tile = [&](int t, auto par_c) __attribute__((always_inline)) {
    constexpr uint32_t KB = decltype(par_c)::value * k2Tile;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_c + krow + (((uint32_t)(2 * s) ^ kx) << 4) + KB);
      sc = mfma32(a, qf[s], sc);
    }
    // K-operand reads four ahead of their MFMAs (bounded register use).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < KS - 4; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    const int kv0 = t * BN;
    if ((kv0 + BN > Nk) || (causal && kv0 + BN - 1 > qw0 + diag)) {
      // One per-lane bound, then a compare with a constant per score (see
      // the d = 128 kernel).
      const int L = causal && qrow + diag < Nk - 1 ? qrow + diag : Nk - 1;
      const int t = L - kv0 - 8 * hl;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (score_key(0, i, 0) > t) sc[i] = kNegInf;
    }
    bf16x8 p[2];
    auto exps = [&]() __attribute__((always_inline)) {
      const float neg_m = -m_run;
      float rs[4];  // each started from its first term (see the d = 128 kernel)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(sc[i], sl2, neg_m));
        rs[i & 3] = i < 4 ? e : rs[i & 3] + e;
        p[i >> 3][i & 7] = (__bf16)e;
      }
      return sum_with_lane_xor32((rs[0] + rs[1]) + (rs[2] + rs[3]));
    };
    float tot = exps();
    if (__any(!(tot <= k2SumHi) || l_run == 0.f)) {
      float mt[6];
#pragma unroll
      for (int j = 0; j < 5; ++j) mt[j] = vmax(vmax(sc[3 * j], sc[3 * j + 1]), sc[3 * j + 2]);
      mt[5] = sc[15];
      const float mx = max_with_lane_xor32(vmax(vmax(mt[0], mt[1]), vmax(vmax(mt[2], mt[3]), vmax(mt[4], mt[5])))) * sl2;
      float m_new = l_run == 0.f ? mx : vmax(m_run, mx);
      if (!(m_new > kNegInf)) m_new = m_run;
      const float alpha = l_run == 0.f ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
      tot = exps();
    }
    l_run += tot;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t base = KB + hf * 16 * k2RowB;
        const uint32_t a0 = vrow[0] + (((uint32_t)(4 * db) ^ vx[0]) << 4) + base;
        const uint32_t a1 = vrow[1] + (((uint32_t)(4 * db) ^ vx[1]) << 4) + base;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_c + a0));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_c + a1));
        o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), p[hf], o[db]);
      }
    // V^T reads four MFMAs ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int s = 0; s < 2 * DB - 4; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  };

  if (grp < n_tiles) load(grp, 2 * grp);
  wait_vmcnt0();
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qf[s]));
  __syncthreads();
  // Step u: group g computes its tile t = NG u + g from slot 2 g + u % 2
  // while its next tile (t + NG) is copied into slot 2 g + (u + 1) % 2. That
  // slot held the group's tile t - NG, whose reads ended before the barrier
  // that closed step u - 1; the copy is waited for before the barrier that
  // closes step u. Both groups run the same number of steps (same barriers).
  const int n_steps = (n_tiles + NG - 1) / NG;
  auto step = [&](int u, auto par_c) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    const int t = NG * u + grp;
    if (t + NG < n_tiles) load(t + NG, 2 * grp + (1 - PAR));
    if (t < n_vis) tile(t, par_c);
    wait_vmcnt0();
    __syncthreads();
  };
  for (int u = 0; u < n_steps; u += 2) {
    step(u, std::integral_constant<int, 0>{});
    if (u + 1 >= n_steps) break;
    step(u + 1, std::integral_constant<int, 1>{});
  }

  // Merge the two groups (same rows, disjoint key sets) and write out. The
  // O exchange holds each lane's accumulator registers 4 at a time (16-byte,
  // conflict-free LDS accesses). O rows are stored through a wave-private
  // LDS staging area, 64 columns at a time: written in accumulator order,
  // read back row-major, so that each 16-byte-per-lane store covers 8 whole
  // 128-byte row pieces instead of 8 bytes of each of 32 rows.
  f32x4* xo = reinterpret_cast<f32x4*>(lds);                        // [4 rw][DB][4 i4][64] fp32 x4
  float* xm = reinterpret_cast<float*>(lds) + 4 * DB * 16 * 64;     // [4 rw][64] m, then [4 rw][64] l
  char* stage = reinterpret_cast<char*>(lds) + L::kStageBase + rw * L::kStageBytes;
  char* o_rows = reinterpret_cast<char*>(O + ((size_t)bh * Nq + qw0) * D);
  const int nvalid = Nq - qw0;
  // Columns 64 c .. 64 c + 63 (d blocks 2 c, 2 c + 1) of this wave's rows:
  // `val(db, i)` gives the final value of accumulator register i of block db.
  auto store_chunk = [&](int c, auto val) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int db = 2 * c + k;
        u32x2 w;
        w[0] = pack_bf16x2(val(db, i4 * 4), val(db, i4 * 4 + 1));
        w[1] = pack_bf16x2(val(db, i4 * 4 + 2), val(db, i4 * 4 + 3));
        *reinterpret_cast<u32x2*>(stage + (lane & 31) * L::kStageRow + (k * 32 + i4 * 8 + hl * 4) * 2) = w;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = j * 8 + (lane >> 3);
      const int cb = (lane & 7) * 16;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * L::kStageRow + cb);
      if (r < nvalid) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(o_rows + (size_t)r * 2 * D + c * 128 + cb));
    }
  };
  if (NG == 1) {
    // One group: each wave holds whole rows. The loop's last barrier has
    // passed, so the tile slots are free for staging.
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < DB / 2; ++c) store_chunk(c, [&](int db, int i) { return o[db][i] * inv; });
    if (lane < 32 && qrow < Nq) LSE[(size_t)bh * Nq + qrow] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
    return;
  }
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        xo[((rw * DB + db) * 4 + i4) * 64 + lane] =
            f32x4{o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
    xm[rw * 64 + lane] = m_run;
    xm[256 + rw * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = xm[rw * 64 + lane];
    const float l1 = xm[256 + rw * 64 + lane];
    const float M = fmaxf(m_run, m1);
    const float a0 = M == kNegInf ? 0.f : fast_exp2(m_run - M);
    const float a1 = M == kNegInf ? 0.f : fast_exp2(m1 - M);
    const float lsum = l_run * a0 + l1 * a1;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float c0 = a0 * inv, c1 = a1 * inv;
#pragma unroll
    for (int c = 0; c < DB / 2; ++c) {
      f32x4 x[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) x[k][i4] = xo[((rw * DB + 2 * c + k) * 4 + i4) * 64 + lane];
      store_chunk(c, [&](int db, int i) { return o[db][i] * c0 + x[db - 2 * c][i >> 2][i & 3] * c1; });
    }
    if (lane < 32 && qrow < Nq) LSE[(size_t)bh * Nq + qrow] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
  }
}

// Grids of at least this many workgroups use the one-group layout (two
// workgroups per CU on the 256 CUs).
constexpr long kWideOneGroupMinWg = 512;

template <int D>
hipError_t launch_wide_d(const FwdArgs& a) {
  const int n_qt = (a.Nq + k2BM - 1) / k2BM;
  const long n_wg = (long)a.B * a.Hq * n_qt;
  if (n_wg == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  if (n_wg >= kWideOneGroupMinWg) {
    hipLaunchKernelGGL((fwd_bf16_wide_kernel<D, 1>), dim3((unsigned)n_wg), dim3(WideLayout<D, 1>::kThreads), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.causal, n_qt, (int)n_wg);
  } else {
    hipLaunchKernelGGL((fwd_bf16_wide_kernel<D, 2>), dim3((unsigned)n_wg), dim3(WideLayout<D, 2>::kThreads), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.causal, n_qt, (int)n_wg);
  }
  return hipGetLastError();
}

}  // namespace

int fwd_wide_layout(int B, int Hq, int Nq) {
  const long n_wg = (long)B * Hq * ((Nq + k2BM - 1) / k2BM);
  return n_wg >= kWideOneGroupMinWg ? kLayoutWideOneGroup : kLayoutWideTwoGroups;
}

hipError_t launch_fwd_bf16_wide(const FwdArgs& a) {
  return a.d == 256 ? launch_wide_d<256>(a) : launch_wide_d<192>(a);
}

}  // namespace fa
