// bf16 attention forward (prefill) for gfx950.
//
// Algorithm: the FA2 loop of "Flash Attention on the 5090 in CUDA C++"
// ("Flash Attention 2 algorithm" pseudocode): a workgroup owns one block of
// query rows of one (batch, head), zeroes its O tile, walks the KV tiles in
// order, scores each tile, applies the online softmax, accumulates P.V and
// stores O once. The online softmax is the running-max / running-denominator /
// rescale recurrence of that page's "v1 -- basic version" bullets, kept in the
// unnormalised form with a single division at the end.
//
// Mapping to CDNA4 (our design; the page's sm120 kernel is prior art only):
//  * 512 threads = 8 waves, two waves per SIMD, 32 query rows per wave. Waves
//    0-3 and 4-7 form two groups in one of two layouts (template ROWG):
//    - row groups (ROWG): the workgroup owns 256 rows, each group 128 of
//      them, and both groups walk every KV tile, so each K/V tile copied into
//      LDS feeds 256 rows. Used when the grid of 256-row blocks still fills
//      the chip.
//    - KV-parity groups: both groups own the same 128 rows; group 0 takes
//      the even KV tiles, group 1 the odd ones, and the two partial results
//      are merged once at the end (same rescale, applied to the two halves).
//      Twice the row blocks, for grids that 256-row blocks would leave short
//      of the 256 CUs.
//    Each tile copy instruction costs the step a fixed amount (whatever it
//    moves, wherever it is issued), and the copies per MFMA are what the two
//    layouts differ in: row groups copy one K and one V tile per step for 512
//    MFMAs per SIMD pair, KV-parity groups two of each.
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs.
//    The wave's Q rows are the B operand and stay in registers for the whole
//    loop; every lane then holds the scores of ONE query row, so the row max
//    needs one cross-lane step and the rescale factor is a per-lane scalar.
//  * O is accumulated transposed, O^T += V^T P^T: the probabilities already
//    sit in B-operand layout (kappa() in fa_common.h), V^T comes from the
//    row-major LDS tile through transposing LDS reads.
//  * Tiles of 64 keys go straight from global memory into XOR-swizzled LDS
//    (global_load_lds, no register staging): four K slots and four V slots;
//    the copies for the next step are in flight while the current step
//    computes.
//  * Two-phase ping-pong between the two waves of each SIMD: in every phase
//    one wave issues only MFMAs (P.V of its previous tile, then the scores of
//    its next tile) while the other runs only the softmax VALU work, with a
//    barrier between phases. The matrix core of each SIMD is fed by one wave
//    (MFMAs and their LDS operand reads) while its VALU runs the other
//    wave's softmax; a single wave doing both stalls its in-order stream on
//    operand-read waits and copy issue.
//  * Guarded reference instead of a per-tile row max: exp2(s - m) is taken
//    against a row reference m (the true max of the row's first tile with a
//    visible key) that only has to keep the tile's row sum at or below 2^64
//    (checked on the row sum the softmax computes anyway); O and l always
//    carry the same factor, so the result is the same exact attention. The
//    row max, the new reference and the O rescale run only on a row's first
//    tile and on the rare tiles that fail the check.
//  * Causal: tiles past the workgroup's last visible key are never loaded; a
//    wave skips the math of tiles its rows cannot see; only tiles that cross
//    the diagonal or the ragged end are masked element-wise.
//  * Q and O move through LDS: each wave copies its 32 Q rows into LDS with
//    the tile copies and reads them back as B operands, and stages its O rows
//    there before storing them. Either way every global access instruction
//    covers whole rows; accessing the rows straight from the MFMA layout
//    would touch 32 rows with 8 or 16 bytes each per instruction, and with
//    eight waves doing so at once the CU's address unit holds up the
//    workgroup's first and last microseconds.
//  * Workgroups are renumbered so that the query blocks of one head run on one
//    XCD (its L2 then serves that head's K/V to all of them). Under the causal
//    mask a workgroup takes the pair of query blocks n - 1 - p and p, so that
//    all workgroups have the same work (a lone block p would see 2 (p + 1) key
//    tiles).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdThreads = 512;
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
constexpr int kSlots = 4;
// Largest row sum of one tile the softmax's common path accepts (see softmax).
constexpr float kSumHi = 18446744073709551616.0f;  // 2^64

template <int D>
struct FwdLayout {
  static constexpr int BN = kFwdBN;
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int V_BASE = kSlots * TILE_BYTES;  // V slots follow the K slots
  static constexpr int CH = D / 8;                    // 16-byte chunks per row
  static constexpr int ROWS_PER_KB = 64 / CH;         // rows one wave copy instruction covers
  static constexpr int BLOCKS = BN * CH / 64;         // wave copy instructions per tile
  static constexpr int NW = 4;                        // the waves of group 0 issue all copies
  static constexpr int COPIES = BLOCKS / NW;          // copy instructions per wave per tile
  static_assert(BLOCKS % NW == 0, "tile must split evenly over waves");
};

// Copy one K or V tile (BN rows x D) from global memory into an LDS slot with
// direct-to-LDS copies. Each wave instruction writes 1 KiB of LDS, lane l at
// byte 16 l; the swizzle is applied on the source side (`goff` holds, per copy
// instruction, the byte offset of the global chunk whose swizzled position is
// the lane's LDS position). A ragged last tile fetches row nvalid-1 in place
// of the missing rows (finite data whose scores are masked and whose
// probabilities are zero).
template <int D>
__device__ __forceinline__ void tile_to_lds(uint32_t slot_lds, const uint16_t* src, int nvalid,
                                            const uint32_t (&goff)[FwdLayout<D>::COPIES], int wave, int lane) {
  using L = FwdLayout<D>;
  if (nvalid >= L::BN) {
#pragma unroll
    for (int i = 0; i < L::COPIES; ++i) dma16_sbase(src, goff[i], slot_lds + (wave + i * L::NW) * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < L::COPIES; ++i) {
      const int blk = wave + i * L::NW;
      const int row = blk * L::ROWS_PER_KB + lane / L::CH;
      const int srow = row < nvalid ? row : nvalid - 1;
      const uint32_t off = (uint32_t)(srow * D + swz<D>(row, lane % L::CH) * 8) * 2u;
      dma16_sbase(src, off, slot_lds + blk * 1024);
    }
  }
}

// Stores of one wave's 32 rows of O through a wave-private LDS area. The
// O^T accumulator gives lane l row l % 32 and, per (d block db, group i4),
// the four columns 32 db + 8 i4 + 4 (l / 32) .. +3: a direct store would
// write 8 bytes into each of 32 rows per instruction. Written to LDS in that
// layout and read back row-major, every 16-byte-per-lane store covers whole
// rows (4 rows at d = 128, 8 at d = 64), so the CU's address unit handles a
// quarter of the pieces. Rows are padded by 16 bytes: the 8-byte writes of
// one instruction then fall on at most two lanes per bank, the 16-byte reads
// on distinct banks.
template <int D>
struct OStage {
  static constexpr int RS = 2 * D + 16;   // padded row stride in bytes
  static constexpr int BYTES = 32 * RS;   // one wave's area
  static constexpr int LPR = 2 * D / 16;  // lanes per row of the read-back
  static constexpr int RPS = 64 / LPR;    // rows per store instruction
};

// Column group (db, i4) of this lane's row into the staging area.
template <int D>
__device__ __forceinline__ void stage_o_cols(char* stage, int db, int i4, u32x2 w, int lane) {
  *reinterpret_cast<u32x2*>(stage + (lane & 31) * OStage<D>::RS + (db * 32 + i4 * 8 + (lane >> 5) * 4) * 2) = w;
}

// The staged rows to global memory, whole rows per instruction (with the
// non-temporal hint: O is written once and not read here, so it need not
// displace the K/V tiles the other workgroups still stream through L2); rows
// at or past `nvalid` are not written.
template <int D>
__device__ __forceinline__ void store_o_staged(const char* stage, uint16_t* o_row0, int nvalid, int lane) {
  using S = OStage<D>;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < 32 / S::RPS; ++j) {
    const int r = j * S::RPS + lane / S::LPR;
    const int c = (lane % S::LPR) * 16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * S::RS + c);
    if (r < nvalid) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(o_row0) + (size_t)r * 2 * D + c));
  }
}

// PAIRED (causal only): each workgroup takes query blocks n_qt - 1 - p and p of
// one head, one after the other, so that every workgroup has the same number
// of visible key tiles ((BM / 64) (n_qt + 1) per pair, instead of
// (BM / 64) (qt + 1) for block qt alone).
template <int D, bool PAIRED, bool ROWG>
__global__ __launch_bounds__(kFwdThreads) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float sl2, int causal,
    int n_qt, int n_wg) {
  using L = FwdLayout<D>;
  constexpr int BN = kFwdBN;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROWB = D * 2;  // bytes per tile row
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kSlots * BN * D];
  const char* lds_c = reinterpret_cast<const char*>(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, rw = wave & 3;
  const int hl = lane >> 5;  // half of the wave

  int wg = blockIdx.x;
  if ((n_wg & 7) == 0) wg = (wg & 7) * (n_wg >> 3) + (wg >> 3);

  // One query block: everything from here to the store of O and LSE.
  auto item = [&](const int bh, const int qt) __attribute__((always_inline)) {
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const uint16_t* Qh = Q + (size_t)bh * Nq * D;
  const uint16_t* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const uint16_t* Vh = V + (size_t)(b * Hkv + g) * Nk * D;

  constexpr int BM = ROWG ? 2 * kFwdBM : kFwdBM;
  // Row groups: wave rw of group g holds 32-row block 2 rw + g (the two waves
  // of a SIMD hold adjacent blocks); KV-parity groups: both hold block rw.
  const int qw0 = qt * BM + (ROWG ? 2 * rw + grp : rw) * 32;
  const int qrow = qw0 + (lane & 31);
  const int diag = Nk - Nq;  // key j visible to row i iff j <= i + diag

  bf16x8 qf[KS];
  // Loop-invariant per-lane LDS byte offsets (relative to `lds`); the slot
  // and the tile's row block are immediates.
  uint32_t koff[KS];
  {
    const int row = kappa(lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = row * ROWB + swz<D>(row, 2 * s + hl) * 16;
  }
  uint32_t voff[DB][2];
  {
    const int w = lane & 15, e = w >> 2, j = w & 3, q16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = hl * 8 + e + 4 * r;
        const int ch = db * 4 + q16 * 2 + (j >> 1);
        voff[db][r] = L::V_BASE + row * ROWB + swz<D>(row, ch) * 16 + (j & 1) * 8;
      }
  }
  uint32_t goff[L::COPIES];
#pragma unroll
  for (int i = 0; i < L::COPIES; ++i) {
    const int row = (rw + i * L::NW) * L::ROWS_PER_KB + lane / L::CH;
    goff[i] = (uint32_t)(row * D + swz<D>(row, lane % L::CH) * 8) * 2u;
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  // Q rows of this wave go through a wave-private LDS area (K slots 2-3 for
  // group 0, V slots 2-3 for group 1, which no copy fills before the first
  // barrier of the loop), laid out as the first 32 rows of a K tile whose
  // row r holds Q row kappa(r): each copy instruction fetches whole rows, and
  // lane l then reads Q row l % 32 through the K operand offsets. Rows past
  // Nq repeat row Nq - 1 (finite data whose results are not stored). The
  // paired KV-parity layout loads Q straight into registers instead: its
  // two items' code then fits 256 registers without spilling.
  constexpr bool kQViaLds = ROWG || !PAIRED;
  constexpr int QCOPIES = 32 * ROWB / 1024;
  const uint32_t qstage = (grp == 0 ? 2 * L::TILE_BYTES : L::V_BASE + 2 * L::TILE_BYTES) + rw * 32 * ROWB;
  if constexpr (kQViaLds) {
#pragma unroll
    for (int i = 0; i < QCOPIES; ++i) {
      const int row = i * L::ROWS_PER_KB + lane / L::CH;
      const int qr = qw0 + kappa(row);
      const int grow = qr < Nq ? qr : Nq - 1;
      dma16_sbase_nt(Qh, (uint32_t)(grow * D + swz<D>(row, lane % L::CH) * 8) * 2u, lds0 + qstage + i * 1024);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = qrow < Nq ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + s * 16 + hl * 8) : bf16x8{};
    }
  }

  int kv_end = Nk;
  if (causal) {
    const long last = (long)qt * BM + BM - 1 + diag;
    kv_end = last < 0 ? 0 : (int)(last + 1 < (long)Nk ? last + 1 : Nk);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;
  // Tiles this wave's rows can see (visibility only shrinks with the tile index).
  int n_vis = n_tiles;
  if (causal) {
    const long lastw = (long)qw0 + 31 + diag;
    const long nv = lastw < 0 ? 0 : lastw / BN + 1;
    n_vis = nv < n_tiles ? (int)nv : n_tiles;
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = 0.f, l_run = 0.f;  // row reference (log2 units) and row sum

  auto load_k = [&](int t) __attribute__((always_inline)) {
    tile_to_lds<D>(lds0 + (t % kSlots) * L::TILE_BYTES, Kh + (size_t)t * BN * D, Nk - t * BN, goff, rw, lane);
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    tile_to_lds<D>(lds0 + L::V_BASE + (t % kSlots) * L::TILE_BYTES, Vh + (size_t)t * BN * D, Nk - t * BN, goff,
                   rw, lane);
  };

  // Scores S^T = K Q^T of one tile (two 32-key blocks) from K slot offset KB.
  auto score = [&](f32x16(&sc)[2], auto kb_c) __attribute__((always_inline)) {
    constexpr int KB = decltype(kb_c)::value;
    sc[0] = f32x16{};
    sc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(lds_c + koff[s] + KB);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(lds_c + koff[s] + KB + 32 * ROWB);
      sc[0] = mfma32(a0, qf[s], sc[0]);
      sc[1] = mfma32(a1, qf[s], sc[1]);
    }
    // Keep the K-operand reads KS ahead of the MFMAs that consume them.
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
  };

  // Online softmax of tile t's scores: mask, exp2 against the row's reference
  // m, fp32 row sums, bf16 probabilities. The reference need not be the
  // running max: any m at or below it that keeps every exp2(s - m) of the
  // tile at or below 2^64 gives the same exact result (O and l always carry
  // the same factor), with the same relative precision, and no fp32 or bf16
  // overflow. So the common path does not compute the row max at all; it
  // checks the tile's row sum instead. The rare path (row max, new reference,
  // rescale of O and l, exponentials again) runs on a row's first tile with a
  // visible key, which sets the reference to that tile's true max (the
  // largest probability of a row whose keys all lie in one tile is then
  // exactly 1), and when the scores jump by tens of binary orders. The row sum l_run
  // holds the total of both halves of the row (lanes l and l ^ 32) in both
  // lanes, so both halves always take the same decisions.
  auto softmax = [&](f32x16(&sc)[2], bf16x8(&p)[2][2], int t) __attribute__((always_inline)) {
    const int kv0 = t * BN;
    const bool need_mask = (kv0 + BN > Nk) || (causal && kv0 + BN - 1 > qw0 + diag);
    if (need_mask) {
      // Key kv0 + c + 8 hl (c the register's offset, score_key) is visible
      // iff it is at most L = min(last key, the row's causal limit): one
      // per-lane bound, then a compare with a constant per score.
      const int L = causal && qrow + diag < Nk - 1 ? qrow + diag : Nk - 1;
      const int t = L - kv0 - 8 * hl;
      // Each 32-key block is classified for the whole wave first (keys
      // 32 mb + 0..23 in this lane's registers): on the causal diagonal one
      // of the two is usually all visible or all masked, and only a mixed
      // block needs the compare per score.
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (__all(mb * 32 + 23 <= t)) continue;
        if (__all(mb * 32 > t)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[mb][i] = kNegInf;
          continue;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = score_key(mb * 32, i, 0);
          if (c > t) sc[mb][i] = kNegInf;
        }
      }
    }
    // Probabilities against the current reference; returns the tile's row sum.
    auto exps = [&]() __attribute__((always_inline)) {
      const float neg_m = -m_run;
      // Four partial row sums, each started from its first term (an add to
      // 0.0 is not folded away: it would turn -0 into +0).
      float rs[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(__builtin_fmaf(sc[mb][i], sl2, neg_m));
          rs[i & 3] = mb == 0 && i < 4 ? e : rs[i & 3] + e;
          p[mb][i >> 3][i & 7] = (__bf16)e;
        }
      return sum_with_lane_xor32((rs[0] + rs[1]) + (rs[2] + rs[3]));
    };
    float tot = exps();
    if (__any(!(tot <= kSumHi) || l_run == 0.f)) {
      // Row max as a tree of 3-input maxima.
      float mt[11];
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        const int i0 = 3 * j, i1 = 3 * j + 1, i2 = 3 * j + 2;
        mt[j] = vmax(vmax(sc[i0 >> 4][i0 & 15], sc[i1 >> 4][i1 & 15]), sc[i2 >> 4][i2 & 15]);
      }
      mt[10] = vmax(sc[1][14], sc[1][15]);
      const float u0 = vmax(vmax(mt[0], mt[1]), mt[2]), u1 = vmax(vmax(mt[3], mt[4]), mt[5]);
      const float u2 = vmax(vmax(mt[6], mt[7]), mt[8]), u3 = vmax(mt[9], mt[10]);
      const float mx = max_with_lane_xor32(vmax(vmax(u0, u1), vmax(u2, u3))) * sl2;
      // New reference: the running max, or this tile's max while the row has
      // accumulated nothing yet (l_run is then exactly 0, and so is O). A row
      // with no visible key yet keeps its reference.
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
  };

  // O^T += V^T P^T from V slot offset VB.
  auto pv = [&](const bf16x8(&p)[2][2], auto vb_c) __attribute__((always_inline)) {
    constexpr int VB = decltype(vb_c)::value;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int kb = (mb * 32 + hf * 16) * ROWB;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_c + voff[db][0] + VB + kb));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_c + voff[db][1] + VB + kb));
          o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), p[mb][hf], o[db]);
        }
  };

  // Prologue: K tiles 0 and 1, in flight together with the Q loads. The Q
  // registers are consumed right after the common wait, so that the
  // compiler's own wait for them (which would also wait for every tile copy
  // in flight) is placed here and not inside the loop.
  if constexpr (ROWG) {
    if (n_tiles > 0) {
      if (grp == 0) load_k(0); else load_v(0);
    }
  } else if (grp == 1) {
    if (n_tiles > 0) load_k(0);
    if (n_tiles > 1) load_k(1);
  }
  wait_vmcnt0();
  if constexpr (kQViaLds) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(lds_c + qstage + koff[s]);
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qf[s]));
  __syncthreads();

  // Two-phase ping-pong. The two waves of a SIMD belong to different groups;
  // in each phase one of them issues only MFMAs (and their LDS operand
  // reads) while the other runs only VALU work (the softmax), and a barrier
  // separates the phases:
  //   step s   phase A                           | phase B
  //   group 0: P.V 2s-2, scores 2s                 | copy K 2s+3, V 2s+1; softmax 2s
  //   group 1: copy K 2s+2, V 2s; softmax 2s-1     | P.V 2s-1, scores 2s+1
  // Each group issues its copies at the start of its VALU phase (as a burst:
  // spreading them through the softmax or moving some into the MFMA phase
  // gains nothing) and waits for them
  // one phase before the other group reads them: group 1 at the end of the
  // step, group 0 before the next mid-step barrier. Scores and probabilities
  // stay in registers across the barriers. Tile t lives in K slot t % 4 and V
  // slot t % 4; step s reads K 2s, 2s+1 and V 2s-2, 2s-1, and every slot is
  // refilled one step after its last use.
  f32x16 sc[2];
  bf16x8 p[2][2];
  auto step_body = [&](auto grp_c, auto par_c, int step) __attribute__((always_inline)) {
    constexpr int GRP = decltype(grp_c)::value;
    constexpr int PAR = decltype(par_c)::value;  // step parity
    const int t0 = 2 * step;
    if constexpr (GRP == 0) {
      if (step > 0 && t0 - 2 < n_vis) pv(p, std::integral_constant<int, 2 * (1 - PAR) * L::TILE_BYTES>{});
      if (t0 < n_vis) score(sc, std::integral_constant<int, 2 * PAR * L::TILE_BYTES>{});
      wait_vmcnt0();
      __syncthreads();
      if (t0 + 3 < n_tiles) load_k(t0 + 3);
      if (t0 + 1 < n_tiles) load_v(t0 + 1);
      if (t0 < n_vis) softmax(sc, p, t0);
      __syncthreads();
    } else {
      if (t0 + 2 < n_tiles) load_k(t0 + 2);
      if (t0 < n_tiles) load_v(t0);
      const bool prev = step > 0 && t0 - 1 < n_vis;
      if (prev) softmax(sc, p, t0 - 1);
      __syncthreads();
      if (prev) pv(p, std::integral_constant<int, (2 * (1 - PAR) + 1) * L::TILE_BYTES>{});
      if (t0 + 1 < n_vis) score(sc, std::integral_constant<int, (2 * PAR + 1) * L::TILE_BYTES>{});
      wait_vmcnt0();
      __syncthreads();
    }
  };

  // Each group runs its own copy of the loop; both execute the same number of
  // steps (the last one finishes P.V of the last tiles) and so the same
  // barriers. Group 0's copies of the last step are waited for below.
  const int last_step = (n_tiles + 1) / 2;
  auto run = [&](auto grp_c) __attribute__((always_inline)) {
    for (int step = 0; step <= last_step; step += 2) {
      step_body(grp_c, std::integral_constant<int, 0>{}, step);
      if (step + 1 > last_step) break;
      step_body(grp_c, std::integral_constant<int, 1>{}, step + 1);
    }
  };
  // Row groups: both groups walk every tile, group 1 one phase behind group 0
  // (each group on its own rows, so the softmax of one and the MFMAs of the
  // other still alternate on every SIMD).
  //   step s   phase A                        | phase B
  //   group 0: P.V s-1, scores s               | copy V s+1; softmax s
  //   group 1: copy K s+1; softmax s-1         | P.V s-1, scores s
  // K s and V s live in slot s % 4. Group 1 waits for K s+1 at the end of
  // step s, group 0 for V s+1 at the end of phase A of step s+1; each slot
  // is refilled three steps after its last read.
  auto step_rows = [&](auto grp_c, auto s4_c, int s) __attribute__((always_inline)) {
    constexpr int GRP = decltype(grp_c)::value;
    constexpr int S4 = decltype(s4_c)::value;
    constexpr int KB = S4 * L::TILE_BYTES;
    constexpr int VB = ((S4 + 3) % 4) * L::TILE_BYTES;
    if constexpr (GRP == 0) {
      if (s > 0 && s - 1 < n_vis) pv(p, std::integral_constant<int, VB>{});
      if (s < n_vis) score(sc, std::integral_constant<int, KB>{});
      wait_vmcnt0();
      __syncthreads();
      if (s + 1 < n_tiles) load_v(s + 1);
      if (s < n_vis) softmax(sc, p, s);
      __syncthreads();
    } else {
      if (s + 1 < n_tiles) load_k(s + 1);
      const bool prev = s > 0 && s - 1 < n_vis;
      if (prev) softmax(sc, p, s - 1);
      __syncthreads();
      if (prev) pv(p, std::integral_constant<int, VB>{});
      if (s < n_vis) score(sc, std::integral_constant<int, KB>{});
      wait_vmcnt0();
      __syncthreads();
    }
  };
  auto run_rows = [&](auto grp_c) __attribute__((always_inline)) {
    for (int s = 0; s <= n_tiles; s += 4) {
      step_rows(grp_c, std::integral_constant<int, 0>{}, s);
      if (s + 1 > n_tiles) break;
      step_rows(grp_c, std::integral_constant<int, 1>{}, s + 1);
      if (s + 2 > n_tiles) break;
      step_rows(grp_c, std::integral_constant<int, 2>{}, s + 2);
      if (s + 3 > n_tiles) break;
      step_rows(grp_c, std::integral_constant<int, 3>{}, s + 3);
    }
  };
  if constexpr (ROWG) {
    if (grp == 0) {
      run_rows(std::integral_constant<int, 0>{});
    } else {
      run_rows(std::integral_constant<int, 1>{});
    }
    wait_vmcnt0();
    // Each wave holds whole rows: normalise and store. After the loop's last
    // barrier no wave reads the tile slots any more, so each wave stages its
    // rows in its own part of them.
    {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      char* stage = reinterpret_cast<char*>(lds) + wave * OStage<D>::BYTES;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][i4 * 4] * inv, o[db][i4 * 4 + 1] * inv);
          w[1] = pack_bf16x2(o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv);
          stage_o_cols<D>(stage, db, i4, w, lane);
        }
      store_o_staged<D>(stage, O + ((size_t)bh * Nq + qw0) * D, Nq - qw0, lane);
      if (lane < 32 && qrow < Nq)
        LSE[(size_t)bh * Nq + qrow] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
    }
    return;
  }
  if (grp == 0) {
    run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }
  wait_vmcnt0();
  __syncthreads();

  // Merge the two groups (same rows, disjoint key sets) and write out. The
  // O exchange holds each lane's accumulator registers 4 at a time, so that
  // every LDS access moves 16 bytes per lane (conflict-free: consecutive
  // lanes, consecutive 16-byte chunks).
  f32x4* xo = reinterpret_cast<f32x4*>(lds);                     // [4 rw][DB][4 i4][64] fp32 x4
  float* xm = reinterpret_cast<float*>(lds) + 4 * DB * 16 * 64;  // [4 rw][64] m, then [4 rw][64] l
  constexpr int kMergeBytes = (4 * DB * 16 * 64 + 2 * 4 * 64) * 4;
  static_assert(kMergeBytes + 4 * OStage<D>::BYTES <= (int)sizeof(lds), "merge and staging exceed LDS");
  static_assert(8 * OStage<D>::BYTES <= (int)sizeof(lds), "row-group staging exceeds LDS");
  const float l_tot = l_run;  // already the total of both lane halves
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        xo[((rw * DB + db) * 4 + i4) * 64 + lane] =
            f32x4{o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
    xm[rw * 64 + lane] = m_run;
    xm[256 + rw * 64 + lane] = l_tot;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = xm[rw * 64 + lane];
    const float l1 = xm[256 + rw * 64 + lane];
    const float M = fmaxf(m_run, m1);
    const float a0 = M == kNegInf ? 0.f : fast_exp2(m_run - M);
    const float a1 = M == kNegInf ? 0.f : fast_exp2(m1 - M);
    const float lsum = l_tot * a0 + l1 * a1;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float c0 = a0 * inv, c1 = a1 * inv;
    // Staging areas follow the exchange area (group 1 no longer reads LDS).
    char* stage = reinterpret_cast<char*>(lds) + kMergeBytes + rw * OStage<D>::BYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 x = xo[((rw * DB + db) * 4 + i4) * 64 + lane];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = o[db][i4 * 4 + j] * c0 + x[j] * c1;
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        stage_o_cols<D>(stage, db, i4, w, lane);
      }
    store_o_staged<D>(stage, O + ((size_t)bh * Nq + qw0) * D, Nq - qw0, lane);
    if (lane < 32 && qrow < Nq) LSE[(size_t)bh * Nq + qrow] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
  }
  };

  if constexpr (!PAIRED) {
    const int bh = wg / n_qt;
    const int qt = wg - bh * n_qt;
    // Under the causal mask the longest query blocks go first.
    item(bh, causal ? n_qt - 1 - qt : qt);
  } else {
    const int n_pairs = (n_qt + 1) / 2;
    const int bh = wg / n_pairs;
    const int p = wg - bh * n_pairs;
    item(bh, n_qt - 1 - p);
    if (p != n_qt - 1 - p) {
      // The merge area and the tile slots of the first block are reused.
      __syncthreads();
      item(bh, p);
    }
  }
}

// Row groups are used when the grid of 256-row blocks has at least this many
// workgroups (one per CU).
constexpr long kRowGroupsMinWg = 256;

template <int D, bool PAIRED, bool ROWG>
void launch_one(const FwdArgs& a, const FwdPlan& pl) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, PAIRED, ROWG>), dim3((unsigned)pl.n_wg), dim3(kFwdThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, a.causal, pl.n_qt,
                     (int)pl.n_wg);
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdArgs& a) {
  const FwdPlan pl = plan_fwd_bf16(a.B, a.Hq, a.Nq, a.causal);
  if (pl.n_wg == 0) return hipSuccess;
  switch (pl.layout) {
    case kLayoutRows: launch_one<D, false, true>(a, pl); break;
    case kLayoutRowsPaired: launch_one<D, true, true>(a, pl); break;
    case kLayoutKvParityPaired: launch_one<D, true, false>(a, pl); break;
    default: launch_one<D, false, false>(a, pl); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  return a.d == 128 ? launch_fwd_bf16_d<128>(a) : launch_fwd_bf16_d<64>(a);
}

FwdPlan plan_fwd_bf16(int B, int Hq, int Nq, int causal) {
  const int n_qt2 = (Nq + 2 * kFwdBM - 1) / (2 * kFwdBM);
  const bool paired2 = causal && n_qt2 >= 2;
  const long n_wg2 = (long)B * Hq * (paired2 ? (n_qt2 + 1) / 2 : n_qt2);
  if (n_wg2 >= kRowGroupsMinWg) return {paired2 ? kLayoutRowsPaired : kLayoutRows, n_qt2, n_wg2};
  const int n_qt = (Nq + kFwdBM - 1) / kFwdBM;
  if (causal && n_qt >= 2) return {kLayoutKvParityPaired, n_qt, (long)B * Hq * ((n_qt + 1) / 2)};
  return {kLayoutKvParity, n_qt, (long)B * Hq * n_qt};
}

long fwd_bf16_grid(int B, int Hq, int Nq) { return (long)B * Hq * ((Nq + kFwdBM - 1) / kFwdBM); }

}  // namespace fa
