// fp8 (OCP E4M3) attention forward (prefill) for gfx950, head size 128.
//
// What it computes: the same exact attention as the bf16 forward, over inputs
// stored as E4M3 bytes with one fp32 descale factor per tensor (the value of
// a byte is its E4M3 value times the tensor's descale). The pages name 8-bit
// matrix instructions as the reason for writing the kernel by hand ("Flash
// Attention on the 5090 in CUDA C++": the goal stated at the top and "What
// next", MXFP8 MMA) and low-precision paths as FlashAttention-3's direction
// ("Flash Attention", aiunderstanding.org, FAQ); they fix no format, so the
// per-tensor-descale E4M3 reading is ours.
//
// Algorithm and work split are those of the bf16 forward (fa_fwd.hip): the
// FA2 loop of the 5090 page's "Flash Attention 2 algorithm" pseudocode with
// the online softmax of its "v1 -- basic version" bullets, 8 waves in two
// KV-parity groups, two-phase ping-pong (one wave of a SIMD on MFMAs while
// the other runs the softmax), direct global->LDS tile copies, Q and O moved
// through LDS by whole rows, a guarded exponent reference, causal tile
// skipping, XCD-aware workgroup order.
//
// What changes for 8-bit inputs:
//  * Both products use v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (twice
//    the bf16 rate): scores S^T = K Q^T in 4 MFMAs per 64-key tile (two
//    32-key blocks x two 64-wide halves of d), O^T += V^T P^T in 4 MFMAs (one
//    per 32-row block of d, contracting over all 64 keys of the tile).
//  * The MFMA pairs byte j of lane-half h of A with byte j of lane-half h of
//    B (checked on gfx950), so any key order works as long as V^T and P use
//    the same one. P byte j of lane-half h (score register j % 16 of key block
//    j / 16) is key (j/16)*32 + ((j%16)/4)*8 + 4h + j%4 of the tile; the V^T
//    operand gathers exactly these keys with ds_read_b64_tr_b8 (in each group
//    of 16 lanes, output lane i gets byte i % 8 of the 8 bytes addressed by
//    lanes 2e + i/8, e = 0..7: lanes 2e and 2e+1 name one key row, every
//    output lane one d column of 8 keys).
//  * Probabilities are exp2(s*sl2 - m) with the reference m kept kF8Off
//    below the row max of the row's first tile, so they are at most 2^kF8Off
//    there; a tile is accepted on the common path only while its row sum stays
//    at or below 448, the largest finite E4M3 value (the conversion does not
//    saturate), otherwise the row's reference is raised as in the bf16
//    kernel. The row sum l is taken from the fp32 probabilities before they
//    are rounded to E4M3 (round to nearest even) for P.V.
//  * The score scale folds in the Q and K descales; O is multiplied by the V
//    descale in the epilogue. LSE does not depend on the reference offset.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2;

constexpr int kF8Threads = 512;
constexpr int kF8BM = 128;       // query rows per workgroup
constexpr int kF8BN = 64;        // keys per tile
constexpr int kF8D = 128;        // head size (bytes per row)
constexpr int kF8Slots = 4;      // LDS slots per operand
constexpr int kF8Tile = kF8BN * kF8D;          // 8 KiB
constexpr int kF8VBase = kF8Slots * kF8Tile;   // V slots follow the K slots
constexpr int kF8Copies = 2;     // 1 KiB copy instructions per wave per tile (4 waves per group)
constexpr float kF8Off = 4.f;    // log2 of the largest probability after a reference update
constexpr float kF8SumHi = 448.f;
// LDS: 64 KiB of tiles; the final merge reuses it for 66 KiB, followed by
// group 0's O staging areas (4 x 32 rows of 256 + 16 bytes).
constexpr int kF8MergeBytes = 4 * 4 * 16 * 64 * 4 + 2 * 4 * 64 * 4;
constexpr int kF8OStageRow = 2 * kF8D + 16;
constexpr int kF8OStageBytes = 32 * kF8OStageRow;
constexpr int kF8Lds = kF8MergeBytes + 4 * kF8OStageBytes > 2 * kF8VBase ? kF8MergeBytes + 4 * kF8OStageBytes
                                                                         : 2 * kF8VBase;

// 16-byte-chunk XOR swizzle of a 128-byte row. Two rows share the 64 banks
// (odd rows on the upper 32), so the chunk is XORed with a bijection of row
// bits 1..3: (bit 2, bit 1, bit 3) as (bit 0, bit 1, bit 2) of the XOR.
//  * K operand reads (16 consecutive rows at one logical chunk per pass):
//    the bijection puts the 8 even and the 8 odd rows on 8 distinct chunks.
//  * Transposing V reads (one pass = 32 lanes: rows r..r+3 and r+8..r+11,
//    r = 4 hl, at chunks 2 db and 2 db + 1): bits 1 and 3 of the row select
//    the chunk pair, so the four even (and four odd) rows cover all eight
//    chunks. Both are conflict-free (SQ_LDS_BANK_CONFLICT = 0).
__device__ __forceinline__ int swz8(int row, int chunk) {
  return chunk ^ (((row >> 2) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2));
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // Operand formats 0/0: E4M3 for A and B; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Tile copy (64 rows x 128 bytes) into an LDS slot: copy instruction `blk`
// covers rows 8 blk .. 8 blk + 7, lane l's 16 bytes land at byte 16 l of it;
// the swizzle is applied on the source address. A ragged tile fetches row
// nvalid-1 in place of the missing rows (finite data, masked later).
__device__ __forceinline__ void tile8_to_lds(uint32_t slot_lds, const uint8_t* src, int nvalid,
                                             const uint32_t (&goff)[kF8Copies], int rw, int lane) {
  if (nvalid >= kF8BN) {
#pragma unroll
    for (int i = 0; i < kF8Copies; ++i) dma16_sbase(src, goff[i], slot_lds + (rw + 4 * i) * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kF8Copies; ++i) {
      const int blk = rw + 4 * i;
      const int row = blk * 8 + (lane >> 3);
      const int srow = row < nvalid ? row : nvalid - 1;
      dma16_sbase(src, (uint32_t)(srow * kF8D + swz8(row, lane & 7) * 16), slot_lds + blk * 1024);
    }
  }
}

__global__ __launch_bounds__(kF8Threads) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float sl2, float vds,
    int causal, int n_qt, int n_wg) {
  constexpr int BN = kF8BN, D = kF8D;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kF8Lds];
  const char* lds_c = reinterpret_cast<const char*>(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, rw = wave & 3;
  const int hl = lane >> 5;

  int wg = blockIdx.x;
  if ((n_wg & 7) == 0) wg = (wg & 7) * (n_wg >> 3) + (wg >> 3);
  const int bh = wg / n_qt;
  int qt = wg - bh * n_qt;
  if (causal) qt = n_qt - 1 - qt;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const uint8_t* Qh = Q + (size_t)bh * Nq * D;
  const uint8_t* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const uint8_t* Vh = V + (size_t)(b * Hkv + g) * Nk * D;

  const int qw0 = qt * kF8BM + rw * 32;
  const int qrow = qw0 + (lane & 31);
  const int diag = Nk - Nq;

  // Q rows as B operands: half dh of d, lane-half hl holds bytes 64 dh + 32 hl .. +31.
  // They are read from LDS below (see the prologue).
  i32x8 qf[2];

  // Loop-invariant LDS byte offsets. K operand (key row lane % 32 of a 32-key
  // block, chunks 4 dh + 2 hl + c); the block and slot are immediates.
  uint32_t koff[2][2];
  {
    const int row = lane & 31;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
      for (int c = 0; c < 2; ++c) koff[dh][c] = row * D + swz8(row, 4 * dh + 2 * hl + c) * 16;
  }
  // V^T operand: lane i of its 16-lane group names key row e = (i % 16) / 2
  // of the read (rows r..r+3, r+8..r+11 with r = 4 hl) and the 8-byte half
  // i % 2 of chunk 2 db + (lane / 16) % 2. Read t adds (t/2)*32 + (t%2)*16
  // rows, which leaves the swizzle unchanged.
  uint32_t voff[4];
  {
    const int i = lane & 15, e = i >> 1, hh = i & 1, G = (lane >> 4) & 1;
    const int row = (e >> 2) * 8 + hl * 4 + (e & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] = kF8VBase + row * D + swz8(row, 2 * db + G) * 16 + hh * 8;
  }
  uint32_t goff[kF8Copies];
#pragma unroll
  for (int i = 0; i < kF8Copies; ++i) {
    const int row = (rw + 4 * i) * 8 + (lane >> 3);
    goff[i] = (uint32_t)(row * D + swz8(row, lane & 7) * 16);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  // The wave's 32 Q rows are copied by whole rows into a wave-private area
  // laid out as the first 32 rows of a K tile (K slots 2-3 for group 0, V
  // slots 2-3 for group 1, which no copy fills before the loop's first
  // barrier) and read back through the K operand offsets. Rows past Nq
  // repeat row Nq - 1 (finite data whose results are not stored).
  const uint32_t qstage = (grp == 0 ? 2 * kF8Tile : kF8VBase + 2 * kF8Tile) + rw * 32 * D;
#pragma unroll
  for (int i = 0; i < 32 * D / 1024; ++i) {
    const int row = i * 8 + (lane >> 3);
    const int grow = qw0 + row < Nq ? qw0 + row : Nq - 1;
    dma16_sbase_nt(Qh, (uint32_t)(grow * D + swz8(row, lane & 7) * 16), lds0 + qstage + i * 1024);
  }

  int kv_end = Nk;
  if (causal) {
    const long last = (long)qt * kF8BM + kF8BM - 1 + diag;
    kv_end = last < 0 ? 0 : (int)(last + 1 < (long)Nk ? last + 1 : Nk);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;
  int n_vis = n_tiles;
  if (causal) {
    const long lastw = (long)qw0 + 31 + diag;
    const long nv = lastw < 0 ? 0 : lastw / BN + 1;
    n_vis = nv < n_tiles ? (int)nv : n_tiles;
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = 0.f, l_run = 0.f;

  auto load_k = [&](int t) __attribute__((always_inline)) {
    tile8_to_lds(lds0 + (t % kF8Slots) * kF8Tile, Kh + (size_t)t * BN * D, Nk - t * BN, goff, rw, lane);
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    tile8_to_lds(lds0 + kF8VBase + (t % kF8Slots) * kF8Tile, Vh + (size_t)t * BN * D, Nk - t * BN, goff, rw,
                 lane);
  };

  // Scores S^T = K Q^T of one tile from K slot offset KB: sc[mb] covers keys
  // 32 mb .. 32 mb + 31.
  auto score = [&](f32x16(&sc)[2], auto kb_c) __attribute__((always_inline)) {
    constexpr int KB = decltype(kb_c)::value;
    i32x8 a[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(lds_c + koff[dh][0] + KB + mb * 32 * D);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(lds_c + koff[dh][1] + KB + mb * 32 * D);
        a[mb][dh] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                          (int)hi[3]};
      }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sc[mb] = mfma_f8(a[mb][0], qf[0], f32x16{});
      sc[mb] = mfma_f8(a[mb][1], qf[1], sc[mb]);
    }
  };

  // Online softmax of tile t (see the bf16 kernel for the guarded reference;
  // here the reference sits kF8Off below the max and the bound is 448).
  auto softmax = [&](f32x16(&sc)[2], i32x8& pk, int t) __attribute__((always_inline)) {
    const int kv0 = t * BN;
    const bool need_mask = (kv0 + BN > Nk) || (causal && kv0 + BN - 1 > qw0 + diag);
    if (need_mask) {
      // Key kv0 + c + 4 hl is visible iff it is at most L = min(last key, the
      // row's causal limit): one per-lane bound, a compare with a constant
      // per score.
      const int L = causal && qrow + diag < Nk - 1 ? qrow + diag : Nk - 1;
      const int t = L - kv0 - 4 * hl;
      // Each 32-key block is classified for the whole wave first (keys
      // 32 mb + 0..27 in this lane's registers), as in the bf16 kernel.
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (__all(mb * 32 + 27 <= t)) continue;
        if (__all(mb * 32 > t)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[mb][i] = kNegInf;
          continue;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (mb * 32 + (i >> 2) * 8 + (i & 3) > t) sc[mb][i] = kNegInf;
      }
    }
    auto exps = [&]() __attribute__((always_inline)) {
      const float neg_m = -m_run;
      float rs[4];  // each started from its first term (see the bf16 kernel)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float e[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          e[c] = fast_exp2(__builtin_fmaf(sc[w >> 2][(w & 3) * 4 + c], sl2, neg_m));
          rs[c] = w == 0 ? e[c] : rs[c] + e[c];
        }
        // The first conversion writes bytes 0-1 and keeps bytes 2-3 of its
        // third operand, which the second then overwrites: passing the old
        // pk[w] (already consumed by the previous P.V) spares zeroing a
        // register per word.
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], pk[w], false);
        pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], v, true);
      }
      return sum_with_lane_xor32((rs[0] + rs[1]) + (rs[2] + rs[3]));
    };
    float tot = exps();
    if (__any(!(tot <= kF8SumHi) || l_run == 0.f)) {
      float mt[11];
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        const int i0 = 3 * j, i1 = 3 * j + 1, i2 = 3 * j + 2;
        mt[j] = vmax(vmax(sc[i0 >> 4][i0 & 15], sc[i1 >> 4][i1 & 15]), sc[i2 >> 4][i2 & 15]);
      }
      mt[10] = vmax(sc[1][14], sc[1][15]);
      const float u0 = vmax(vmax(mt[0], mt[1]), mt[2]), u1 = vmax(vmax(mt[3], mt[4]), mt[5]);
      const float u2 = vmax(vmax(mt[6], mt[7]), mt[8]), u3 = vmax(mt[9], mt[10]);
      const float mx = max_with_lane_xor32(vmax(vmax(u0, u1), vmax(u2, u3))) * sl2 - kF8Off;
      // New reference: kF8Off below the running max (this tile's max while
      // the row has accumulated nothing); a row with no visible key keeps it.
      float m_new = l_run == 0.f ? mx : vmax(m_run, mx);
      if (!(m_new > kNegInf)) m_new = m_run;
      const float alpha = l_run == 0.f ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m_run = m_new;
      tot = exps();
    }
    l_run += tot;
  };

  // O^T += V^T P^T from V slot offset VB.
  auto pv = [&](const i32x8& pk, auto vb_c) __attribute__((always_inline)) {
    constexpr int VB = decltype(vb_c)::value;
    i32x8 a[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2v r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(lds_c + voff[db] + VB + (t >> 1) * 32 * D + (t & 1) * 16 * D));
        a[db][2 * t] = r[0];
        a[db][2 * t + 1] = r[1];
      }
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_f8(a[db], pk, o[db]);
    // All sixteen operand reads first, then the four MFMAs as they arrive.
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  if (grp == 1) {
    if (n_tiles > 0) load_k(0);
    if (n_tiles > 1) load_k(1);
    if (n_tiles > 0) load_v(0);
  }
  wait_vmcnt0();
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lds_c + qstage + koff[dh][0]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lds_c + qstage + koff[dh][1]);
    qf[dh] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) asm volatile("" ::"v"(qf[dh]));
  __syncthreads();

  // Two-phase ping-pong, as in the bf16 kernel:
  //   step s   phase A                                | phase B
  //   group 0: P.V 2s-2, scores 2s; copy V 2s+1         | copy K 2s+3; softmax 2s
  //   group 1: copy K 2s+2; softmax 2s-1                | P.V 2s-1, scores 2s+1; copy V 2s+2
  // With 8-bit operands the MFMA phase (8 MFMAs per wave) is shorter than the
  // softmax phase, so the V copies are issued by the MFMA wave after its
  // MFMAs, one phase earlier than the K copies of the same tile step; each
  // MFMA phase then waits for every copy except the V copies it just issued
  // (those land a full step before P.V reads them). A V slot is rewritten only
  // after the P.V of the tile four back, which ran in an earlier phase.
  f32x16 sc[2];
  i32x8 pk = i32x8{};
  auto wait_all_but_v = [&](bool v_issued) __attribute__((always_inline)) {
    if (v_issued) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kF8Copies) : "memory");
    } else {
      wait_vmcnt0();
    }
  };
  auto step_body = [&](auto grp_c, auto par_c, int step) __attribute__((always_inline)) {
    constexpr int GRP = decltype(grp_c)::value;
    constexpr int PAR = decltype(par_c)::value;
    const int t0 = 2 * step;
    if constexpr (GRP == 0) {
      if (step > 0 && t0 - 2 < n_vis) pv(pk, std::integral_constant<int, 2 * (1 - PAR) * kF8Tile>{});
      if (t0 < n_vis) score(sc, std::integral_constant<int, 2 * PAR * kF8Tile>{});
      const bool v_issued = t0 + 1 < n_tiles;
      if (v_issued) load_v(t0 + 1);
      wait_all_but_v(v_issued);
      __syncthreads();
      if (t0 + 3 < n_tiles) load_k(t0 + 3);
      if (t0 < n_vis) softmax(sc, pk, t0);
      __syncthreads();
    } else {
      if (t0 + 2 < n_tiles) load_k(t0 + 2);
      const bool prev = step > 0 && t0 - 1 < n_vis;
      if (prev) softmax(sc, pk, t0 - 1);
      __syncthreads();
      if (prev) pv(pk, std::integral_constant<int, (2 * (1 - PAR) + 1) * kF8Tile>{});
      if (t0 + 1 < n_vis) score(sc, std::integral_constant<int, (2 * PAR + 1) * kF8Tile>{});
      const bool v_issued = t0 + 2 < n_tiles;
      if (v_issued) load_v(t0 + 2);
      wait_all_but_v(v_issued);
      __syncthreads();
    }
  };
  const int last_step = (n_tiles + 1) / 2;
  auto run = [&](auto grp_c) __attribute__((always_inline)) {
    for (int step = 0; step <= last_step; step += 2) {
      step_body(grp_c, std::integral_constant<int, 0>{}, step);
      if (step + 1 > last_step) break;
      step_body(grp_c, std::integral_constant<int, 1>{}, step + 1);
    }
  };
  if (grp == 0) {
    run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }
  wait_vmcnt0();
  __syncthreads();

  // Merge the two groups and write out (O^T accumulator: lane l, register i
  // of block db holds d = 32 db + (i/4)*8 + 4 hl + i%4 of query row qrow).
  // O exchange: each lane's accumulator registers 4 at a time (16-byte,
  // conflict-free LDS accesses).
  f32x4* xo = reinterpret_cast<f32x4*>(lds);  // [4 rw][4 db][4 i4][64] fp32 x4
  float* xm = reinterpret_cast<float*>(lds) + 4 * 4 * 16 * 64;
  const float l_tot = l_run;
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        xo[((rw * 4 + db) * 4 + i4) * 64 + lane] =
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
    const float inv = lsum > 0.f ? vds / lsum : 0.f;
    const float c0 = a0 * inv, c1 = a1 * inv;
    // O rows staged in a wave-private, 16-byte-padded LDS area after the
    // exchange area and stored by whole rows (4 rows per instruction)
    // instead of 8 bytes into each of 32 rows.
    char* stage = reinterpret_cast<char*>(lds) + kF8MergeBytes + rw * kF8OStageBytes;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 x = xo[((rw * 4 + db) * 4 + i4) * 64 + lane];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = o[db][i4 * 4 + j] * c0 + x[j] * c1;
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(stage + (lane & 31) * kF8OStageRow + (db * 32 + i4 * 8 + hl * 4) * 2) = w;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int nvalid = Nq - qw0;
    char* o_rows = reinterpret_cast<char*>(O + ((size_t)bh * Nq + qw0) * D);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j * 4 + (lane >> 4);
      const int c = (lane & 15) * 16;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * kF8OStageRow + c);
      if (r < nvalid) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(o_rows + (size_t)r * 2 * D + c));
    }
    if (lane < 32 && qrow < Nq) LSE[(size_t)bh * Nq + qrow] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, float q_descale, float k_descale, float v_descale) {
  const int n_qt = (a.Nq + kF8BM - 1) / kF8BM;
  const long n_wg = (long)a.B * a.Hq * n_qt;
  if (n_wg == 0) return hipSuccess;
  const float sl2 = (float)((double)a.scale * q_descale * k_descale * 1.4426950408889634);
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3((unsigned)n_wg), dim3(kF8Threads), 0, (hipStream_t)a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, (uint16_t*)a.o, a.lse, a.Hq,
                     a.Hkv, a.Nq, a.Nk, sl2, v_descale, a.causal, n_qt, (int)n_wg);
  return hipGetLastError();
}

long fwd_fp8_grid(int B, int Hq, int Nq) { return (long)B * Hq * ((Nq + kF8BM - 1) / kF8BM); }

}  // namespace fa
