// Split-KV attention forward (decode) and the LSE-weighted combine, gfx950.
//
// Decode rows are few (one query per head) and the K/V stream is long, so
// the work is memory bound: the kernel is shaped to keep many K/V bytes in
// flight, not to fill the matrix cores. Partial softmax results of several
// key chunks must be merged; the FlashDecoding++ snippet on the
// "flash attention v3 paper" search-result page names that merge as a cost
// of decode attention. Here each chunk's result is written once (normalised
// O_s, LSE_s) and a second small kernel merges the chunks with the same
// rescale the online softmax applies to tiles ("Flash Attention on the 5090
// in CUDA C++", "v1 -- basic version"), now applied to whole chunks.
//
// Partial kernel, one workgroup per (chunk s, 16-row block, KV head g, batch b):
//  * the rows are the (query head in g's group, query index) pairs, so the
//    Hq/Hkv query heads that share a KV head read each K/V byte once;
//  * 256 threads = 4 waves; the chunk's keys are cut into 32-key blocks and
//    wave w takes blocks w, w+4, ...; each wave streams its blocks with two
//    blocks of K and V in flight in registers (about 32 KiB per wave), so a
//    CU with two workgroups keeps ~256 KiB of loads outstanding;
//  * 16x16x32 bf16 MFMAs (16 rows: a GQA group of 4 wastes less of the tile
//    than a 32-row one): S^T = K Q^T with K straight from registers (each load
//    instruction reads 64 contiguous bytes of 16 key rows), then
//    O^T += V^T P^T with V^T read transposed from a wave-private LDS slice;
//  * each wave keeps its own running (m, l, O); the four are merged through
//    LDS at the end and the chunk's normalised O_s and LSE_s are written.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kSplitThreads = 256;
constexpr int kSplitRows = 16;
constexpr int kBlk = 32;  // keys per wave block

template <int D>
struct SplitStage {
  bf16x8 k[2][D / 32];  // K, sub-block a/b, one 16-byte piece per k-step
  u32x4 v[kBlk * D / 8 / 64];  // V rows, coalesced (16 bytes per lane per instruction)
};

// Key offset (within a 32-key block) of the K row lane i16 feeds to the A
// operand of sub-block `sb`: sub-block a rows 4G'+i hold keys 8G'+i, sub-block
// b rows hold keys 8G'+4+i. Each lane's score registers then cover 8
// consecutive keys, the key-contiguous B operand of the P.V MFMA.
__device__ __forceinline__ int blk_key(int i16, int sb) { return 8 * (i16 >> 2) + 4 * sb + (i16 & 3); }

// Where the key rows of one KV head live.
//  Contiguous: rows key * D of [Nk, D] tensors.
//  Paged: the cache is [num_pages, Hkv, page, D]; logical page j of the
//  sequence is physical page block_table[j]. Pages hold at least 16 keys, so
//  the 32 keys of a block (which starts wherever its chunk does) span at most
//  three pages; `pg` holds the physical pages of logical pages
//  kb / page .. kb / page + 2.
// Physical pages of the (up to) three logical pages a 32-key block touches,
// as three wave-uniform values (an indexed array would be placed in memory).
struct Pages {
  int p0, p1, p2;
};

// kTwoRuns / bases(): a paged block whose keys 0..15 are 16 consecutive rows
// and keys 16..31 another 16 is loaded from the element offsets of those two
// runs (lo, hi) with no per-row arithmetic; bases() is false when the block's
// rows are not two such runs. Contiguous rows keep the per-row path, which
// measured slightly faster for them (376.5 vs 379 us on the decode workload).
template <int D>
struct ContigRows {
  static constexpr bool kTwoRuns = false;
  const uint16_t* k;
  const uint16_t* v;
  __device__ __forceinline__ size_t row(int key, int /*kb*/, const Pages& /*pg*/) const { return (size_t)key * D; }
  __device__ __forceinline__ bool bases(int, const Pages&, size_t&, size_t&) const { return false; }
};
template <int D>
struct PagedRows {
  static constexpr bool kTwoRuns = true;
  const uint16_t* k;  // cache base + head offset (g * page * D)
  const uint16_t* v;
  int log2_page;
  int head_stride;    // Hkv * page * D
  __device__ __forceinline__ size_t row(int key, int kb, const Pages& pg) const {
    const int sub = (key >> log2_page) - (kb >> log2_page);
    // Arithmetic rather than a select chain on sub: the compiler turns such
    // a chain into an indexed table in memory.
    const int page = pg.p0 + (sub >= 1 ? pg.p1 - pg.p0 : 0) + (sub >= 2 ? pg.p2 - pg.p1 : 0);
    return (size_t)page * head_stride + (size_t)(key & ((1 << log2_page) - 1)) * D;
  }
  // Two runs when the block lies in one page, or when its second half starts
  // a page (16-key pages with the block on a page edge).
  __device__ __forceinline__ bool bases(int kb, const Pages& pg, size_t& lo, size_t& hi) const {
    const int p = 1 << log2_page, off = kb & (p - 1);
    lo = (size_t)pg.p0 * head_stride + (size_t)off * D;
    if (off + 32 <= p) {
      hi = lo + 16 * D;
      return true;
    }
    hi = (size_t)pg.p1 * head_stride;
    return off + 16 == p;
  }
};

// A wave-uniform global pointer, marked as such (kept in scalar registers, so
// loads take it as their scalar base with a 32-bit lane offset).
typedef const __attribute__((address_space(1))) char gchar;
typedef const __attribute__((address_space(1))) u32x4 gu32x4;
__device__ __forceinline__ gchar* uniform_ptr(const void* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}

// Every K and V byte of a decode step is read once, so the loads carry the
// non-temporal hint (they then do not displace other data in the caches):
// 377 -> 354 us for the contiguous decode workload, 387 -> 369 us paged.
template <int D, typename Rows>
__device__ __forceinline__ void load_stage(SplitStage<D>& st, const Rows& src, int kb, int k1, const Pages& pg,
                                           int lane) {
  constexpr int KS = D / 32;
  constexpr int CH = D / 8, RPI = 64 / CH;
  const int i16 = lane & 15, g4 = lane >> 4;
  size_t lo = 0, hi = 0;
  if (Rows::kTwoRuns && kb + kBlk <= k1 && src.bases(kb, pg, lo, hi)) {
    // Full block in two runs of 16 rows: every address is a wave-uniform run
    // base, a loop-invariant lane offset and an immediate (no per-row
    // arithmetic). K lanes i16 < 8 hold keys 0..15 (blk_key), V instruction t
    // rows t RPI + lane / CH.
    const size_t kbase = i16 < 8 ? lo : hi;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const uint16_t* row = src.k + kbase + (blk_key(i16, sb) & 15) * D + 8 * g4;
#pragma unroll
      for (int s = 0; s < KS; ++s) st.k[sb][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(row + 32 * s));
    }
    gchar* v0 = uniform_ptr(src.v + lo);
    gchar* v1 = uniform_ptr(src.v + hi);
    const uint32_t vl = (uint32_t)(((lane / CH) * D + (lane % CH) * 8) * 2);
#pragma unroll
    for (int t = 0; t < kBlk * D / 8 / 64; ++t) {
      gchar* vb = t * RPI < 16 ? v0 : v1;
      st.v[t] = __builtin_nontemporal_load(reinterpret_cast<gu32x4*>(vb + vl + ((t * RPI) % 16) * D * 2));
    }
    return;
  }
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    int key = kb + blk_key(i16, sb);
    key = key < k1 ? key : k1 - 1;
    const uint16_t* row = src.k + src.row(key, kb, pg) + 8 * g4;
#pragma unroll
    for (int s = 0; s < KS; ++s) st.k[sb][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(row + 32 * s));
  }
#pragma unroll
  for (int t = 0; t < kBlk * D / 8 / 64; ++t) {
    int key = kb + t * RPI + lane / CH;
    key = key < k1 ? key : k1 - 1;
    st.v[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src.v + src.row(key, kb, pg) + (lane % CH) * 8));
  }
}

// PAGED: K and V are page caches [num_pages, Hkv, 2^log2_page, D], each
// sequence's pages listed in block_table [B, max_pages] and its key count in
// seq_lens [B]; the chunk size is then per sequence. Table entries and lengths
// out of range are clamped into range (memory stays in bounds).
template <int D, bool PAGED>
__global__ __launch_bounds__(kSplitThreads, 2) void splitkv_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ LSEpart, int Hq, int Hkv, int Nq, int Nk,
    float sl2, int causal, int S, int chunk, const int* __restrict__ block_table,
    const int* __restrict__ seq_lens, int num_pages, int log2_page, int max_pages) {
  constexpr int KS = D / 32;    // k-steps of the score MFMA
  constexpr int DB = D / 16;    // 16-wide d blocks of O
  constexpr int CH = D / 8, RPI = 64 / CH, VI = kBlk * D / 8 / 64;
  __shared__ __attribute__((aligned(1024))) uint16_t vlds[4][kBlk * D];  // one V block per wave
  __shared__ float ms[4][kSplitRows], ls[4][kSplitRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;
  const int s = blockIdx.x % S, rb = blockIdx.x / S;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, R = G * Nq;
  const int r = rb * kSplitRows + i16;
  const bool rvalid = r < R;
  const int hh = rvalid ? r / Nq : 0, qi = rvalid ? r - hh * Nq : 0;
  const int head = g * G + hh;
  const int* bt = block_table + (size_t)b * max_pages;
  if constexpr (PAGED) {
    const long cap = (long)max_pages << log2_page;
    const long n = seq_lens[b];
    Nk = n < 0 ? 0 : (int)(n < cap ? n : cap);
    chunk = (int)(((long)Nk + S - 1) / S);
  }
  const int diag = Nk - Nq;

  bf16x8 qf[KS];
  {
    const uint16_t* qrow = Q + ((size_t)(b * Hq + head) * Nq + qi) * D + 8 * g4;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = rvalid ? *reinterpret_cast<const bf16x8*>(qrow + 32 * k) : bf16x8{};
  }

  const long k0l = (long)s * chunk;
  const int k0 = k0l < Nk ? (int)k0l : Nk;
  const int k1 = (long)k0 + chunk < (long)Nk ? k0 + chunk : Nk;
  const int nblk = (k1 - k0 + kBlk - 1) / kBlk;
  const int nbw = nblk > wave ? (nblk - wave + 3) / 4 : 0;  // blocks of this wave
  const int lim = causal ? qi + diag : 0x7fffffff;

  using Rows = typename std::conditional<PAGED, PagedRows<D>, ContigRows<D>>::type;
  Rows src;
  if constexpr (PAGED) {
    const size_t head_off = (size_t)g << log2_page;
    src = Rows{K + head_off * D, V + head_off * D, log2_page, (Hkv << log2_page) * D};
  } else {
    src = Rows{K + (size_t)(b * Hkv + g) * Nk * D, V + (size_t)(b * Hkv + g) * Nk * D};
  }
  // Physical pages of the block starting at key kb (unused when contiguous).
  // The wave keeps a window of 64 consecutive table entries in one register
  // (lane j: logical page win + j, already clamped into [0, num_pages)), read
  // with one vector load, so the loop reads page numbers with v_readlane
  // instead of waiting on memory; the window moves only when a block needs a
  // page past it (chunks longer than 64 pages).
  int win = 0, tbl = 0;
  auto load_window = [&](int lp) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      win = lp;
      const int l = lp + lane < max_pages ? lp + lane : max_pages - 1;
      const int p = bt[l];
      tbl = p < 0 ? 0 : (p < num_pages ? p : num_pages - 1);
    }
  };
  auto pages_of = [&](int kb, Pages& pg) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int lp = kb >> log2_page;
      if (lp - win + 2 >= 64) load_window(lp);
      pg.p0 = __builtin_amdgcn_readlane(tbl, lp - win);
      pg.p1 = __builtin_amdgcn_readlane(tbl, lp - win + 1);
      pg.p2 = __builtin_amdgcn_readlane(tbl, lp - win + 2);
    } else {
      pg = Pages{0, 0, 0};
    }
  };
  if constexpr (PAGED) {
    if (max_pages > 0) load_window(k0 >> log2_page);
  }
  uint16_t* vw = vlds[wave];
  const char* vw_c = reinterpret_cast<const char*>(vw);

  // Loop-invariant LDS offsets: V stores (row t*RPI + lane/CH, chunk lane%CH)
  // and the transposed V^T operand reads.
  uint32_t vst_off[VI];
#pragma unroll
  for (int t = 0; t < VI; ++t) {
    const int row = t * RPI + lane / CH;
    vst_off[t] = (row * D + swz<D>(row, lane % CH) * 8) * 2;
  }
  uint32_t vtr_off[DB][2];
  {
    const int e = i16 >> 2, c = i16 & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g4 + 4 * h + e;
        const int col = 16 * db + 4 * c;
        vtr_off[db][h] = (row * D + swz<D>(row, col / 8) * 8 + (col & 7)) * 2;
      }
  }

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

  SplitStage<D> st[2];
  // Page numbers are fetched one block ahead of the loads that use them.
  Pages pg_cur{0, 0, 0}, pg_next{0, 0, 0};
  if (nbw > 0) {
    pages_of(k0 + kBlk * wave, pg_cur);
    load_stage<D>(st[0], src, k0 + kBlk * wave, k1, pg_cur, lane);
  }
  if (nbw > 1) {
    pages_of(k0 + kBlk * (wave + 4), pg_cur);
    load_stage<D>(st[1], src, k0 + kBlk * (wave + 4), k1, pg_cur, lane);
  }
  if (nbw > 2) pages_of(k0 + kBlk * (wave + 8), pg_next);

  auto block = [&](SplitStage<D>& cur, int i) {
    const int kb = k0 + kBlk * (wave + 4 * i);
#pragma unroll
    for (int t = 0; t < VI; ++t) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(vw) + vst_off[t]) = cur.v[t];
    f32x4 sc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      sc[0] = mfma16(cur.k[0][k], qf[k], sc[0]);
      sc[1] = mfma16(cur.k[1][k], qf[k], sc[1]);
    }
    if (i + 2 < nbw) {
      const Pages nb = pg_next;
      if (i + 3 < nbw) pages_of(k0 + kBlk * (wave + 4 * (i + 3)), pg_next);
      load_stage<D>(cur, src, k0 + kBlk * (wave + 4 * (i + 2)), k1, nb, lane);
    }
    if (kb + kBlk > k1 || causal) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kb + 8 * g4 + 4 * sb + j;
          if (key >= k1 || key > lim) sc[sb][j] = kNegInf;
        }
    }
    float mx = vmax(vmax(vmax(sc[0][0], sc[0][1]), sc[0][2]),
                    vmax(vmax(sc[0][3], sc[1][0]), vmax(vmax(sc[1][1], sc[1][2]), sc[1][3])));
    mx = max_with_lane_xor32(max_with_lane_xor16(mx)) * sl2;
    const float m_new = vmax(m_run, mx);
    const float base = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    bf16x8 p;
    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = fast_exp2(__builtin_fmaf(sc[sb][j], sl2, -base));
        rs += e;
        p[4 * sb + j] = (__bf16)e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vw_c + vtr_off[db][0]));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vw_c + vtr_off[db][1]));
      o[db] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), p, o[db] * alpha);
    }
  };
  for (int i = 0; i < nbw; i += 2) {
    block(st[0], i);
    if (i + 1 >= nbw) break;
    block(st[1], i + 1);
  }

  // Merge the four waves' (m, l, O~) through LDS.
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  __syncthreads();
  float* os = reinterpret_cast<float*>(&vlds[0][0]);  // [4][DB][4][64] fp32 (16 KiB per wave at D=128)
  if (lane < kSplitRows) {
    ms[wave][lane] = m_run;
    ls[wave][lane] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) os[((wave * DB + db) * 4 + i) * 64 + lane] = o[db][i];
  __syncthreads();
  // Thread (row, d): row = idx / D, d = idx % D; O^T element (d, row) sits in
  // register i = d % 4 of lane 16 * ((d % 16) / 4) + row, block d / 16.
  for (int idx = tid; idx < kSplitRows * D; idx += kSplitThreads) {
    const int row = idx / D, d = idx - row * D;
    const int rr = rb * kSplitRows + row;
    if (rr >= R) continue;
    const int h2 = g * G + rr / Nq, q2 = rr % Nq;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w][row]);
    float val = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float den = 0.f, num = 0.f;
      const int src_lane = 16 * ((d & 15) >> 2) + row;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = fast_exp2(ms[w][row] - M);
        den += ls[w][row] * sc;
        num += os[((w * DB + (d >> 4)) * 4 + (d & 3)) * 64 + src_lane] * sc;
      }
      val = num / den;
      lse = (M + fast_log2(den)) * kLn2;
    }
    const size_t pr = ((size_t)(b * Hq + h2) * S + s) * Nq + q2;
    Opart[pr * D + d] = val;
    if (d == 0) LSEpart[pr] = lse;
  }
}

// One wave per output row. With at most 64 chunks every lane reads one
// chunk's LSE, so the max and the weights need no serial loop over chunks;
// the O rows of four chunks are then loaded together per step. More chunks
// take the plain loop.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Opart,
                                                      const float* __restrict__ LSEpart,
                                                      uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                      long rows, int Nq, int S) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const long bh = row / Nq;
  const int qi = (int)(row - bh * Nq);
  const float* lp = LSEpart + (size_t)bh * S * Nq + qi;
  const float* op = Opart + ((size_t)bh * S * Nq + qi) * D + lane * PER;
  const size_t ostride = (size_t)Nq * D;
  float M = kNegInf, den = 0.f;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  if (S <= 64) {
    const float ls = lane < S ? lp[(size_t)lane * Nq] : kNegInf;
    M = ls;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    const float w = (lane < S && M != kNegInf) ? expf(ls - M) : 0.f;
    den = w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m, 64);
    if (M != kNegInf) {
      int s = 0;
      for (; s + 4 <= S; s += 4) {
        float v[4][PER], ww[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ww[j] = __shfl(w, s + j, 64);
#pragma unroll
          for (int p = 0; p < PER; ++p) v[j][p] = op[(size_t)(s + j) * ostride + p];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int p = 0; p < PER; ++p) acc[p] = __builtin_fmaf(ww[j], v[j][p], acc[p]);
      }
      for (; s < S; ++s) {
        const float ws = __shfl(w, s, 64);
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = __builtin_fmaf(ws, op[(size_t)s * ostride + p], acc[p]);
      }
    }
  } else {
    for (int s = 0; s < S; ++s) M = fmaxf(M, lp[(size_t)s * Nq]);
    if (M != kNegInf) {
      for (int s = 0; s < S; ++s) {
        const float w = expf(lp[(size_t)s * Nq] - M);
        den += w;
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = __builtin_fmaf(w, op[(size_t)s * ostride + p], acc[p]);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* orow = O + (size_t)row * D + lane * PER;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    __bf16 x = (__bf16)(acc[p] * inv);
    orow[p] = __builtin_bit_cast(uint16_t, x);
  }
  if (lane == 0) LSE[row] = den > 0.f ? M + logf(den) : kNegInf;
}

template <int D>
hipError_t launch_partial_d(const SplitArgs& a) {
  const FwdArgs& f = a.f;
  const int G = f.Hq / f.Hkv;
  const int nrb = (G * f.Nq + kSplitRows - 1) / kSplitRows;
  if (f.B == 0 || nrb == 0) return hipSuccess;
  const int S = a.num_splits;
  const int chunk = (int)(((long)f.Nk + S - 1) / S);
  const float sl2 = f.scale * kLog2e;
  auto* kernel = a.paged ? splitkv_partial_kernel<D, true> : splitkv_partial_kernel<D, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(S * nrb), (unsigned)f.Hkv, (unsigned)f.B), dim3(kSplitThreads), 0,
                     (hipStream_t)f.stream, (const uint16_t*)f.q, (const uint16_t*)f.k, (const uint16_t*)f.v,
                     a.o_part, a.lse_part, f.Hq, f.Hkv, f.Nq, f.Nk, sl2, f.causal, S, chunk, a.block_table,
                     a.seq_lens, a.num_pages, a.log2_page, a.max_pages);
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine_d(const CombineArgs& a) {
  const long rows = (long)a.B * a.Hq * a.Nq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, (hipStream_t)a.stream,
                     a.o_part, a.lse_part, (uint16_t*)a.o, a.lse, rows, a.Nq, a.num_splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv_partial(const SplitArgs& a) {
  return a.f.d == 128 ? launch_partial_d<128>(a) : launch_partial_d<64>(a);
}

hipError_t launch_combine(const CombineArgs& a) {
  return a.d == 128 ? launch_combine_d<128>(a) : launch_combine_d<64>(a);
}

long splitkv_grid(int B, int Hq, int Hkv, int Nq, int num_splits) {
  const long G = Hq / Hkv;
  return (long)num_splits * ((G * Nq + kSplitRows - 1) / kSplitRows);
}

long combine_grid(int B, int Hq, int Nq) { return ((long)B * Hq * Nq + 3) / 4; }

}  // namespace fa
