// bf16 attention backward (dQ, dK, dV) for gfx950, head size 64 or 128.
//
// The gradients are the chain rule through the forward definition (the pages
// print no backward algorithm): with P recomputed from the saved LSE,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO_i * O_i),
//   dQ = dS K * scale,  dK = dS^T Q * scale.
// Like the forward (the FA2 loop of "Flash Attention on the 5090 in CUDA
// C++"), the Nq x Nk matrices never reach HBM: they live in registers and LDS
// one 64 x 64 tile at a time.
//
// Kernels:
//  * bwd_prep_kernel: D_i in fp32 and a zeroed fp32 dQ accumulator (workspace).
//  * bwd_main_kernel: one workgroup (4 waves) per (batch, KV head, 128-key
//    block); each wave owns 32 keys of the block. Their K and V rows stay in
//    registers as the B operands of S = Q K^T and dP = dO V^T, and K also
//    sits in LDS for dQ. The workgroup walks the query heads of its GQA
//    group and their 64-row query blocks (under the causal mask only the
//    blocks that see a key of the block). Per query block:
//      - Q, dO, LSE, D rows into LDS;
//      - S and dP (64 rows x the wave's 32 keys) with 32x32x16 bf16 MFMAs;
//        P = exp2(S scale log2e - LSE log2e), dS = P (dP - D) in fp32,
//        masked entries 0 (masks only where a ragged or diagonal block
//        needs them);
//      - P and dS stay in registers: in the MFMA result each lane holds one
//        key and 16 rows, which is the A operand of dV += P^T dO and
//        dK += dS^T Q once dO and Q are read in that row order; dK and dV
//        (32 keys x d per wave) accumulate in registers;
//      - dS^T goes to LDS, and dQ (64 rows x d) = dS K over the 128 keys is
//        added, a 32-row x (d/2) block per wave, to the fp32 accumulator
//        with vector atomics (query blocks are shared by every key block;
//        128 keys per workgroup halve these adds against 64).
//    The next query block's Q, dO, LSE and D are loaded into registers while
//    the current one is computed, and stored to LDS before the current dQ
//    adds are issued (the wait for a load also waits for every earlier
//    atomic of the wave).
//    Column-wise operands (dO, Q, K and dS read across rows) come from the
//    transposing LDS read ds_read_b64_tr_b16 (lane semantics in fa_common.h);
//    rows are padded by 16 bytes so that row-wise 16-byte reads of 16
//    consecutive rows touch distinct banks.
//  * bwd_dq_kernel: dQ accumulator -> bf16.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdBQ = 64;  // query rows per block
constexpr int kBwdBK = 128;  // keys per workgroup
constexpr int kBwdKH = kBwdBK / 64;  // 32-key sub-blocks per wave in the key-side products
constexpr int kPStride = kBwdBQ + 8;  // P^T / dS^T row stride (elements)

template <int D>
struct BwdLayout {
  static constexpr int RS = D + 8;  // row stride of the K, Q and dO tiles (elements)
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + kBwdBK * RS;
  static constexpr int DO_OFF = Q_OFF + kBwdBQ * RS;
  static constexpr int DST_OFF = DO_OFF + kBwdBQ * RS;
  static constexpr int ELEMS = DST_OFF + kBwdBK * kPStride;  // bf16 elements; then 2 x 64 floats
  static constexpr int KS = D / 16;  // 16-wide d steps of S and dP
  static constexpr int DT = D / 32;  // 32-wide d tiles of dK and dV (each wave: all of d)
  static constexpr int DB = D / 64;  // 32-wide d tiles of dQ per wave (each wave: half of d)
};

// Operand of a 32x32x16 MFMA read across rows of a row-major bf16 tile
// (row stride RS elements): lane l gets column c0 + l % 32 of rows
// r0 + 8 (l / 32) + 0..7, i.e. 8 consecutive k values of one m (A) or n (B).
// Two transposing reads, each giving four rows.
template <int RS>
__device__ __forceinline__ bf16x8 col_operand(const uint16_t* tile, int r0, int c0, int lane) {
  const int grp = lane >> 4, w = lane & 15, e = w >> 2, j = w & 3;
  const int row = r0 + (lane >> 5) * 8 + e;
  const int col = c0 + (grp & 1) * 16 + j * 4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + row * RS + col));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + (row + 4) * RS + col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same read for a B operand that pairs with an A operand taken straight
// from a 32x32 MFMA result. In that result lane l holds rows
// 8 (i / 4) + 4 (l / 32) + i % 4 (i = 0..15) of column l % 32, so elements
// 0..7 of lane l are rows 4 (l / 32) + 0..3 and 8 + 4 (l / 32) + 0..3 (and
// elements 8..15 the same rows + 16). Lane l gets column c0 + l % 32 of rows
// r0 + 4 (l / 32) + 0..3 and r0 + 8 + 4 (l / 32) + 0..3: the k index of the
// product runs over those rows in the result's order.
template <int RS>
__device__ __forceinline__ bf16x8 col_operand_c(const uint16_t* tile, int r0, int c0, int lane) {
  const int grp = lane >> 4, w = lane & 15, e = w >> 2, j = w & 3;
  const int row = r0 + (lane >> 5) * 4 + e;
  const int col = c0 + (grp & 1) * 16 + j * 4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + row * RS + col));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + (row + 8) * RS + col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand read along a row: lane l gets elements k0 + 8 (l / 32) + 0..7 of
// row r0 + l % 32.
template <int RS>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(tile + (r0 + (lane & 31)) * RS + k0 + (lane >> 5) * 8);
}

// Copy `nrows` valid rows (of ROWS) of a [rows][D] bf16 tensor into a padded
// LDS tile; missing rows are zero.
template <int D, int ROWS>
__device__ __forceinline__ void load_rows(uint16_t* tile, const uint16_t* __restrict__ src, int nrows, int tid) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < ROWS * CH / kBwdThreads; ++i) {
    const int id = tid + i * kBwdThreads;
    const int row = id / CH, ch = id % CH;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < nrows) v = *reinterpret_cast<const u32x4*>(src + (size_t)row * D + ch * 8);
    *reinterpret_cast<u32x4*>(tile + row * BwdLayout<D>::RS + ch * 8) = v;
  }
}

// The same copy in two halves: global loads into registers (issued one query
// block ahead, so their latency hides under the current block's work), then
// the stores into the LDS tile.
template <int D>
struct RowsInFlight {
  static constexpr int CH = D / 8;
  static constexpr int N = 64 * CH / kBwdThreads;
  u32x4 r[N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int nrows, int tid) {
    if (nrows == 64) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int id = tid + i * kBwdThreads;
        r[i] = *reinterpret_cast<const u32x4*>(src + (size_t)(id / CH) * D + (id % CH) * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = tid + i * kBwdThreads;
      const int row = id / CH, ch = id % CH;
      r[i] = row < nrows ? *reinterpret_cast<const u32x4*>(src + (size_t)row * D + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = tid + i * kBwdThreads;
      *reinterpret_cast<u32x4*>(tile + (id / CH) * BwdLayout<D>::RS + (id % CH) * 8) = r[i];
    }
  }
};

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                       float* __restrict__ Dsum, float* __restrict__ dq_acc,
                                                       long rows) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float s = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += 64) {
    const float o = (float)__builtin_bit_cast(__bf16, O[row * D + c]);
    const float g = (float)__builtin_bit_cast(__bf16, dO[row * D + c]);
    s = __builtin_fmaf(o, g, s);
    dq_acc[row * D + c] = 0.f;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) Dsum[row] = s;
}

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int Nq,
    int Nk, float scale, float sl2, int causal, int n_kb) {
  using L = BwdLayout<D>;
  constexpr int RS = L::RS, KS = L::KS, DT = L::DT;
  __shared__ __attribute__((aligned(16))) uint16_t lds[L::ELEMS + 2 * 64 * 2];
  uint16_t* Ks = lds + L::K_OFF;
  uint16_t* Qs = lds + L::Q_OFF;
  uint16_t* dOs = lds + L::DO_OFF;
  uint16_t* dST = lds + L::DST_OFF;
  float* lse2 = reinterpret_cast<float*>(lds + L::ELEMS);
  float* dsum = lse2 + 64;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int half = wave & 1, dh = wave >> 1;  // dQ block owned by this wave

  // Key-block-major order: under the causal mask the first key blocks see the
  // most query blocks, so the longest workgroups start first; with B * Hkv a
  // multiple of 8 all key blocks of a head also land on one XCD (shared L2
  // for that head's Q and dO).
  const int n_bg = gridDim.x / n_kb;
  const int kb = blockIdx.x / n_bg;
  const int bg = blockIdx.x - kb * n_bg;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int group = Hq / Hkv;
  const int k0 = kb * kBwdBK;
  const int nk = Nk - k0 < kBwdBK ? Nk - k0 : kBwdBK;
  const uint16_t* Kh = K + ((size_t)(b * Hkv + g) * Nk + k0) * D;
  const uint16_t* Vh = V + ((size_t)(b * Hkv + g) * Nk + k0) * D;
  const int diag = Nk - Nq;

  // K in LDS for dQ = dS K. Each wave owns 32 keys of the block for S, dP, dK
  // and dV: their K and V rows stay in registers as the B operands of
  // S = Q K^T and dP = dO V^T (lane l: key wave*32 + l%32, d = 16 ks + 8 (l/32) + 0..7).
  load_rows<D, kBwdBK>(Ks, Kh, nk, tid);
  const int kw = wave * 32 + (lane & 31);
  bf16x8 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = vop[ks] = bf16x8{};
    if (kw < nk) {
      kop[ks] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)kw * D + ks * 16 + hl * 8);
      vop[ks] = *reinterpret_cast<const bf16x8*>(Vh + (size_t)kw * D + ks * 16 + hl * 8);
    }
  }
  // Retire these loads here (vmcnt 0; expcnt and lgkmcnt left alone): left
  // pending into the loop, the per-register wait tracking would make the
  // first MFMA of every query block wait for that block's prefetch loads too.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x16 dv[DT], dk[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dv[i] = dk[i] = f32x16{};

  // Query blocks that see a key of this block: under the causal mask, row i
  // sees key j iff j <= i + diag, so rows below k0 - diag see none.
  int qb0 = 0;
  if (causal) {
    const long first = (long)k0 - diag;
    qb0 = first <= 0 ? 0 : (int)(first / kBwdBQ);
  }
  const int n_qb = (Nq + kBwdBQ - 1) / kBwdBQ;
  // Work items: (query head of the group, query block), query block fastest.
  const int per_head = n_qb > qb0 ? n_qb - qb0 : 0;
  const int n_items = group * per_head;
  RowsInFlight<D> qn, don;
  float lse_n = kNegInf, d_n = 0.f;
  auto fetch = [&](int item) __attribute__((always_inline)) {
    const int hh = item / per_head, qb = qb0 + item % per_head;
    const size_t bh = (size_t)b * Hq + g * group + hh;
    const int q0 = qb * kBwdBQ;
    const int nq = Nq - q0 < kBwdBQ ? Nq - q0 : kBwdBQ;
    qn.load(Q + (bh * Nq + q0) * D, nq, tid);
    don.load(dO + (bh * Nq + q0) * D, nq, tid);
    if (tid < 64) {
      lse_n = tid < nq ? LSE[bh * Nq + q0 + tid] : kNegInf;
      d_n = tid < nq ? Dsum[bh * Nq + q0 + tid] : 0.f;
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
    qn.store(Qs, tid);
    don.store(dOs, tid);
    if (tid < 64) {
      // A row without keys (LSE = -inf) or past Nq gets P = 0: exp2(-inf).
      lse2[tid] = lse_n > kNegInf ? lse_n * kLog2e : __builtin_huge_valf();
      dsum[tid] = d_n;
    }
  };
  if (n_items > 0) {
    fetch(0);
    stage();
  }

  const int key = k0 + kw;
  for (int item = 0; item < n_items; ++item) {
    const int hh = item / per_head, qb = qb0 + item % per_head;
    const int h = g * group + hh;
    const size_t bh = (size_t)b * Hq + h;
    const int q0 = qb * kBwdBQ;
    const int nq = Nq - q0 < kBwdBQ ? Nq - q0 : kBwdBQ;
    // This block's Q, dO, LSE and D are in LDS, and the previous block's
    // reads of dS^T are done.
    __syncthreads();
    if (item + 1 < n_items) fetch(item + 1);

    // Masks are needed only at a ragged key block or where the causal
    // diagonal crosses the block (row 0 of the block sees its last key
    // otherwise); rows past Nq have P = 0 through their LSE either way.
    const bool full = nk == kBwdBK && (!causal || k0 + kBwdBK - 1 <= q0 + diag);
    // One straight-line body per case, so that the exponentials of one
    // 32-row tile can be scheduled under the MFMAs of the other.
    auto tiles = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        // S and dP: 32 rows x this wave's 32 keys. All A operands of a
        // product are read before its MFMAs (one wave per SIMD: nothing
        // else hides the LDS latency), dO's while the S MFMAs run.
        bf16x8 opa[KS];
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) opa[ks] = row_operand<RS>(Qs, qt * 32, ks * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32(opa[ks], kop[ks], s);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) opa[ks] = row_operand<RS>(dOs, qt * 32, ks * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dp = mfma32(opa[ks], vop[ks], dp);
        __builtin_amdgcn_sched_barrier(0);

        // P and dS. C layout: lane l holds key kw, rows qt*32 + 8 (i/4) + 4 hl + i%4.
        // Elements 8 h2 + 0..7 are the A operand (k = those rows) of one
        // 16-row step of dV += P^T dO and dK += dS^T Q; dS^T also goes to LDS for dQ.
        u32x4 pa[2], da[2];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int ql = qt * 32 + i4 * 8 + hl * 4;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + ql);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsum + ql);
          float pv[4], dsv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = i4 * 4 + j;
            float x = __builtin_fmaf(s[i], sl2, -l4[j]);
            if (decltype(masked)::value) {
              const bool vis = key < Nk && (!causal || key <= q0 + ql + j + diag);
              x = vis ? x : kNegInf;
            }
            pv[j] = fast_exp2(x);
            dsv[j] = pv[j] * (dp[i] - d4[j]);
          }
          const uint32_t p0 = pack_bf16x2(pv[0], pv[1]), p1 = pack_bf16x2(pv[2], pv[3]);
          const uint32_t d0 = pack_bf16x2(dsv[0], dsv[1]), d1 = pack_bf16x2(dsv[2], dsv[3]);
          pa[i4 >> 1][(i4 & 1) * 2] = p0;
          pa[i4 >> 1][(i4 & 1) * 2 + 1] = p1;
          da[i4 >> 1][(i4 & 1) * 2] = d0;
          da[i4 >> 1][(i4 & 1) * 2 + 1] = d1;
          *reinterpret_cast<u32x2*>(dST + kw * kPStride + ql) = u32x2{d0, d1};
        }
        // dV += P^T dO and dK += dS^T Q: this wave's 32 keys x all of d, B
        // operands read in the row order of the A operands, all of a 16-row
        // step before its MFMAs.
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 ap = __builtin_bit_cast(bf16x8, pa[h2]);
          const bf16x8 as = __builtin_bit_cast(bf16x8, da[h2]);
          const int r0 = qt * 32 + h2 * 16;
          bf16x8 bo[DT], bq[DT];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            bo[dt] = col_operand_c<RS>(dOs, r0, dt * 32, lane);
            bq[dt] = col_operand_c<RS>(Qs, r0, dt * 32, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            dv[dt] = mfma32(ap, bo[dt], dv[dt]);
            dk[dt] = mfma32(as, bq[dt], dk[dt]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if (full)
      tiles(std::false_type{});
    else
      tiles(std::true_type{});
    // dS^T of all 128 keys is in LDS, and Qs, dOs, LSE and D are no longer
    // read: the next block goes in now, before this block's dQ atomics, so
    // that waiting for its loads never waits for those adds as well.
    __syncthreads();
    if (item + 1 < n_items) stage();

    // dQ rows half*32.. (+ q0), d blocks dh*(D/2) + 32 i: dS K over the 128 keys.
    f32x16 dq[L::DB];
#pragma unroll
    for (int i = 0; i < L::DB; ++i) dq[i] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kBwdBK / 16; ++ks) {
      const bf16x8 a = col_operand<kPStride>(dST, ks * 16, half * 32, lane);
#pragma unroll
      for (int i = 0; i < L::DB; ++i) dq[i] = mfma32(a, col_operand<RS>(Ks, ks * 16, dh * (D / 2) + i * 32, lane), dq[i]);
    }
    // C layout: lane l holds d column c0 + l%32, rows (i/4)*8 + 4 hl + i%4.
    float* dq_row = dq_acc + (bh * Nq + q0 + half * 32 + hl * 4) * D + dh * (D / 2) + (lane & 31);
    if (nq == kBwdBQ) {
#pragma unroll
      for (int i = 0; i < L::DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) unsafeAtomicAdd(dq_row + ((r >> 2) * 8 + (r & 3)) * D + i * 32, dq[i][r] * scale);
    } else {
#pragma unroll
      for (int i = 0; i < L::DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = half * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (ql < nq) unsafeAtomicAdd(dq_row + ((r >> 2) * 8 + (r & 3)) * D + i * 32, dq[i][r] * scale);
        }
    }
  }

  // dK (times scale) and dV, bf16: lane holds d column, key rows wave*32 + (i/4)*8 + 4 hl + i%4.
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d = dt * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = wave * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
      if (kl < nk) {
        const size_t off = ((size_t)(b * Hkv + g) * Nk + k0 + kl) * D + d;
        dK[off] = __builtin_bit_cast(uint16_t, (__bf16)(dk[dt][r] * scale));
        dV[off] = __builtin_bit_cast(uint16_t, (__bf16)dv[dt][r]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                     long n) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  // n is a multiple of 64 (rows of d = 64 or 128 elements).
  const f32x4 v = *reinterpret_cast<const f32x4*>(acc + i);
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(dq + i) = w;
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  const long rows = (long)a.f.B * a.f.Hq * a.f.Nq;
  hipStream_t st = (hipStream_t)a.f.stream;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dsum, a.dq_acc, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_kb = (a.f.Nk + kBwdBK - 1) / kBwdBK;
  const long n_wg = (long)a.f.B * a.f.Hkv * n_kb;
  if (n_wg > 0) {
    hipLaunchKernelGGL(bwd_main_kernel<D>, dim3((unsigned)n_wg), dim3(kBwdThreads), 0, st, (const uint16_t*)a.f.q,
                       (const uint16_t*)a.f.k, (const uint16_t*)a.f.v, (const uint16_t*)a.dout, a.f.lse, a.dsum,
                       a.dq_acc, (uint16_t*)a.dk, (uint16_t*)a.dv, a.f.Hq, a.f.Hkv, a.f.Nq, a.f.Nk, a.f.scale,
                       a.f.scale * kLog2e, a.f.causal, n_kb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long n = rows * D;
  if (n > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, a.dq_acc,
                       (uint16_t*)a.dq, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) { return a.f.d == 128 ? launch_bwd_d<128>(a) : launch_bwd_d<64>(a); }

long bwd_grid(int B, int Hkv, int Nk) { return (long)B * Hkv * ((Nk + kBwdBK - 1) / kBwdBK); }

}  // namespace fa
