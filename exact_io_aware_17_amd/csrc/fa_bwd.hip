// bf16 attention backward (dQ, dK, dV) for gfx950, head size 64 or 128.
//
// The gradients are the chain rule through the forward definition (the pages
// print no backward algorithm): with P recomputed from the saved LSE,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO_i * O_i),
//   dQ = dS K * scale,  dK = dS^T Q * scale.
// Like the forward (the FA2 loop of "Flash Attention on the 5090 in CUDA
// C++"), the Nq x Nk matrices never reach HBM: they live in registers one
// 32 x 32 tile at a time.
//
// Kernels (no atomics: every output element is written by one lane):
//  * bwd_prep_kernel: D_i in fp32 (workspace).
//  * bwd_dkdv_kernel: one workgroup (8 waves, two per SIMD) per (batch, KV
//    head, 128-key block). Waves w and w + 4 share 32 keys, whose K rows stay
//    in registers as the B operands of S = Q K^T (V sits in LDS for
//    dP = dO V^T). The workgroup walks the query heads of its GQA group and
//    their 64-row query blocks (under the causal mask only the blocks that
//    see a key of the block), Q, dO, LSE and D double-buffered in LDS (the
//    next block's rows are loaded into registers by the four waves that
//    would otherwise wait at the block's exchange barrier, and stored into
//    LDS after the block's products). Per query block:
//      - wave w + 4 r computes, for the 32-row half r of the block, S and dP
//        (32 rows x the pair's 32 keys) with 32x32x16 bf16 MFMAs;
//        P = exp2(S scale log2e - LSE log2e), dS = P (dP - D) in fp32,
//        masked entries 0 (masks only where a ragged or diagonal block
//        needs them);
//      - in the MFMA result each lane holds one key and 16 rows, which is
//        the A operand of dV += P^T dO and dK += dS^T Q once dO and Q are
//        read in that row order: the pair swaps these bf16 operands through
//        LDS, and each wave accumulates dK and dV over all 64 rows for its
//        half of d (32 keys x d/2 in registers), so that a wave fits in half
//        of the SIMD's registers and one wave's softmax runs under the
//        other's MFMAs. A wave runs the products of its own 32 rows from
//        registers before the swap barrier and reads only its partner's
//        operands after it.
//  * bwd_dq_kernel: one workgroup (8 waves, two per SIMD) per (batch, query
//    head, 128-row block). Waves w and w + 4 share 32 rows, whose Q and dO
//    stay in registers. S and dP are recomputed transposed, S^T = K Q^T and
//    dP^T = V dO^T, 128 keys at a time (K double-buffered and V single-
//    buffered in LDS, the block after next in flight in registers), wave
//    w + 4 r taking the two 32-key tiles of keys 64 r..64 r + 63 of each
//    block: in that MFMA result each lane holds one query row, so LSE and D
//    are one value per lane, and its 16 keys are the B operand of
//    dQ^T += K^T dS^T once K is read in that key order. The pair swaps these
//    bf16 operands through LDS, and each wave accumulates dQ^T
//    over all 128 keys for its half of d (d/2 x 32 rows in registers until
//    the end).
//    Recomputing S and dP here costs two more products than adding each key
//    block's dQ into an fp32 accumulator with atomics, but those adds
//    (B Hq Nq d of them per 128 keys) are carried out memory-side at a rate
//    that bounded the whole pass.
//  Column-wise operands (dO, Q and K read across rows) come from the
//  transposing LDS read ds_read_b64_tr_b16 (lane semantics in fa_common.h);
//  rows are padded so that row-wise 16-byte reads of 16 consecutive rows
//  touch distinct banks and the transposing reads are at most 2-way. All
//  LDS operands of a product are read before its MFMAs (with one wave per
//  SIMD nothing else hides the LDS latency).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 512;  // dK/dV and dQ kernels: 8 waves, two per SIMD
constexpr int kBwdBQ = 64;    // dK/dV kernel: query rows per block
constexpr int kBwdBK = 128;   // dK/dV kernel: keys per workgroup (32 per wave)
constexpr int kDqRows = 128;  // dQ kernel: query rows per workgroup (32 per wave)
constexpr int kDqBK = 128;    // dQ kernel: keys per block (two 32-key tiles per wave)

template <int D>
struct BwdLayout {
  // Row stride of the Q, dO, K and V tiles (elements). The padding sets the
  // bank shift between rows (64 banks of 4 bytes): 48 bytes at d = 128 leave
  // the 16-byte row reads conflict-free and the transposing reads 2-way
  // (16 bytes: 4-way), 16 bytes at d = 64 give the same.
  static constexpr int RS = D == 128 ? D + 24 : D + 8;
  static constexpr int TILE = kBwdBQ * RS;  // one 64-row tile
  static constexpr int KS = D / 16;  // 16-wide d steps of S and dP
  static constexpr int DT = D / 32;  // 32-wide d tiles of dK, dV and dQ (each wave: all of d)
};

// Operand of a 32x32x16 MFMA read across rows of a row-major bf16 tile (row
// stride RS elements), for use with an operand taken straight from a 32x32
// MFMA result. In that result lane l holds rows
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

// Copy of 64 rows of a [rows][D] bf16 tensor into a padded LDS tile in two
// halves: global loads into registers (issued one block ahead, so that their
// latency hides under the current block's work), then the stores into the
// tile. Rows past `nrows` repeat row nrows - 1: finite data whose products
// the kernels zero (keys past Nk are masked, rows past Nq have P = 0 through
// their LSE); a tile with no valid row is zero and issues no load. Every
// load is unconditional: a select between a load and zero makes the
// compiler zero the destination first, and it then waits for all loads in
// flight before each such write, which serialises the block's loads.
template <int D, int NT = kBwdThreads>
struct RowsInFlight {
  static constexpr int CH = D / 8;
  static constexpr int N = 64 * CH / NT;
  u32x4 r[N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int nrows, int tid) {
    if (nrows <= 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) r[i] = u32x4{0u, 0u, 0u, 0u};
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = tid + i * NT;
      const int row = id / CH, ch = id % CH;
      const int rr = row < nrows ? row : nrows - 1;
      r[i] = *reinterpret_cast<const u32x4*>(src + (size_t)rr * D + ch * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = tid + i * NT;
      *reinterpret_cast<u32x4*>(tile + (id / CH) * BwdLayout<D>::RS + (id % CH) * 8) = r[i];
    }
  }
};


template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                       float* __restrict__ Dsum, long rows) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float s = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += 64) {
    const float o = (float)__builtin_bit_cast(__bf16, O[row * D + c]);
    const float g = (float)__builtin_bit_cast(__bf16, dO[row * D + c]);
    s = __builtin_fmaf(o, g, s);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) Dsum[row] = s;
}

// Retire every outstanding vector-memory load (vmcnt 0; expcnt and lgkmcnt
// left alone). Loads of loop-invariant registers issued before a loop and left
// pending into it would make the first use in every iteration wait for that
// iteration's own prefetch loads as well.
__device__ __forceinline__ void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int Nq, int Nk, float scale, float sl2,
    int causal, int n_kb) {
  using L = BwdLayout<D>;
  constexpr int RS = L::RS, KS = L::KS, DH = L::DT / 2;
  // [buffer][Q, dO] tiles; the block's 128 V rows; per wave 64 lanes x 64
  // bytes of P and dS operands for its partner; [buffer][LSE * log2e, D]
  // rows of 64 floats.
  constexpr int XCH = 8 * 64 * 32;  // bf16 elements of the operand exchange
  __shared__ __attribute__((aligned(16))) uint16_t lds[6 * L::TILE + XCH + 2 * 2 * 64 * 2];
  uint16_t* Vs = lds + 4 * L::TILE;
  u32x4* xch = reinterpret_cast<u32x4*>(lds + 6 * L::TILE);
  float* rowv = reinterpret_cast<float*>(lds + 6 * L::TILE + XCH);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;

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

  // Waves w and w + 4 (one SIMD) share 32 keys: wave w computes S, dP, P
  // and dS for rows 0..31 of each query block and wave w + 4 for rows
  // 32..63; they swap the bf16 P and dS operands through LDS, and each then
  // accumulates dK and dV over all 64 rows for one half of d. So a wave needs
  // half the accumulators and fits in half of the SIMD's registers, and the
  // two waves of a SIMD overlap one's softmax with the other's MFMAs.
  // K rows are the B operands of S = Q K^T (lane l holds key kg*32 + l%32,
  // d = 16 ks + 8 (l/32) + 0..7); V goes to LDS for dP = dO V^T (keys past Nk
  // are zero).
  const int kg = wave & 3, role = wave >> 2;
  const int kw = kg * 32 + (lane & 31);
  bf16x8 kop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = bf16x8{};
    if (kw < nk) kop[ks] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)kw * D + ks * 16 + hl * 8);
  }
  {
    RowsInFlight<D> vr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      vr.load(Vh + (size_t)h * 64 * D, nk - h * 64, tid);
      vr.store(Vs + h * 64 * RS, tid);
    }
  }
  wait_vm_loads();

  f32x16 dv[DH], dk[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) dv[i] = dk[i] = f32x16{};

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
  // The next block's Q and dO rows are loaded and staged by the role-0 waves
  // alone (threads 0..255), which wait at the swap barrier for their slower
  // partners anyway: their loads issue there instead of on every wave's
  // critical path.
  RowsInFlight<D, kBwdThreads / 2> qn, don;
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
  auto stage = [&](int buf) __attribute__((always_inline)) {
    qn.store(lds + (2 * buf) * L::TILE, tid);
    don.store(lds + (2 * buf + 1) * L::TILE, tid);
    if (tid < 64) {
      // A row without keys (LSE = -inf) or past Nq gets P = 0: exp2(-inf).
      rowv[buf * 128 + tid] = lse_n > kNegInf ? lse_n * kLog2e : __builtin_huge_valf();
      rowv[buf * 128 + 64 + tid] = d_n;
    }
  };
  if (n_items > 0 && role == 0) {
    fetch(0);
    stage(0);
  }

  const int key = k0 + kw;
  for (int item = 0; item < n_items; ++item) {
    const int qb = qb0 + item % per_head;
    const int q0 = qb * kBwdBQ;
    const int buf = item & 1;
    const uint16_t* Qs = lds + (2 * buf) * L::TILE;
    const uint16_t* dOs = lds + (2 * buf + 1) * L::TILE;
    const float* lse2 = rowv + buf * 128;
    const float* dsum = lse2 + 64;
    // This block's rows are in LDS, and every wave is done with the other
    // buffer (the previous block), which the next block now goes into.
    __syncthreads();

    // Masks are needed only at a ragged key block or where the causal
    // diagonal crosses the block (row 0 of the block sees its last key
    // otherwise); rows past Nq have P = 0 through their LSE either way.
    const bool full = nk == kBwdBK && (!causal || k0 + kBwdBK - 1 <= q0 + diag);
    // S and dP of a 32-row tile: 32 rows x this wave's 32 keys; the dO rows
    // are read while the S MFMAs run.
    auto sdp = [&](int qt, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
      s = dp = f32x16{};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 opa[KS / 2];
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) opa[k] = row_operand<RS>(Qs, qt * 32, (h * KS / 2 + k) * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) s = mfma32(opa[k], kop[h * KS / 2 + k], s);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 opa[KS / 2], opb[KS / 2];
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) {
          opa[k] = row_operand<RS>(dOs, qt * 32, (h * KS / 2 + k) * 16, lane);
          opb[k] = row_operand<RS>(Vs, kg * 32, (h * KS / 2 + k) * 16, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) dp = mfma32(opa[k], opb[k], dp);
      }
    };
    // P and dS. C layout: lane l holds key kw, rows qt*32 + 8 (i/4) + 4 hl + i%4.
    // Elements 8 h2 + 0..7 are the A operand (k = those rows) of one 16-row
    // step of dV += P^T dO and dK += dS^T Q.
    auto p_ds = [&](auto masked, int qt, const f32x16& s, const f32x16& dp, u32x4* pa, u32x4* da)
                    __attribute__((always_inline)) {
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
        pa[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(pv[0], pv[1]);
        pa[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
        da[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(dsv[0], dsv[1]);
        da[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
    };
    // dV += P^T dO and dK += dS^T Q: this wave's 32 keys x all of d, B
    // operands read in the row order of the A operands.
    auto dvdk = [&](int qt, const u32x4* pa, const u32x4* da) __attribute__((always_inline)) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 ap = __builtin_bit_cast(bf16x8, pa[h2]);
        const bf16x8 as = __builtin_bit_cast(bf16x8, da[h2]);
        const int r0 = qt * 32 + h2 * 16;
        bf16x8 bo[DH], bq[DH];
#pragma unroll
        for (int dt = 0; dt < DH; ++dt) {
          bo[dt] = col_operand_c<RS>(dOs, r0, (role * DH + dt) * 32, lane);
          bq[dt] = col_operand_c<RS>(Qs, r0, (role * DH + dt) * 32, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < DH; ++dt) {
          dv[dt] = mfma32(ap, bo[dt], dv[dt]);
          dk[dt] = mfma32(as, bq[dt], dk[dt]);
        }
      }
    };
    // One straight-line body per case: this wave's tile, then the swap.
    u32x4 pa[2], da[2];  // this wave's tile, [16-row step]
    auto tiles = [&](auto masked) __attribute__((always_inline)) {
      f32x16 s, dp;
      sdp(role, s, dp);
      __builtin_amdgcn_sched_barrier(0);
      p_ds(masked, role, s, dp, pa, da);
      u32x4* mine = xch + wave * 64 * 4;
      mine[lane] = pa[0];
      mine[64 + lane] = pa[1];
      mine[128 + lane] = da[0];
      mine[192 + lane] = da[1];
    };
    if (full)
      tiles(std::false_type{});
    else
      tiles(std::true_type{});
    if (role == 0 && item + 1 < n_items) fetch(item + 1);
    // This wave's own tile needs no exchange: its dV/dK products run before
    // the barrier, under the partner's softmax.
    dvdk(role, pa, da);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // the partner's P and dS are in LDS
    {
      // The partner's tile: written by wave kg + 4 (1 - role).
      const int qt = role ^ 1;
      const u32x4* src = xch + (kg + 4 * qt) * 64 * 4;
      u32x4 pb[2], db[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        pb[h2] = src[h2 * 64 + lane];
        db[h2] = src[128 + h2 * 64 + lane];
      }
      dvdk(qt, pb, db);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (role == 0 && item + 1 < n_items) stage(buf ^ 1);
  }

  // dK (times scale) and dV, bf16: lane holds d column (role DH + dt) 32 +
  // l % 32 of key rows kg 32 + (r/4) 8 + 4 hl + r % 4. Stored straight from
  // that layout, each instruction would write 2 bytes per lane; instead each
  // wave stages its 32 keys x DH 32 columns of both in LDS (key-row-major,
  // rows padded by 16 bytes) and stores 16 bytes per lane, whole row halves
  // per instruction.
  constexpr int SC = DH * 32;        // columns per wave
  constexpr int SRS = SC * 2 + 16;   // staged row stride, bytes
  constexpr int SB = 32 * SRS;       // one tensor's staged rows
  static_assert(8 * 2 * SB <= (int)sizeof(lds), "dK/dV staging exceeds LDS");
  __syncthreads();  // no wave reads the tiles or the exchange area any more
  char* st = reinterpret_cast<char*>(lds) + wave * 2 * SB;
#pragma unroll
  for (int dt = 0; dt < DH; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = ((r >> 2) * 8 + hl * 4 + (r & 3)) * SRS + (dt * 32 + (lane & 31)) * 2;
      *reinterpret_cast<uint16_t*>(st + off) = __builtin_bit_cast(uint16_t, (__bf16)(dk[dt][r] * scale));
      *reinterpret_cast<uint16_t*>(st + SB + off) = __builtin_bit_cast(uint16_t, (__bf16)dv[dt][r]);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int LPR = SC * 2 / 16;  // lanes per staged row
  constexpr int RPS = 64 / LPR;     // rows per store instruction
  const size_t row0 = (size_t)(b * Hkv + g) * Nk + k0 + kg * 32;
#pragma unroll
  for (int j = 0; j < 32 / RPS; ++j) {
    const int r = j * RPS + lane / LPR;
    const int c = (lane % LPR) * 16;
    const u32x4 vk = *reinterpret_cast<const u32x4*>(st + r * SRS + c);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(st + SB + r * SRS + c);
    if (kg * 32 + r < nk) {
      const size_t off = (row0 + r) * D * 2 + role * SC * 2 + c;
      __builtin_nontemporal_store(vk, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dK) + off));
      __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dV) + off));
    }
  }
}

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int Nq, int Nk, float scale, float sl2, int causal, int n_qb) {
  using L = BwdLayout<D>;
  constexpr int RS = L::RS, KS = L::KS, DH = L::DT / 2;
  // Two K buffers and one V buffer of kDqBK rows, then per wave two tiles of
  // 64 lanes x 32 bytes of dS^T operands for its partner.
  constexpr int TB = kDqBK * RS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * TB + 8 * 256 * 8];
  u32x4* xch = reinterpret_cast<u32x4*>(lds + 3 * TB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;

  // Row blocks in reverse order (under the causal mask the last rows see the
  // most keys, so the longest workgroups start first), (batch, head) fastest:
  // with B * Hq a multiple of 8 all row blocks of a head land on one XCD.
  const int n_bh = gridDim.x / n_qb;
  const int qr = blockIdx.x / n_bh;
  const int bh = blockIdx.x - qr * n_bh;
  const int qb = n_qb - 1 - qr;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const int q0 = qb * kDqRows;
  const int diag = Nk - Nq;

  // Waves w and w + 4 (one SIMD) share 32 rows: of each 128-key block, wave
  // w + 4 r computes S^T, dP^T and dS^T for the two 32-key tiles of keys
  // 64 r..64 r + 63; the pair swaps the bf16 dS^T operands through LDS, and
  // each wave accumulates dQ^T over all 128 keys for one half of d (so that
  // two waves share a SIMD).
  // This lane's query row, its Q and dO as the B operands of S^T = K Q^T and
  // dP^T = V dO^T (d = 16 ks + 8 (l/32) + 0..7), its LSE and D.
  const int rg = wave & 3, role = wave >> 2;
  const int qw = q0 + rg * 32 + (lane & 31);
  const bool qin = qw < Nq;
  const size_t qoff = ((size_t)bh * Nq + (qin ? qw : 0)) * D;
  bf16x8 qop[KS], dop[KS];
  float l2 = __builtin_huge_valf(), drow = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = dop[ks] = bf16x8{};
    if (qin) {
      qop[ks] = *reinterpret_cast<const bf16x8*>(Q + qoff + ks * 16 + hl * 8);
      dop[ks] = *reinterpret_cast<const bf16x8*>(dO + qoff + ks * 16 + hl * 8);
    }
  }
  if (qin) {
    // A row without keys (LSE = -inf) gets P = 0: exp2(-inf).
    const float l = LSE[(size_t)bh * Nq + qw];
    l2 = l > kNegInf ? l * kLog2e : __builtin_huge_valf();
    drow = Dsum[(size_t)bh * Nq + qw];
  }
  wait_vm_loads();

  f32x16 dq[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) dq[i] = f32x16{};

  // Keys the block's last row sees: under the causal mask row i sees key j
  // iff j <= i + diag.
  int kend = Nk;
  if (causal) {
    const long last = (long)(q0 + kDqRows < Nq ? q0 + kDqRows : Nq) - 1 + diag + 1;
    kend = last < 0 ? 0 : (last < Nk ? (int)last : Nk);
  }
  const int n_kb = (kend + kDqBK - 1) / kDqBK;
  const uint16_t* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const uint16_t* Vh = V + (size_t)(b * Hkv + g) * Nk * D;
  // K double-buffered and V single-buffered in LDS: after the swap barrier of
  // block j every wave is done with V(j) and with K(j - 1), so block j + 1
  // goes in then, from registers loaded one block earlier.
  RowsInFlight<D> kn[2], vn[2];
  auto load_block = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int first = j * kDqBK + h * 64;
      const int rows = Nk - first < 64 ? Nk - first : 64;
      kn[h].load(Kh + (size_t)first * D, rows, tid);
      vn[h].load(Vh + (size_t)first * D, rows, tid);
    }
  };
  auto store_block = [&](int kb_buf) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kn[h].store(lds + kb_buf * TB + h * 64 * RS, tid);
      vn[h].store(lds + 2 * TB + h * 64 * RS, tid);
    }
  };
  if (n_kb > 0) {
    load_block(0);
    store_block(0);
    if (n_kb > 1) load_block(1);
  }

  for (int j = 0; j < n_kb; ++j) {
    const int k0 = j * kDqBK;
    const int buf = j & 1;
    const uint16_t* Ks = lds + buf * TB;
    const uint16_t* Vs = lds + 2 * TB;
    // Block j's K and V are in LDS, and the previous block's dS^T swap has
    // been read.
    __syncthreads();

    // Masks only at a ragged key block or where the causal diagonal crosses
    // the block for the workgroup's first row.
    const bool full = k0 + kDqBK <= Nk && (!causal || k0 + kDqBK - 1 <= q0 + diag);
    // S^T and dP^T of a 32-key tile: 32 keys x this wave's 32 rows.
    // The V rows are read while the S^T MFMAs run.
    auto sdp = [&](int kt, f32x16& st, f32x16& dpt) __attribute__((always_inline)) {
      bf16x8 opa[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) opa[ks] = row_operand<RS>(Ks, kt * 32, ks * 16, lane);
      __builtin_amdgcn_sched_barrier(0);
      st = dpt = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st = mfma32(opa[ks], qop[ks], st);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) opa[ks] = row_operand<RS>(Vs, kt * 32, ks * 16, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dpt = mfma32(opa[ks], dop[ks], dpt);
    };
    // dS^T. C layout: lane l holds row qw, keys k0 + kt*32 + 8 (i/4) + 4 hl + i%4;
    // elements 8 h2 + 0..7 are the B operand (k = those keys) of one 16-key
    // step of dQ^T += K^T dS^T.
    auto ds_t = [&](auto masked, int kt, const f32x16& st, const f32x16& dpt, u32x4* bs) __attribute__((always_inline)) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float dsv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = i4 * 4 + jj;
          float x = __builtin_fmaf(st[i], sl2, -l2);
          if (decltype(masked)::value) {
            const int key = k0 + kt * 32 + i4 * 8 + hl * 4 + jj;
            const bool vis = key < Nk && (!causal || key <= qw + diag);
            x = vis ? x : kNegInf;
          }
          dsv[jj] = fast_exp2(x) * (dpt[i] - drow);
        }
        bs[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(dsv[0], dsv[1]);
        bs[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
    };
    // dQ^T += K^T dS^T for one 32-key tile: A operand K read across key rows
    // in the order of the B operand's elements.
    auto dq_mm = [&](int kt, const u32x4* bs) __attribute__((always_inline)) {
      bf16x8 ka[2][DH];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < DH; ++dt)
          ka[h2][dt] = col_operand_c<RS>(Ks, kt * 32 + h2 * 16, (role * DH + dt) * 32, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 bsv = __builtin_bit_cast(bf16x8, bs[h2]);
#pragma unroll
        for (int dt = 0; dt < DH; ++dt) dq[dt] = mfma32(ka[h2][dt], bsv, dq[dt]);
      }
    };
    // One straight-line body per case: this wave's two key tiles (keys
    // 64 role .. 64 role + 63 of the block), then the swap.
    auto tiles = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 st, dpt;
        u32x4 bs[2];
        sdp(2 * role + tt, st, dpt);
        __builtin_amdgcn_sched_barrier(0);
        ds_t(masked, 2 * role + tt, st, dpt, bs);
        u32x4* mine = xch + wave * 256 + tt * 128;
        mine[lane] = bs[0];
        mine[64 + lane] = bs[1];
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (full)
      tiles(std::false_type{});
    else
      tiles(std::true_type{});
    __syncthreads();  // all four key tiles' dS^T of every row group are in LDS
    if (j + 1 < n_kb) {
      store_block(buf ^ 1);
      if (j + 2 < n_kb) load_block(j + 2);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      // Key tile kt's dS^T: written by wave rg + 4 (kt / 2), its tile kt % 2.
      const u32x4* src = xch + (rg + 4 * (kt >> 1)) * 256 + (kt & 1) * 128;
      u32x4 bs[2];
      bs[0] = src[lane];
      bs[1] = src[64 + lane];
      dq_mm(kt, bs);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // dQ (times scale), bf16. C layout of dQ^T: lane l holds row qw, d columns
  // (role DH + dt)*32 + 8 a + 4 hl + 0..3 (a = 0..3) in elements 4 a + 0..3.
  // Staged per wave in LDS (row-major, rows padded by 16 bytes) and stored 16
  // bytes per lane, whole row halves per instruction, instead of 8 bytes into
  // each of 32 rows.
  constexpr int SC = DH * 32;       // columns per wave
  constexpr int SRS = SC * 2 + 16;  // staged row stride, bytes
  static_assert(8 * 32 * SRS <= (int)sizeof(lds), "dQ staging exceeds LDS");
  __syncthreads();  // no wave reads the K/V tiles or the exchange area any more
  char* st = reinterpret_cast<char*>(lds) + wave * 32 * SRS;
#pragma unroll
  for (int dt = 0; dt < DH; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x2 w = u32x2{pack_bf16x2(dq[dt][4 * a] * scale, dq[dt][4 * a + 1] * scale),
                            pack_bf16x2(dq[dt][4 * a + 2] * scale, dq[dt][4 * a + 3] * scale)};
      *reinterpret_cast<u32x2*>(st + (lane & 31) * SRS + (dt * 32 + a * 8 + hl * 4) * 2) = w;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int LPR = SC * 2 / 16;  // lanes per staged row
  constexpr int RPS = 64 / LPR;     // rows per store instruction
  const int qrow0 = q0 + rg * 32;
#pragma unroll
  for (int j = 0; j < 32 / RPS; ++j) {
    const int r = j * RPS + lane / LPR;
    const int c = (lane % LPR) * 16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * SRS + c);
    if (qrow0 + r < Nq)
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dQ) + ((size_t)bh * Nq + qrow0 + r) * D * 2 +
                                      role * SC * 2 + c));
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  const long rows = (long)a.f.B * a.f.Hq * a.f.Nq;
  hipStream_t st = (hipStream_t)a.f.stream;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dsum, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float sl2 = a.f.scale * kLog2e;
  const int n_kb = (a.f.Nk + kBwdBK - 1) / kBwdBK;
  const long n_wg = (long)a.f.B * a.f.Hkv * n_kb;
  if (n_wg > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)n_wg), dim3(kBwdThreads), 0, st, (const uint16_t*)a.f.q,
                       (const uint16_t*)a.f.k, (const uint16_t*)a.f.v, (const uint16_t*)a.dout, a.f.lse, a.dsum,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, a.f.Hq, a.f.Hkv, a.f.Nq, a.f.Nk, a.f.scale, sl2,
                       a.f.causal, n_kb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qb = (a.f.Nq + kDqRows - 1) / kDqRows;
  const long n_wq = (long)a.f.B * a.f.Hq * n_qb;
  if (n_wq > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)n_wq), dim3(kBwdThreads), 0, st, (const uint16_t*)a.f.q,
                       (const uint16_t*)a.f.k, (const uint16_t*)a.f.v, (const uint16_t*)a.dout, a.f.lse, a.dsum,
                       (uint16_t*)a.dq, a.f.Hq, a.f.Hkv, a.f.Nq, a.f.Nk, a.f.scale, sl2, a.f.causal, n_qb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) { return a.f.d == 128 ? launch_bwd_d<128>(a) : launch_bwd_d<64>(a); }

long bwd_grid(int B, int Hkv, int Nk) { return (long)B * Hkv * ((Nk + kBwdBK - 1) / kBwdBK); }

}  // namespace fa
