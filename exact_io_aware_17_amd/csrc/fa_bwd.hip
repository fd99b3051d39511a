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
//    block). K and V of the block stay in LDS; the workgroup walks the query
//    heads of its GQA group and their 64-row query blocks (under the causal
//    mask only the blocks that see a key of the block). Per query block:
//      - Q, dO, LSE, D rows into LDS;
//      - S and dP (64 x 128) with 32x32x16 bf16 MFMAs, a 32-row x 64-key
//        block per wave; P = exp2(S scale log2e - LSE log2e), dS = P (dP - D)
//        in fp32, masked entries 0; P^T and dS^T go to LDS in bf16;
//      - dV += P^T dO and dK += dS^T Q (128 keys x d) accumulate in
//        registers, a 64-key x (d/2) block per wave;
//      - dQ (64 rows x d) = dS K over the 128 keys: each wave's 32-row x
//        (d/2) block is added to the fp32 accumulator with vector atomics
//        (query blocks are shared by every key block; 128 keys per workgroup
//        halve these adds, and the per-key cost of each query block, against
//        64).
//    The next query block's Q, dO, LSE and D are loaded into registers while
//    the current one is computed.
//    Column-wise operands (dO, Q, K and dS read across rows) come from the
//    transposing LDS read ds_read_b64_tr_b16 (lane semantics in fa_common.h);
//    rows are padded by 16 bytes so that row-wise 16-byte reads of 16
//    consecutive rows touch distinct banks.
//  * bwd_dq_kernel: dQ accumulator -> bf16.
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
  static constexpr int RS = D + 8;  // row stride of K, V, Q, dO tiles (elements)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + kBwdBK * RS;
  static constexpr int Q_OFF = V_OFF + kBwdBK * RS;
  static constexpr int DO_OFF = Q_OFF + kBwdBQ * RS;
  static constexpr int PT_OFF = DO_OFF + kBwdBQ * RS;
  static constexpr int DST_OFF = PT_OFF + kBwdBK * kPStride;
  static constexpr int ELEMS = DST_OFF + kBwdBK * kPStride;  // bf16 elements; then 2 x 64 floats
  static constexpr int DB = D / 64;  // 32-wide d blocks per wave (each wave owns half of d)
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
  constexpr int RS = L::RS;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t lds[L::ELEMS + 2 * 64 * 2];
  uint16_t* Ks = lds + L::K_OFF;
  uint16_t* Vs = lds + L::V_OFF;
  uint16_t* Qs = lds + L::Q_OFF;
  uint16_t* dOs = lds + L::DO_OFF;
  uint16_t* PT = lds + L::PT_OFF;
  uint16_t* dST = lds + L::DST_OFF;
  float* lse2 = reinterpret_cast<float*>(lds + L::ELEMS);
  float* dsum = lse2 + 64;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int half = wave & 1, dh = wave >> 1;  // quadrant / block owned by this wave

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

  load_rows<D, kBwdBK>(Ks, Kh, nk, tid);
  load_rows<D, kBwdBK>(Vs, Vh, nk, tid);

  f32x16 dv[kBwdKH][L::DB], dk[kBwdKH][L::DB];
#pragma unroll
  for (int kk = 0; kk < kBwdKH; ++kk)
#pragma unroll
    for (int i = 0; i < L::DB; ++i) dv[kk][i] = dk[kk][i] = f32x16{};

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
  if (n_items > 0) fetch(0);

  for (int item = 0; item < n_items; ++item) {
    const int hh = item / per_head, qb = qb0 + item % per_head;
    const int h = g * group + hh;
    const size_t bh = (size_t)b * Hq + h;
    {
      const int q0 = qb * kBwdBQ;
      const int nq = Nq - q0 < kBwdBQ ? Nq - q0 : kBwdBQ;
      __syncthreads();  // the previous block's reads of Qs, dOs, PT, dST are done
      qn.store(Qs, tid);
      don.store(dOs, tid);
      if (tid < 64) {
        // A row without keys (LSE = -inf) or past Nq gets P = 0: exp2(-inf).
        lse2[tid] = lse_n > kNegInf ? lse_n * kLog2e : __builtin_huge_valf();
        dsum[tid] = d_n;
      }
      if (item + 1 < n_items) fetch(item + 1);
      __syncthreads();

      // S and dP: query half wq, keys wk*64 + 32 kk (kk = 0, 1) of this wave.
      const int wq = wave >> 1, wk = wave & 1;
#pragma unroll
      for (int kk = 0; kk < kBwdKH; ++kk) {
      const int kr0 = wk * 64 + kk * 32;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(row_operand<RS>(Qs, wq * 32, ks * 16, lane), row_operand<RS>(Ks, kr0, ks * 16, lane), s);
        dp = mfma32(row_operand<RS>(dOs, wq * 32, ks * 16, lane), row_operand<RS>(Vs, kr0, ks * 16, lane), dp);
      }
      // C layout: lane l holds key kr0 + l%32, query rows wq*32 + (i/4)*8 + 4 hl + i%4.
      const int kl = kr0 + (lane & 31);
      const int key = k0 + kl;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int ql = wq * 32 + i4 * 8 + hl * 4;
        uint32_t pw[2], dw[2];
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          float pv[2], dv2[2];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int i = i4 * 4 + j + jj;
            const int qr = ql + j + jj;
            const bool vis = key < Nk && (!causal || key <= q0 + qr + diag);
            const float p = vis ? fast_exp2(__builtin_fmaf(s[i], sl2, -lse2[qr])) : 0.f;
            pv[jj] = p;
            dv2[jj] = p * (dp[i] - dsum[qr]);
          }
          pw[j >> 1] = pack_bf16x2(pv[0], pv[1]);
          dw[j >> 1] = pack_bf16x2(dv2[0], dv2[1]);
        }
        *reinterpret_cast<u32x2*>(PT + kl * kPStride + ql) = u32x2{pw[0], pw[1]};
        *reinterpret_cast<u32x2*>(dST + kl * kPStride + ql) = u32x2{dw[0], dw[1]};
      }
      }
      __syncthreads();

      // dV += P^T dO and dK += dS^T Q: keys half*64 + 32 kk, d blocks dh*(D/2) + 32 i.
#pragma unroll
      for (int ks = 0; ks < kBwdBQ / 16; ++ks) {
        bf16x8 bo[L::DB], bq[L::DB];
#pragma unroll
        for (int i = 0; i < L::DB; ++i) {
          const int c0 = dh * (D / 2) + i * 32;
          bo[i] = col_operand<RS>(dOs, ks * 16, c0, lane);
          bq[i] = col_operand<RS>(Qs, ks * 16, c0, lane);
        }
#pragma unroll
        for (int kk = 0; kk < kBwdKH; ++kk) {
          const bf16x8 ap = row_operand<kPStride>(PT, half * 64 + kk * 32, ks * 16, lane);
          const bf16x8 as = row_operand<kPStride>(dST, half * 64 + kk * 32, ks * 16, lane);
#pragma unroll
          for (int i = 0; i < L::DB; ++i) {
            dv[kk][i] = mfma32(ap, bo[i], dv[kk][i]);
            dk[kk][i] = mfma32(as, bq[i], dk[kk][i]);
          }
        }
      }
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
#pragma unroll
      for (int i = 0; i < L::DB; ++i) {
        const int d = dh * (D / 2) + i * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = half * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (ql < nq) unsafeAtomicAdd(dq_acc + (bh * Nq + q0 + ql) * D + d, dq[i][r] * scale);
        }
      }
    }
  }

  // dK (times scale) and dV, bf16: lane holds d column, key rows (i/4)*8 + 4 hl + i%4.
#pragma unroll
  for (int kk = 0; kk < kBwdKH; ++kk)
#pragma unroll
  for (int i = 0; i < L::DB; ++i) {
    const int d = dh * (D / 2) + i * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = half * 64 + kk * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
      if (kl < nk) {
        const size_t off = ((size_t)(b * Hkv + g) * Nk + k0 + kl) * D + d;
        dK[off] = __builtin_bit_cast(uint16_t, (__bf16)(dk[kk][i][r] * scale));
        dV[off] = __builtin_bit_cast(uint16_t, (__bf16)dv[kk][i][r]);
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
