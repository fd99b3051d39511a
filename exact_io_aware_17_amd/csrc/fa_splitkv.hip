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
// Partial kernel, one workgroup per (chunk s, 32-row block, KV head g, batch b):
//  * the rows are the (query head in g's group, query index) pairs, so the
//    Hq/Hkv query heads that share a KV head read each K/V byte once;
//  * 256 threads = 4 waves; tiles of 128 keys are loaded cooperatively and
//    each wave scores and accumulates its own 32 keys of the tile with the
//    same transposed MFMA layout as the prefill kernel, keeping its own
//    running (m, l, O);
//  * the next tile's global loads are in flight during the current tile's math;
//  * at the end the four waves' states are merged through LDS.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kSplitThreads = 256;
constexpr int kSplitBN = 128;
constexpr int kSplitRows = 32;

template <int D>
__global__ __launch_bounds__(kSplitThreads) void splitkv_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ LSEpart, int Hq, int Hkv, int Nq, int Nk,
    float sl2, int causal, int S, int chunk) {
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][kSplitBN * D];
  __shared__ float ms[4][kSplitRows], ls[4][kSplitRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x % S, rb = blockIdx.x / S;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, R = G * Nq;
  const int r = rb * kSplitRows + (lane & 31);
  const bool rvalid = r < R;
  const int hh = rvalid ? r / Nq : 0, qi = rvalid ? r - hh * Nq : 0;
  const int head = g * G + hh;
  const int diag = Nk - Nq;

  bf16x8 qf[KS];
  const uint16_t* qrow = Q + ((size_t)(b * Hq + head) * Nq + qi) * D;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    qf[k] = rvalid ? *reinterpret_cast<const bf16x8*>(qrow + k * 16 + (lane >> 5) * 8) : bf16x8{};
  }

  const long k0l = (long)s * chunk;
  const int k0 = k0l < Nk ? (int)k0l : Nk;
  const int k1 = (long)k0 + chunk < (long)Nk ? k0 + chunk : Nk;
  const int n_tiles = (k1 - k0 + kSplitBN - 1) / kSplitBN;
  const int lim = causal ? qi + diag : 0x7fffffff;

  const uint16_t* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const uint16_t* Vh = V + (size_t)(b * Hkv + g) * Nk * D;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  TileCopy<D, kSplitBN, kSplitThreads> kc, vc;
  if (n_tiles > 0) {
    kc.load(Kh + (size_t)k0 * D, k1 - k0, tid);
    vc.load(Vh + (size_t)k0 * D, k1 - k0, tid);
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = k0 + t * kSplitBN;
    __syncthreads();
    kc.store(smem[0], tid);
    vc.store(smem[1], tid);
    __syncthreads();
    if (t + 1 < n_tiles) {
      kc.load(Kh + (size_t)(kv0 + kSplitBN) * D, k1 - kv0 - kSplitBN, tid);
      vc.load(Vh + (size_t)(kv0 + kSplitBN) * D, k1 - kv0 - kSplitBN, tid);
    }
    const int r0 = wave * 32;
    if (kv0 + r0 < k1) {
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k) sacc = mfma32(load_k_operand<D>(smem[0], r0, k, lane), qf[k], sacc);
      if (kv0 + r0 + 32 > k1 || causal) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + score_key(r0, i, lane);
          if (key >= k1 || key > lim) sacc[i] = kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
      bf16x8 p[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(sacc[i], sl2, -m_use));
        rs += e;
        p[i >> 3][i & 7] = (__bf16)e;
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = mfma32(load_vt_operand<D>(smem[1], r0 + hf * 16, db, lane), p[hf], o[db]);
    }
  }

  // Merge the four waves' (m, l, O~) through LDS.
  __syncthreads();
  float* os = reinterpret_cast<float*>(&smem[0][0]);  // [4][32][D] fp32, fits in the tile buffers
  const float l_tot = l_run + wave_xor32(l_run);
  if (lane < 32) {
    ms[wave][lane] = m_run;
    ls[wave][lane] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = db * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      os[(wave * kSplitRows + (lane & 31)) * D + d] = o[db][i];
    }
  __syncthreads();
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
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = fast_exp2(ms[w][row] - M);
        den += ls[w][row] * sc;
        num += os[(w * kSplitRows + row) * D + d] * sc;
      }
      val = num / den;
      lse = (M + fast_log2(den)) * kLn2;
    }
    const size_t pr = ((size_t)(b * Hq + h2) * S + s) * Nq + q2;
    Opart[pr * D + d] = val;
    if (d == 0) LSEpart[pr] = lse;
  }
}

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
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[(size_t)s * Nq]);
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  float den = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float w = expf(lp[(size_t)s * Nq] - M);
      den += w;
#pragma unroll
      for (int p = 0; p < PER; ++p) acc[p] = __builtin_fmaf(w, op[(size_t)s * Nq * D + p], acc[p]);
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
  hipLaunchKernelGGL(splitkv_partial_kernel<D>, dim3((unsigned)(S * nrb), (unsigned)f.Hkv, (unsigned)f.B),
                     dim3(kSplitThreads), 0, (hipStream_t)f.stream, (const uint16_t*)f.q, (const uint16_t*)f.k,
                     (const uint16_t*)f.v, a.o_part, a.lse_part, f.Hq, f.Hkv, f.Nq, f.Nk, sl2, f.causal, S,
                     chunk);
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
