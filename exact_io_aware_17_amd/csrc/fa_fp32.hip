// fp32 attention forward: the debug / reference path of the library.
//
// Plain FMA arithmetic, one thread per query row, K/V tiles of 32 keys staged
// in LDS and the online softmax applied key by key (the running max, running
// denominator and rescale of "Flash Attention on the 5090 in CUDA C++",
// "v1 -- basic version"). Exact expf/logf are used so that the result stays
// within about 1e-6 of the exact fp64 value. Speed is not a goal of this path.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(kF32Rows) void fwd_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float scale,
    int causal, int n_qt) {
  __shared__ float qs[kF32Rows][D + 1];
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const int t = threadIdx.x;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const float* Qh = Q + (size_t)bh * Nq * D;
  const float* Kh = K + (size_t)(b * Hkv + g) * Nk * D;
  const float* Vh = V + (size_t)(b * Hkv + g) * Nk * D;
  const int row0 = qt * kF32Rows, row = row0 + t;
  const int diag = Nk - Nq;

  for (int idx = t; idx < kF32Rows * D; idx += kF32Rows) {
    const int r = idx / D, c = idx % D;
    qs[r][c] = (row0 + r < Nq) ? Qh[(size_t)(row0 + r) * D + c] : 0.f;
  }
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = kNegInf, l = 0.f;

  int kv_end = Nk;
  if (causal) {
    const long last = (long)row0 + kF32Rows - 1 + diag;
    kv_end = last < 0 ? 0 : (int)(last + 1 < (long)Nk ? last + 1 : Nk);
  }
  for (int kv0 = 0; kv0 < kv_end; kv0 += kF32Keys) {
    __syncthreads();
    for (int idx = t; idx < kF32Keys * D; idx += kF32Rows) {
      const int r = idx / D, c = idx % D;
      const bool ok = kv0 + r < Nk;
      ks[r][c] = ok ? Kh[(size_t)(kv0 + r) * D + c] : 0.f;
      vs[r][c] = ok ? Vh[(size_t)(kv0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    if (row < Nq) {
      for (int j = 0; j < kF32Keys; ++j) {
        const int key = kv0 + j;
        if (key >= Nk || (causal && key > row + diag)) continue;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s = __builtin_fmaf(qs[t][c], ks[j][c], s);
        s *= scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(o[c], alpha, p * vs[j][c]);
        m = m_new;
      }
    }
  }
  if (row < Nq) {
    float* orow = O + ((size_t)bh * Nq + row) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
    LSE[(size_t)bh * Nq + row] = l > 0.f ? m + logf(l) : kNegInf;
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  const int n_qt = (a.Nq + kF32Rows - 1) / kF32Rows;
  const long n_wg = (long)a.B * a.Hq * n_qt;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3((unsigned)n_wg), dim3(kF32Rows), 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Hq,
                     a.Hkv, a.Nq, a.Nk, a.scale, a.causal, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdArgs& a) { return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a); }

long fwd_fp32_grid(int B, int Hq, int Nq) { return (long)B * Hq * ((Nq + kF32Rows - 1) / kF32Rows); }

}  // namespace fa
