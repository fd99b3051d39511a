// bf16 attention forward (prefill) for gfx950.
//
// Algorithm: the FA2 loop of "Flash Attention on the 5090 in CUDA C++"
// ("Flash Attention 2 algorithm" pseudocode): one workgroup owns one block of
// query rows of one (batch, head), zeroes its O tile, walks the KV tiles in
// order, scores each tile, applies the online softmax and accumulates P.V, and
// stores O once. The online softmax is the running-max / running-denominator /
// rescale recurrence of that page's "v1 -- basic version" bullets, kept in the
// unnormalised form with one division at the end.
//
// Mapping to CDNA4 (our design, not the page's sm120 one):
//  * 256 threads = 4 waves; each wave owns 32 query rows, the workgroup 128.
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs:
//    the Q rows of the wave are the B operand and stay in registers for the
//    whole KV loop; every lane then holds 32 scores of ONE query row, so the
//    row max needs one cross-lane step (lane ^ 32) and the rescale factor is a
//    per-lane scalar.
//  * O is accumulated transposed, O^T += V^T P^T: the probabilities are already
//    in B-operand layout (see kappa()), V^T comes from row-major LDS through
//    transposing reads.
//  * K/V tiles of 64 keys are double buffered in XOR-swizzled LDS; the next
//    tile's global loads are in flight while the current tile is computed.
//  * Causal: KV tiles past the workgroup's last visible key are never loaded;
//    waves whose rows see nothing of a tile skip its math; only tiles that
//    cross the diagonal (or the ragged end) are masked element-wise.
//  * Workgroups are renumbered so that consecutive query blocks of one head
//    land on the same XCD (shared L2 for that head's K/V); under the causal
//    mask the longest query blocks are issued first.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdThreads = 256;
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;

template <int D>
__global__ __launch_bounds__(kFwdThreads) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
    float sl2, int causal, int n_qt, int n_wg) {
  constexpr int BN = kFwdBN;
  constexpr int KS = D / 16;  // k-steps of the score MFMA
  constexpr int DB = D / 32;  // d blocks of the output
  constexpr int MB = BN / 32; // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][BN * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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

  const int qw0 = qt * kFwdBM + wave * 32;
  const int qrow = qw0 + (lane & 31);
  const int diag = Nk - Nq;  // key j visible to row i iff j <= i + diag

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < Nq) {
      qf[s] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + s * 16 + (lane >> 5) * 8);
    } else {
      qf[s] = bf16x8{};
    }
  }

  int kv_end = Nk;
  if (causal) {
    const long last = (long)qt * kFwdBM + kFwdBM - 1 + diag;
    kv_end = last < 0 ? 0 : (int)(last + 1 < (long)Nk ? last + 1 : Nk);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  TileCopy<D, BN, kFwdThreads> kc, vc;
  if (n_tiles > 0) {
    kc.load(Kh, Nk, tid);
    vc.load(Vh, Nk, tid);
    kc.store(smem[0][0], tid);
    vc.store(smem[0][1], tid);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * BN;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) {
      kc.load(Kh + (size_t)(kv0 + BN) * D, Nk - kv0 - BN, tid);
      vc.load(Vh + (size_t)(kv0 + BN) * D, Nk - kv0 - BN, tid);
    }
    const uint16_t* ks = smem[t & 1][0];
    const uint16_t* vs = smem[t & 1][1];
    const bool wave_live = !causal || (kv0 <= qw0 + 31 + diag);
    if (wave_live) {
      f32x16 sacc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        sacc[mb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc[mb] = mfma32(load_k_operand<D>(ks, mb * 32, s, lane), qf[s], sacc[mb]);
      }
      const bool need_mask = (kv0 + BN > Nk) || (causal && kv0 + BN - 1 > qw0 + diag);
      if (need_mask) {
        const int lim = causal ? qrow + diag : 0x7fffffff;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + score_key(mb * 32, i, lane);
            if (key >= Nk || key > lim) sacc[mb][i] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][i]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
      bf16x8 p[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(__builtin_fmaf(sacc[mb][i], sl2, -m_use));
          rs += e;
          p[mb][i >> 3][i & 7] = (__bf16)e;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            o[db] = mfma32(load_vt_operand<D>(vs, mb * 32 + hf * 16, db, lane), p[mb][hf], o[db]);
    }
    if (has_next) {
      kc.store(smem[(t + 1) & 1][0], tid);
      vc.store(smem[(t + 1) & 1][1], tid);
    }
    __syncthreads();
  }

  // Epilogue: O = O~ / l, LSE = ln(2) * (m + log2 l); rows without keys: 0, -inf.
  const float l_tot = l_run + wave_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Nq) {
    uint16_t* orow = O + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + i4 * 8 + (lane >> 5) * 4;
        u32x2 w;
        w[0] = pack_bf16x2(o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv);
        w[1] = pack_bf16x2(o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (lane < 32) {
      LSE[(size_t)bh * Nq + qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdArgs& a) {
  const int n_qt = (a.Nq + kFwdBM - 1) / kFwdBM;
  const long n_wg = (long)a.B * a.Hq * n_qt;
  if (n_wg == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3((unsigned)n_wg), dim3(kFwdThreads), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.causal, n_qt, (int)n_wg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  return a.d == 128 ? launch_fwd_bf16_d<128>(a) : launch_fwd_bf16_d<64>(a);
}

long fwd_bf16_grid(int B, int Hq, int Nq) { return (long)B * Hq * ((Nq + kFwdBM - 1) / kFwdBM); }

}  // namespace fa
